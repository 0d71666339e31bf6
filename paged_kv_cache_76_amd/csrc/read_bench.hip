// Plain device reads with no arithmetic: the achievable HBM rates the
// kernels of this library are measured against (a front-to-back stream, and
// the random-tile pattern of a block-table read).  Not part of the method.
#include "pa_internal.h"

namespace pa {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

#ifndef PA_READ_UNROLL
#define PA_READ_UNROLL 8
#endif
#ifndef PA_READ_WG_PER_CU
#define PA_READ_WG_PER_CU 16  // best of 4, 8, 16 with 4-16 loads in flight (stream and tile reads)
#endif
constexpr int kReadThreads = 256;
constexpr int kReadUnroll = PA_READ_UNROLL;  // 16-byte loads in flight per thread
// the fold is written out only if it equals this (no real data is expected to)
constexpr uint32_t kSinkMagic = 0x9e3779b9u;

__device__ __forceinline__ void sink_fold(u32x4 acc, u32x4* sink) {
  if (acc.x == kSinkMagic && acc.y == ~kSinkMagic && acc.z == kSinkMagic && acc.w == ~kSinkMagic) *sink = acc;
}

// Each workgroup reads contiguous chunks of kReadThreads * kReadUnroll * 16
// bytes (32 KiB), chunk c + k * gridDim.x for k = 0, 1, ...
__global__ __launch_bounds__(kReadThreads) void read_stream_kernel(const u32x4* __restrict__ buf, int64_t nvec,
                                                                  u32x4* __restrict__ sink) {
  constexpr int64_t kChunk = kReadThreads * kReadUnroll;
  u32x4 acc = {0, 0, 0, 0};
  for (int64_t base = (int64_t)blockIdx.x * kChunk; base < nvec; base += (int64_t)gridDim.x * kChunk) {
    u32x4 v[kReadUnroll];
    if (base + kChunk <= nvec) {
#pragma unroll
      for (int u = 0; u < kReadUnroll; ++u) v[u] = __builtin_nontemporal_load(&buf[base + u * kReadThreads + threadIdx.x]);
    } else {
#pragma unroll
      for (int u = 0; u < kReadUnroll; ++u) {
        const int64_t i = base + u * kReadThreads + threadIdx.x;
        v[u] = i < nvec ? __builtin_nontemporal_load(&buf[i]) : u32x4{0, 0, 0, 0};
      }
    }
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) acc ^= v[u];
  }
  sink_fold(acc, sink);
}

// One workgroup reads kReadUnroll tiles at a time (16 bytes per thread per
// tile step); tiles go to workgroups round-robin.
__global__ __launch_bounds__(kReadThreads) void read_tiles_kernel(const u32x4* __restrict__ buf, int64_t tile_vec,
                                                                 int32_t num_tiles, const int32_t* __restrict__ tiles,
                                                                 int32_t n, u32x4* __restrict__ sink) {
  u32x4 acc = {0, 0, 0, 0};
  for (int32_t t0 = blockIdx.x * kReadUnroll; t0 < n; t0 += gridDim.x * kReadUnroll) {
    int32_t id[kReadUnroll];
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) id[u] = t0 + u < n ? tiles[t0 + u] : -1;
    for (int64_t e = threadIdx.x; e < tile_vec; e += kReadThreads) {
      u32x4 v[kReadUnroll];
#pragma unroll
      for (int u = 0; u < kReadUnroll; ++u) {
        const bool ok = id[u] >= 0 && id[u] < num_tiles;
        v[u] = ok ? __builtin_nontemporal_load(&buf[(int64_t)id[u] * tile_vec + e]) : u32x4{0, 0, 0, 0};
      }
#pragma unroll
      for (int u = 0; u < kReadUnroll; ++u) acc ^= v[u];
    }
  }
  sink_fold(acc, sink);
}

int read_grid(int64_t work_items) {
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) == hipSuccess) hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  const int64_t want = (int64_t)cus * PA_READ_WG_PER_CU;  // 256-thread workgroups per CU
  return (int)(work_items < want ? (work_items > 0 ? work_items : 1) : want);
}

}  // namespace

hipError_t launch_read_stream(const void* buf, int64_t bytes, void* sink, hipStream_t stream) {
  const int64_t nvec = bytes / 16;
  const int grid = read_grid((nvec + kReadThreads * kReadUnroll - 1) / (kReadThreads * kReadUnroll));
  hipLaunchKernelGGL(read_stream_kernel, dim3(grid), dim3(kReadThreads), 0, stream, (const u32x4*)buf, nvec,
                     (u32x4*)sink);
  return hipGetLastError();
}

hipError_t launch_read_tiles(const void* buf, int64_t tile_bytes, int32_t num_tiles, const int32_t* tiles,
                             int32_t n, void* sink, hipStream_t stream) {
  const int grid = read_grid(((int64_t)n + kReadUnroll - 1) / kReadUnroll);
  hipLaunchKernelGGL(read_tiles_kernel, dim3(grid), dim3(kReadThreads), 0, stream, (const u32x4*)buf,
                     tile_bytes / 16, num_tiles, tiles, n, (u32x4*)sink);
  return hipGetLastError();
}

}  // namespace pa
