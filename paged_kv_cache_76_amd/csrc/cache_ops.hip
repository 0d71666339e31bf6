// Slot-mapped cache writes and batched whole-block copies.
//
// "vLLM / PagedAttention" (awesome.papernotes.org), key design 5: the new
// keys/values of each layer are reshaped into the block-read layout and
// written to their positions in one fused operation, and the many small block
// copies caused by copy-on-write are batched into one kernel rather than one
// memcpy per block.  Both operations are pure data movement, so the kernels
// move opaque 16-byte vectors and are dtype-agnostic: results are bit-exact by
// construction.
//
// Both kernels are HBM-bound (zero arithmetic).  A 16-byte load per lane makes
// one wave touch 1 KiB of consecutive bytes per instruction.
#include "pa_internal.h"

namespace pa {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// grid.x = token t, grid.y = chunk of 256 16-byte vectors of that token's
// [H][d] row.  The slot is loaded once per workgroup (wave-uniform).
__global__ __launch_bounds__(kWriteThreads) void reshape_and_cache_kernel(
    const u32x4* __restrict__ key, const u32x4* __restrict__ value,
    u32x4* __restrict__ kpool, u32x4* __restrict__ vpool,
    const int64_t* __restrict__ slot_mapping, int32_t num_heads, int32_t vec_per_row,
    int32_t block_size, int64_t num_slots) {
  const int64_t t = blockIdx.x;
  const int64_t slot = slot_mapping[t];
  if (slot < 0 || slot >= num_slots) return;  // skipped token / outside the pool
  const int32_t per_token = num_heads * vec_per_row;
  const int32_t i = blockIdx.y * kWriteThreads + threadIdx.x;
  if (i >= per_token) return;
  const int32_t h = i / vec_per_row;
  const int32_t v = i - h * vec_per_row;
  const int64_t blk = slot / block_size;
  const int64_t off = slot - blk * block_size;
  const int64_t src = t * per_token + i;
  const int64_t dst = ((blk * num_heads + h) * block_size + off) * vec_per_row + v;
  const u32x4 kv = __builtin_nontemporal_load(&key[src]);
  const u32x4 vv = __builtin_nontemporal_load(&value[src]);
  kpool[dst] = kv;
  vpool[dst] = vv;
}

// grid.x = pair index * 2 + pool (0: keys, 1: values), grid.y = chunk of
// kCopyThreads x kCopyUnroll 16-byte vectors (16 KiB) of the block.
__global__ __launch_bounds__(kCopyThreads) void copy_blocks_kernel(
    u32x4* __restrict__ kpool, u32x4* __restrict__ vpool, const int64_t* __restrict__ pairs,
    int64_t vec_per_block, int64_t num_blocks) {
  const int64_t pair = blockIdx.x >> 1;
  u32x4* __restrict__ pool = (blockIdx.x & 1) ? vpool : kpool;
  const int64_t src = pairs[2 * pair];
  const int64_t dst = pairs[2 * pair + 1];
  if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks) return;
  const int64_t base = (int64_t)blockIdx.y * (kCopyThreads * kCopyUnroll) + threadIdx.x;
  u32x4 buf[kCopyUnroll];
#pragma unroll
  for (int u = 0; u < kCopyUnroll; ++u) {
    const int64_t e = base + u * kCopyThreads;
    if (e < vec_per_block) buf[u] = pool[src * vec_per_block + e];
  }
#pragma unroll
  for (int u = 0; u < kCopyUnroll; ++u) {
    const int64_t e = base + u * kCopyThreads;
    if (e < vec_per_block) pool[dst * vec_per_block + e] = buf[u];
  }
}

// Whole-block copies between two pools of the same block shape (device and
// pinned host memory for swapping).  grid.x = pair * 2 + pool, grid.y = chunk.
__global__ __launch_bounds__(kCopyThreads) void swap_blocks_kernel(
    const u32x4* __restrict__ src_k, const u32x4* __restrict__ src_v, u32x4* __restrict__ dst_k,
    u32x4* __restrict__ dst_v, const int64_t* __restrict__ pairs, int64_t vec_per_block, int64_t src_blocks,
    int64_t dst_blocks) {
  const int64_t pair = blockIdx.x >> 1;
  const u32x4* __restrict__ src = (blockIdx.x & 1) ? src_v : src_k;
  u32x4* __restrict__ dst = (blockIdx.x & 1) ? dst_v : dst_k;
  const int64_t s = pairs[2 * pair];
  const int64_t d = pairs[2 * pair + 1];
  if (s < 0 || s >= src_blocks || d < 0 || d >= dst_blocks) return;
  const int64_t base = (int64_t)blockIdx.y * (kCopyThreads * kCopyUnroll) + threadIdx.x;
  u32x4 buf[kCopyUnroll];
#pragma unroll
  for (int u = 0; u < kCopyUnroll; ++u) {
    const int64_t e = base + u * kCopyThreads;
    if (e < vec_per_block) buf[u] = __builtin_nontemporal_load(&src[s * vec_per_block + e]);
  }
#pragma unroll
  for (int u = 0; u < kCopyUnroll; ++u) {
    const int64_t e = base + u * kCopyThreads;
    if (e < vec_per_block) dst[d * vec_per_block + e] = buf[u];
  }
}

// Staging of a swap through the copy engines: gather = the device blocks of
// pairs i0 .. i0 + count - 1 into consecutive staging slots (swap-out),
// scatter = consecutive staging slots into their device blocks (swap-in).
// A pair with an id outside its pool moves nothing.  grid.x = item * 2 +
// pool, grid.y = chunk of the block, as copy_blocks_kernel.
__global__ __launch_bounds__(kCopyThreads) void stage_blocks_kernel(
    u32x4* __restrict__ kpool, u32x4* __restrict__ vpool, u32x4* __restrict__ stage_k, u32x4* __restrict__ stage_v,
    const int64_t* __restrict__ pairs, int64_t i0, int64_t vec_per_block, int64_t src_blocks, int64_t dst_blocks,
    int32_t gather) {
  const int64_t j = blockIdx.x >> 1;
  u32x4* __restrict__ pool = (blockIdx.x & 1) ? vpool : kpool;
  u32x4* __restrict__ stage = (blockIdx.x & 1) ? stage_v : stage_k;
  const int64_t s = pairs[2 * (i0 + j)];
  const int64_t d = pairs[2 * (i0 + j) + 1];
  if (s < 0 || s >= src_blocks || d < 0 || d >= dst_blocks) return;
  const int64_t blk = gather ? s : d;  // the device block
  const u32x4* __restrict__ from = gather ? pool + blk * vec_per_block : stage + j * vec_per_block;
  u32x4* __restrict__ to = gather ? stage + j * vec_per_block : pool + blk * vec_per_block;
  const int64_t base = (int64_t)blockIdx.y * (kCopyThreads * kCopyUnroll) + threadIdx.x;
  u32x4 buf[kCopyUnroll];
#pragma unroll
  for (int u = 0; u < kCopyUnroll; ++u) {
    const int64_t e = base + u * kCopyThreads;
    if (e < vec_per_block) buf[u] = __builtin_nontemporal_load(&from[e]);
  }
#pragma unroll
  for (int u = 0; u < kCopyUnroll; ++u) {
    const int64_t e = base + u * kCopyThreads;
    if (e < vec_per_block) to[e] = buf[u];
  }
}

}  // namespace

hipError_t launch_stage_blocks(const Cache& c, void* stage_k, void* stage_v, const int64_t* pairs, int64_t i0,
                               int32_t count, int64_t src_blocks, int64_t dst_blocks, bool gather,
                               hipStream_t stream) {
  const int64_t block_bytes =
      (int64_t)c.num_heads * c.block_size * c.head_dim * dtype_bytes(c.dtype);
  dim3 grid((unsigned)(2 * count), (unsigned)copy_grid_y(c));
  hipLaunchKernelGGL(stage_blocks_kernel, grid, dim3(kCopyThreads), 0, stream, (u32x4*)c.k, (u32x4*)c.v,
                     (u32x4*)stage_k, (u32x4*)stage_v, pairs, i0, block_bytes / 16, src_blocks, dst_blocks,
                     gather ? 1 : 0);
  return hipGetLastError();
}

hipError_t launch_swap_blocks(const Cache& c, void* host_k, void* host_v, int32_t host_blocks,
                              const int64_t* pairs, int32_t n, bool to_host, hipStream_t stream) {
  const int64_t block_bytes =
      (int64_t)c.num_heads * c.block_size * c.head_dim * dtype_bytes(c.dtype);
  const int64_t vec_per_block = block_bytes / 16;
  dim3 grid((unsigned)(2 * n), (unsigned)copy_grid_y(c));
  const u32x4* src_k = (const u32x4*)(to_host ? c.k : host_k);
  const u32x4* src_v = (const u32x4*)(to_host ? c.v : host_v);
  u32x4* dst_k = (u32x4*)(to_host ? host_k : c.k);
  u32x4* dst_v = (u32x4*)(to_host ? host_v : c.v);
  const int64_t src_blocks = to_host ? c.num_blocks : host_blocks;
  const int64_t dst_blocks = to_host ? host_blocks : c.num_blocks;
  hipLaunchKernelGGL(swap_blocks_kernel, grid, dim3(kCopyThreads), 0, stream, src_k, src_v, dst_k, dst_v, pairs,
                     vec_per_block, src_blocks, dst_blocks);
  return hipGetLastError();
}

hipError_t launch_reshape_and_cache(const Cache& c, const void* key, const void* value,
                                    const int64_t* slot_mapping, int32_t T, hipStream_t stream) {
  const int32_t row_bytes = c.head_dim * dtype_bytes(c.dtype);
  const int32_t vec_per_row = row_bytes / 16;
  const int32_t per_token = c.num_heads * vec_per_row;
  dim3 grid((unsigned)T, (unsigned)((per_token + kWriteThreads - 1) / kWriteThreads));
  hipLaunchKernelGGL(reshape_and_cache_kernel, grid, dim3(kWriteThreads), 0, stream,
                     (const u32x4*)key, (const u32x4*)value, (u32x4*)c.k, (u32x4*)c.v,
                     slot_mapping, c.num_heads, vec_per_row, c.block_size,
                     (int64_t)c.num_blocks * c.block_size);
  return hipGetLastError();
}

hipError_t launch_copy_blocks(const Cache& c, const int64_t* pairs, int32_t n, hipStream_t stream) {
  const int64_t block_bytes =
      (int64_t)c.num_heads * c.block_size * c.head_dim * dtype_bytes(c.dtype);
  const int64_t vec_per_block = block_bytes / 16;
  dim3 grid((unsigned)(2 * n), (unsigned)copy_grid_y(c));
  hipLaunchKernelGGL(copy_blocks_kernel, grid, dim3(kCopyThreads), 0, stream, (u32x4*)c.k,
                     (u32x4*)c.v, pairs, vec_per_block, (int64_t)c.num_blocks);
  return hipGetLastError();
}

}  // namespace pa
