// C-ABI of libpagedattn: argument validation, dispatch and error reporting.
// Every check below runs on the host before any HIP call, so a rejected call
// touches neither the device nor the stream.
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>

#include <stdlib.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <string>
#include <vector>

#include "pa_internal.h"

namespace {

thread_local std::string g_last_error;

// index-precondition checks before every launch (PA_DEBUG=1 in the
// environment when the library loads, or pa_set_debug)
std::atomic<int> g_debug{[] {
  const char* e = getenv("PA_DEBUG");
  return (e && *e && *e != '0') ? 1 : 0;
}()};

pa_status vfail(pa_status st, const char* fmt, va_list ap) {
  char buf[512];
  vsnprintf(buf, sizeof buf, fmt, ap);
  g_last_error = buf;
  return st;
}

pa_status fail(pa_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vfail(st, fmt, ap);
  va_end(ap);
  return st;
}

// Debug mode: a synchronous copy of a device index array to the host.
template <typename T>
pa_status fetch(const char* fn, const T* dev, int64_t count, hipStream_t stream, std::vector<T>* host) {
  host->assign((size_t)count, T{});
  if (count == 0) return PA_OK;
  if (hipMemcpyAsync(host->data(), dev, (size_t)count * sizeof(T), hipMemcpyDeviceToHost, stream) != hipSuccess ||
      hipStreamSynchronize(stream) != hipSuccess) {
    (void)hipGetLastError();
    return fail(PA_ERR_INVALID_ARG, "%s: the debug check could not read an index array", fn);
  }
  return PA_OK;
}

// Debug mode: the table/length preconditions of the attention calls.
pa_status debug_tables(const char* fn, const pa::Cache& c, const int32_t* tables, int32_t max_blocks,
                       const int32_t* lens, int32_t S, int32_t max_context_len, hipStream_t stream) {
  std::vector<int32_t> t, l;
  pa_status st = fetch(fn, tables, (int64_t)S * max_blocks, stream, &t);
  if (st == PA_OK) st = fetch(fn, lens, S, stream, &l);
  if (st == PA_OK)
    st = pa_check_block_tables(t.data(), S, max_blocks, l.data(), max_context_len, c.block_size, c.num_blocks);
  return st;
}

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }
bool valid_dtype(int t) { return t == PA_F32 || t == PA_F16 || t == PA_BF16; }
bool pow2(int32_t x) { return x > 0 && (x & (x - 1)) == 0; }

pa_status check_cache(const char* fn, const pa_kv_cache* c, pa::Cache* out) {
  if (!c) return fail(PA_ERR_INVALID_ARG, "%s: cache is NULL", fn);
  if (!valid_dtype((int)c->dtype)) return fail(PA_ERR_INVALID_ARG, "%s: bad cache dtype %d", fn, (int)c->dtype);
  if (!c->k || !c->v) return fail(PA_ERR_INVALID_ARG, "%s: cache pool pointer is NULL", fn);
  if (!aligned(c->k, 16) || !aligned(c->v, 16))
    return fail(PA_ERR_INVALID_ARG, "%s: cache pools must be 16-byte aligned", fn);
  if (c->num_blocks < 1 || c->num_heads < 1 || c->head_dim < 1 || c->block_size < 1)
    return fail(PA_ERR_INVALID_ARG, "%s: cache sizes must be >= 1 (blocks %d heads %d dim %d block %d)", fn,
                c->num_blocks, c->num_heads, c->head_dim, c->block_size);
  if (!pow2(c->block_size))
    return fail(PA_ERR_INVALID_ARG, "%s: block_size %d is not a power of two", fn, c->block_size);
  const int64_t row_bytes = (int64_t)c->head_dim * pa::dtype_bytes(c->dtype);
  if (row_bytes % 16 != 0)
    return fail(PA_ERR_UNSUPPORTED, "%s: head_dim*sizeof(dtype) = %lld is not a multiple of 16 bytes", fn,
                (long long)row_bytes);
  out->k = c->k;
  out->v = c->v;
  out->num_blocks = c->num_blocks;
  out->num_heads = c->num_heads;
  out->head_dim = c->head_dim;
  out->block_size = c->block_size;
  out->dtype = c->dtype;
  return PA_OK;
}

// Copies and swaps launch 2n x ceil(block vectors / per-workgroup vectors)
// workgroups; each dimension's work-items must fit 32 bits.
pa_status check_copy_grid(const char* fn, const pa::Cache& c, int32_t n) {
  const int64_t x_items = 2 * (int64_t)n * pa::kCopyThreads;
  const int64_t y_groups = pa::copy_grid_y(c);
  if (x_items > (int64_t)UINT32_MAX || y_groups * pa::kCopyThreads > (int64_t)UINT32_MAX)
    return fail(PA_ERR_INVALID_ARG, "%s: %d pairs (x %lld chunks per block) exceed the launch limit", fn, n,
                (long long)y_groups);
  return PA_OK;
}

pa_status launched(const char* fn, hipError_t err) {
  if (err != hipSuccess) return fail(PA_ERR_LAUNCH, "%s: launch failed: %s", fn, hipGetErrorString(err));
  return PA_OK;
}

}  // namespace

namespace pa {
pa_status check_fail(pa_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vfail(st, fmt, ap);
  va_end(ap);
  return st;
}
}  // namespace pa

extern "C" {

void pa_set_debug(int32_t on) { g_debug.store(on ? 1 : 0); }

int32_t pa_get_debug(void) { return g_debug.load(); }

pa_status pa_reshape_and_cache(const pa_kv_cache* cache, const void* key, const void* value,
                               const int64_t* slot_mapping, int32_t T, void* stream) {
  const char* fn = "pa_reshape_and_cache";
  pa::Cache c;
  pa_status st = check_cache(fn, cache, &c);
  if (st != PA_OK) return st;
  if (T < 0) return fail(PA_ERR_INVALID_ARG, "%s: T = %d < 0", fn, T);
  if (T == 0) return PA_OK;
  if (!key || !value || !slot_mapping) return fail(PA_ERR_INVALID_ARG, "%s: NULL key/value/slot_mapping", fn);
  if (!aligned(key, 16) || !aligned(value, 16))
    return fail(PA_ERR_INVALID_ARG, "%s: key/value must be 16-byte aligned", fn);
  if (!aligned(slot_mapping, 8)) return fail(PA_ERR_INVALID_ARG, "%s: slot_mapping must be 8-byte aligned", fn);
  if ((int64_t)T * pa::kWriteThreads > (int64_t)UINT32_MAX)
    return fail(PA_ERR_INVALID_ARG, "%s: T = %d tokens exceed the launch limit", fn, T);
  if (g_debug.load()) {
    std::vector<int64_t> slots;
    st = fetch(fn, slot_mapping, T, (hipStream_t)stream, &slots);
    if (st == PA_OK) st = pa_check_slot_mapping(slots.data(), T, (int64_t)c.num_blocks * c.block_size);
    if (st != PA_OK) return st;
  }
  return launched(fn, pa::launch_reshape_and_cache(c, key, value, slot_mapping, T, (hipStream_t)stream));
}

pa_status pa_copy_blocks(const pa_kv_cache* cache, const int64_t* pairs, int32_t n, void* stream) {
  const char* fn = "pa_copy_blocks";
  pa::Cache c;
  pa_status st = check_cache(fn, cache, &c);
  if (st != PA_OK) return st;
  if (n < 0) return fail(PA_ERR_INVALID_ARG, "%s: n = %d < 0", fn, n);
  if (n == 0) return PA_OK;
  if (!pairs) return fail(PA_ERR_INVALID_ARG, "%s: pairs is NULL", fn);
  if (!aligned(pairs, 8)) return fail(PA_ERR_INVALID_ARG, "%s: pairs must be 8-byte aligned", fn);
  st = check_copy_grid(fn, c, n);
  if (st != PA_OK) return st;
  if (g_debug.load()) {
    std::vector<int64_t> p;
    st = fetch(fn, pairs, 2 * (int64_t)n, (hipStream_t)stream, &p);
    if (st == PA_OK) st = pa_check_copy_pairs(p.data(), n, c.num_blocks, c.num_blocks, 1);
    if (st != PA_OK) return st;
  }
  return launched(fn, pa::launch_copy_blocks(c, pairs, n, (hipStream_t)stream));
}

pa_status pa_swap_blocks(const pa_kv_cache* cache, void* host_k, void* host_v, int32_t host_num_blocks,
                         const int64_t* pairs, int32_t n, pa_swap_dir dir, void* stream) {
  const char* fn = "pa_swap_blocks";
  pa::Cache c;
  pa_status st = check_cache(fn, cache, &c);
  if (st != PA_OK) return st;
  if (dir != PA_SWAP_OUT && dir != PA_SWAP_IN) return fail(PA_ERR_INVALID_ARG, "%s: bad direction %d", fn, (int)dir);
  if (n < 0 || host_num_blocks < 0) return fail(PA_ERR_INVALID_ARG, "%s: negative size", fn);
  if (n == 0) return PA_OK;
  if (!pairs || !host_k || !host_v) return fail(PA_ERR_INVALID_ARG, "%s: NULL pairs/host pool", fn);
  if (!aligned(pairs, 8) || !aligned(host_k, 16) || !aligned(host_v, 16))
    return fail(PA_ERR_INVALID_ARG, "%s: misaligned pairs/host pool", fn);
  st = check_copy_grid(fn, c, n);
  if (st != PA_OK) return st;
  // the kernel dereferences the host pools: they must be pinned host memory
  // the device can address (a pageable pointer would fault the GPU)
  void* dev_ptr[2] = {nullptr, nullptr};
  void* host_ptr[2] = {host_k, host_v};
  for (int i = 0; i < 2; ++i) {
    hipPointerAttribute_t attr;
    if (hipPointerGetAttributes(&attr, host_ptr[i]) != hipSuccess || attr.type != hipMemoryTypeHost ||
        attr.devicePointer == nullptr) {
      (void)hipGetLastError();  // clear the query's error state
      return fail(PA_ERR_INVALID_ARG, "%s: host pool %d is not pinned, device-accessible host memory", fn, i);
    }
    dev_ptr[i] = attr.devicePointer;
  }
  if (g_debug.load()) {
    std::vector<int64_t> p;
    st = fetch(fn, pairs, 2 * (int64_t)n, (hipStream_t)stream, &p);
    if (st == PA_OK) {
      const bool out = dir == PA_SWAP_OUT;
      st = pa_check_copy_pairs(p.data(), n, out ? c.num_blocks : host_num_blocks, out ? host_num_blocks : c.num_blocks,
                               0);
    }
    if (st != PA_OK) return st;
  }
  return launched(fn, pa::launch_swap_blocks(c, dev_ptr[0], dev_ptr[1], host_num_blocks, pairs, n,
                                             dir == PA_SWAP_OUT, (hipStream_t)stream));
}

size_t pa_swap_staging_bytes(const pa_kv_cache* cache, int32_t blocks) {
  pa::Cache c;
  if (check_cache("pa_swap_staging_bytes", cache, &c) != PA_OK || blocks < 1) return 0;
  return (size_t)2 * blocks * c.num_heads * c.block_size * c.head_dim * pa::dtype_bytes(c.dtype);
}

pa_status pa_swap_blocks_dma(const pa_kv_cache* cache, void* host_k, void* host_v, int32_t host_num_blocks,
                             const int64_t* pairs, const int64_t* pairs_host, int32_t n, pa_swap_dir dir,
                             void* staging, size_t staging_bytes, void* stream) {
  const char* fn = "pa_swap_blocks_dma";
  pa::Cache c;
  pa_status st = check_cache(fn, cache, &c);
  if (st != PA_OK) return st;
  if (dir != PA_SWAP_OUT && dir != PA_SWAP_IN) return fail(PA_ERR_INVALID_ARG, "%s: bad direction %d", fn, (int)dir);
  if (n < 0 || host_num_blocks < 0) return fail(PA_ERR_INVALID_ARG, "%s: negative size", fn);
  if (n == 0) return PA_OK;
  if (!pairs || !pairs_host || !host_k || !host_v || !staging)
    return fail(PA_ERR_INVALID_ARG, "%s: NULL pairs/host pool/staging", fn);
  if (!aligned(pairs, 8) || !aligned(host_k, 16) || !aligned(host_v, 16) || !aligned(staging, 16))
    return fail(PA_ERR_INVALID_ARG, "%s: misaligned pairs/host pool/staging", fn);
  const size_t block_bytes = (size_t)c.num_heads * c.block_size * c.head_dim * pa::dtype_bytes(c.dtype);
  // staging slots: a key block and a value block each
  const int64_t slots = (int64_t)(staging_bytes / (2 * block_bytes));
  if (slots < 1)
    return fail(PA_ERR_WORKSPACE, "%s: staging of %zu bytes holds no block (%zu needed per block)", fn, staging_bytes,
                2 * block_bytes);
  const int32_t chunk = (int32_t)std::min<int64_t>(slots, n);
  st = check_copy_grid(fn, c, chunk);
  if (st != PA_OK) return st;
  // the copy engines read or write the host pools directly: pinned memory
  void* host_ptr[2] = {host_k, host_v};
  for (int i = 0; i < 2; ++i) {
    hipPointerAttribute_t attr;
    if (hipPointerGetAttributes(&attr, host_ptr[i]) != hipSuccess || attr.type != hipMemoryTypeHost) {
      (void)hipGetLastError();
      return fail(PA_ERR_INVALID_ARG, "%s: host pool %d is not pinned host memory", fn, i);
    }
  }
  const bool out = dir == PA_SWAP_OUT;
  const int64_t src_blocks = out ? c.num_blocks : host_num_blocks;
  const int64_t dst_blocks = out ? host_num_blocks : c.num_blocks;
  if (g_debug.load()) {
    std::vector<int64_t> p;
    st = fetch(fn, pairs, 2 * (int64_t)n, (hipStream_t)stream, &p);
    if (st != PA_OK) return st;
    for (int64_t i = 0; i < 2 * (int64_t)n; ++i)
      if (p[i] != pairs_host[i])
        return fail(PA_ERR_INVALID_ARG, "%s: pairs and pairs_host differ at pair %lld", fn, (long long)(i / 2));
    st = pa_check_copy_pairs(pairs_host, n, (int32_t)src_blocks, (int32_t)dst_blocks, 0);
    if (st != PA_OK) return st;
  }
  hipStream_t s = (hipStream_t)stream;
  char* stage[2] = {(char*)staging, (char*)staging + slots * block_bytes};
  char* host[2] = {(char*)host_k, (char*)host_v};
  auto valid = [&](int64_t i) {
    const int64_t a = pairs_host[2 * i], b = pairs_host[2 * i + 1];
    return a >= 0 && a < src_blocks && b >= 0 && b < dst_blocks;
  };
  for (int64_t i0 = 0; i0 < n; i0 += chunk) {
    const int32_t cnt = (int32_t)std::min<int64_t>(chunk, n - i0);
    if (out) {
      hipError_t err = pa::launch_stage_blocks(c, stage[0], stage[1], pairs, i0, cnt, src_blocks, dst_blocks, true, s);
      if (err != hipSuccess) return launched(fn, err);
    }
    // one copy per pool for each run of valid pairs whose host ids are
    // consecutive (their staging slots always are)
    for (int64_t j = 0; j < cnt;) {
      if (!valid(i0 + j)) {
        ++j;
        continue;
      }
      const int64_t host_id = pairs_host[2 * (i0 + j) + (out ? 1 : 0)];
      int64_t len = 1;
      while (j + len < cnt && valid(i0 + j + len) && pairs_host[2 * (i0 + j + len) + (out ? 1 : 0)] == host_id + len)
        ++len;
      for (int pool = 0; pool < 2; ++pool) {
        char* h = host[pool] + host_id * block_bytes;
        char* g = stage[pool] + j * block_bytes;
        const hipError_t err = out ? hipMemcpyAsync(h, g, len * block_bytes, hipMemcpyDeviceToHost, s)
                                   : hipMemcpyAsync(g, h, len * block_bytes, hipMemcpyHostToDevice, s);
        if (err != hipSuccess) return launched(fn, err);
      }
      j += len;
    }
    if (!out) {
      hipError_t err = pa::launch_stage_blocks(c, stage[0], stage[1], pairs, i0, cnt, src_blocks, dst_blocks, false, s);
      if (err != hipSuccess) return launched(fn, err);
    }
  }
  return PA_OK;
}

size_t pa_decode_workspace_bytes(const pa_kv_cache* cache, int32_t S, int32_t max_context_len) {
  pa::Cache c;
  if (check_cache("pa_decode_workspace_bytes", cache, &c) != PA_OK) return (size_t)-1;
  if (S < 0 || max_context_len < 0) {
    fail(PA_ERR_INVALID_ARG, "pa_decode_workspace_bytes: negative size");
    return (size_t)-1;
  }
  if (pa::decode_partition_tokens(c.dtype, c.head_dim, c.block_size) == 0) {
    fail(PA_ERR_UNSUPPORTED, "pa_decode_workspace_bytes: (dtype %d, head_dim %d, block_size %d) not built",
         (int)c.dtype, c.head_dim, c.block_size);
    return (size_t)-1;
  }
  return pa::decode_workspace_bytes(c, S, max_context_len);
}

namespace {

// Checks shared by the decode entry points (everything but the workspace).
pa_status check_decode(const char* fn, const pa::Cache& c, const void* out, pa_dtype out_dtype, const void* query,
                       const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* context_lens,
                       int32_t S, int32_t max_context_len, float scale, int32_t group_size = 1,
                       bool append = false) {
  if (out_dtype != c.dtype && out_dtype != PA_F32)
    return fail(PA_ERR_INVALID_ARG, "%s: out_dtype must be the cache dtype or PA_F32", fn);
  if (!out || !query || !block_tables || !context_lens)
    return fail(PA_ERR_INVALID_ARG, "%s: NULL out/query/block_tables/context_lens", fn);
  if (!aligned(out, 16) || !aligned(query, 16))
    return fail(PA_ERR_INVALID_ARG, "%s: out/query must be 16-byte aligned", fn);
  if (!aligned(block_tables, 4) || !aligned(context_lens, 4))
    return fail(PA_ERR_INVALID_ARG, "%s: block_tables/context_lens must be 4-byte aligned", fn);
  if (max_context_len < 1) return fail(PA_ERR_INVALID_ARG, "%s: max_context_len = %d < 1", fn, max_context_len);
  if (max_blocks_per_seq < 1 || (int64_t)max_blocks_per_seq * c.block_size < max_context_len)
    return fail(PA_ERR_INVALID_ARG, "%s: max_blocks_per_seq = %d cannot hold %d tokens of block %d", fn,
                max_blocks_per_seq, max_context_len, c.block_size);
  if (!std::isfinite(scale)) return fail(PA_ERR_INVALID_ARG, "%s: scale is not finite", fn);
  const int P = pa::decode_partition_tokens(c.dtype, c.head_dim, c.block_size);
  if (P == 0)
    return fail(PA_ERR_UNSUPPORTED, "%s: (dtype %d, head_dim %d, block_size %d) not built", fn, (int)c.dtype,
                c.head_dim, c.block_size);
  // a launch's work-items are counted in 32 bits
  if (S > 0 && pa::decode_work_items(c, S, max_context_len, group_size, append) > (int64_t)UINT32_MAX)
    return fail(PA_ERR_INVALID_ARG, "%s: the launch of S*H*partitions workgroups does not fit", fn);
  return PA_OK;
}

pa_status check_workspace(const char* fn, size_t need, const void* workspace, size_t workspace_bytes) {
  if (need == 0) return PA_OK;
  if (!workspace || workspace_bytes < need)
    return fail(PA_ERR_WORKSPACE, "%s: workspace of %zu bytes given, %zu needed", fn,
                workspace ? workspace_bytes : (size_t)0, need);
  if (!aligned(workspace, 16)) return fail(PA_ERR_INVALID_ARG, "%s: workspace must be 16-byte aligned", fn);
  return PA_OK;
}

}  // namespace

pa_status pa_paged_decode(const pa_kv_cache* cache, void* out, pa_dtype out_dtype, const void* query,
                          const int32_t* block_tables, int32_t max_blocks_per_seq,
                          const int32_t* context_lens, int32_t S, int32_t max_context_len, float scale,
                          void* workspace, size_t workspace_bytes, void* stream) {
  const char* fn = "pa_paged_decode";
  pa::Cache c;
  pa_status st = check_cache(fn, cache, &c);
  if (st != PA_OK) return st;
  if (S < 0) return fail(PA_ERR_INVALID_ARG, "%s: S = %d < 0", fn, S);
  if (S == 0) return PA_OK;
  st = check_decode(fn, c, out, out_dtype, query, block_tables, max_blocks_per_seq, context_lens, S,
                    max_context_len, scale);
  if (st != PA_OK) return st;
  const size_t need = pa::decode_workspace_needed(c, S, max_context_len);
  st = check_workspace(fn, need, workspace, workspace_bytes);
  if (st != PA_OK) return st;
  if (g_debug.load()) {
    st = debug_tables(fn, c, block_tables, max_blocks_per_seq, context_lens, S, max_context_len, (hipStream_t)stream);
    if (st != PA_OK) return st;
  }
  return launched(fn, pa::launch_paged_decode(c, out, out_dtype, query, block_tables, max_blocks_per_seq,
                                              context_lens, S, max_context_len, scale,
                                              need > 0 ? workspace : nullptr, (hipStream_t)stream));
}

pa_status pa_paged_decode_noalloc(const pa_kv_cache* cache, void* out, pa_dtype out_dtype, const void* query,
                                  const int32_t* block_tables, int32_t max_blocks_per_seq,
                                  const int32_t* context_lens, int32_t S, int32_t max_context_len, float scale,
                                  void* stream) {
  const char* fn = "pa_paged_decode_noalloc";
  pa::Cache c;
  pa_status st = check_cache(fn, cache, &c);
  if (st != PA_OK) return st;
  if (S < 0) return fail(PA_ERR_INVALID_ARG, "%s: S = %d < 0", fn, S);
  if (S == 0) return PA_OK;
  st = check_decode(fn, c, out, out_dtype, query, block_tables, max_blocks_per_seq, context_lens, S,
                    max_context_len, scale);
  if (st != PA_OK) return st;
  const size_t need = pa::decode_workspace_needed(c, S, max_context_len);
  if (need > (size_t)PA_NOALLOC_SCRATCH_BYTES)
    return fail(PA_ERR_WORKSPACE, "%s: this call needs %zu bytes of scratch, the library's array holds %zu", fn,
                need, (size_t)PA_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  if (need > 0) {
    const hipError_t err = pa::noalloc_scratch(&ws);
    if (err != hipSuccess)
      return fail(PA_ERR_LAUNCH, "%s: no device address for the scratch array: %s", fn, hipGetErrorString(err));
  }
  return launched(fn, pa::launch_paged_decode(c, out, out_dtype, query, block_tables, max_blocks_per_seq,
                                              context_lens, S, max_context_len, scale, ws, (hipStream_t)stream));
}

size_t pa_decode_grouped_workspace_bytes(const pa_kv_cache* cache, int32_t S, int32_t max_context_len,
                                         int32_t group_size) {
  const char* fn = "pa_decode_grouped_workspace_bytes";
  pa::Cache c;
  if (check_cache(fn, cache, &c) != PA_OK) return (size_t)-1;
  if (S < 0 || max_context_len < 0 || (group_size != 1 && group_size != 2 && group_size != 4)) {
    fail(PA_ERR_INVALID_ARG, "%s: negative size or group_size not in {1, 2, 4}", fn);
    return (size_t)-1;
  }
  if (pa::decode_partition_tokens(c.dtype, c.head_dim, c.block_size) == 0) {
    fail(PA_ERR_UNSUPPORTED, "%s: (dtype %d, head_dim %d, block_size %d) not built", fn, (int)c.dtype,
         c.head_dim, c.block_size);
    return (size_t)-1;
  }
  return pa::decode_grouped_workspace_bytes(c, S, max_context_len, group_size);
}

pa_status pa_paged_decode_grouped(const pa_kv_cache* cache, void* out, pa_dtype out_dtype, const void* query,
                                  const int32_t* block_tables, int32_t max_blocks_per_seq,
                                  const int32_t* context_lens, int32_t S, int32_t max_context_len,
                                  float scale, int32_t group_size, void* workspace, size_t workspace_bytes,
                                  void* stream) {
  const char* fn = "pa_paged_decode_grouped";
  pa::Cache c;
  pa_status st = check_cache(fn, cache, &c);
  if (st != PA_OK) return st;
  if (S < 0) return fail(PA_ERR_INVALID_ARG, "%s: S = %d < 0", fn, S);
  if (group_size != 1 && group_size != 2 && group_size != 4)
    return fail(PA_ERR_INVALID_ARG, "%s: group_size = %d not in {1, 2, 4}", fn, group_size);
  if (S == 0) return PA_OK;
  st = check_decode(fn, c, out, out_dtype, query, block_tables, max_blocks_per_seq, context_lens, S,
                    max_context_len, scale, group_size);
  if (st != PA_OK) return st;
  const size_t need = pa::decode_grouped_workspace_bytes(c, S, max_context_len, group_size);
  st = check_workspace(fn, need, workspace, workspace_bytes);
  if (st != PA_OK) return st;
  if (g_debug.load()) {
    st = debug_tables(fn, c, block_tables, max_blocks_per_seq, context_lens, S, max_context_len, (hipStream_t)stream);
    if (st != PA_OK) return st;
  }
  return launched(fn, pa::launch_paged_decode_grouped(c, out, out_dtype, query, block_tables, max_blocks_per_seq,
                                                      context_lens, S, max_context_len, scale, group_size,
                                                      need > 0 ? workspace : nullptr, (hipStream_t)stream));
}

pa_status pa_paged_decode_append(const pa_kv_cache* cache, void* out, pa_dtype out_dtype, const void* query,
                                 const void* key, const void* value, const int32_t* cow_src,
                                 const int32_t* block_tables,
                                 int32_t max_blocks_per_seq, const int32_t* context_lens, int32_t S,
                                 int32_t max_context_len, float scale, int32_t group_size, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  const char* fn = "pa_paged_decode_append";
  pa::Cache c;
  pa_status st = check_cache(fn, cache, &c);
  if (st != PA_OK) return st;
  if (S < 0) return fail(PA_ERR_INVALID_ARG, "%s: S = %d < 0", fn, S);
  if (group_size != 1 && group_size != 2 && group_size != 4)
    return fail(PA_ERR_INVALID_ARG, "%s: group_size = %d not in {1, 2, 4}", fn, group_size);
  if (S == 0) return PA_OK;
  st = check_decode(fn, c, out, out_dtype, query, block_tables, max_blocks_per_seq, context_lens, S,
                    max_context_len, scale, group_size, true);
  if (st != PA_OK) return st;
  if (!key || !value) return fail(PA_ERR_INVALID_ARG, "%s: NULL key/value", fn);
  if (!aligned(key, 16) || !aligned(value, 16))
    return fail(PA_ERR_INVALID_ARG, "%s: key/value must be 16-byte aligned", fn);
  if (cow_src && !aligned(cow_src, 4)) return fail(PA_ERR_INVALID_ARG, "%s: cow_src must be 4-byte aligned", fn);
  const size_t need = group_size == 1 ? pa::decode_workspace_needed(c, S, max_context_len)
                                      : pa::decode_grouped_workspace_bytes(c, S, max_context_len, group_size);
  st = check_workspace(fn, need, workspace, workspace_bytes);
  if (st != PA_OK) return st;
  if (g_debug.load()) {
    // the tables and lengths as for a decode; new tokens in distinct slots no other row reads
    std::vector<int32_t> t, l;
    st = fetch(fn, block_tables, (int64_t)S * max_blocks_per_seq, (hipStream_t)stream, &t);
    if (st == PA_OK) st = fetch(fn, context_lens, S, (hipStream_t)stream, &l);
    if (st == PA_OK)
      st = pa_check_block_tables(t.data(), S, max_blocks_per_seq, l.data(), max_context_len, c.block_size,
                                 c.num_blocks);
    std::vector<int32_t> cw;
    if (st == PA_OK && cow_src) st = fetch(fn, cow_src, S, (hipStream_t)stream, &cw);
    if (st == PA_OK)
      st = pa_check_append_slots(t.data(), S, max_blocks_per_seq, l.data(), c.block_size,
                                 cow_src ? cw.data() : nullptr, c.num_blocks);
    if (st != PA_OK) return st;
  }
  void* ws = need > 0 ? workspace : nullptr;
  const hipError_t err =
      group_size == 1
          ? pa::launch_paged_decode(c, out, out_dtype, query, block_tables, max_blocks_per_seq, context_lens, S,
                                    max_context_len, scale, ws, (hipStream_t)stream, key, value, cow_src)
          : pa::launch_paged_decode_grouped(c, out, out_dtype, query, block_tables, max_blocks_per_seq,
                                            context_lens, S, max_context_len, scale, group_size, ws,
                                            (hipStream_t)stream, key, value, cow_src);
  return launched(fn, err);
}

pa_status pa_paged_prefill(const pa_kv_cache* cache, void* out, pa_dtype out_dtype, const void* query,
                           const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* cu_q_lens,
                           const int32_t* context_lens, int32_t S, int32_t max_q_len, int32_t max_context_len,
                           float scale, void* stream) {
  const char* fn = "pa_paged_prefill";
  pa::Cache c;
  pa_status st = check_cache(fn, cache, &c);
  if (st != PA_OK) return st;
  if (S < 0) return fail(PA_ERR_INVALID_ARG, "%s: S = %d < 0", fn, S);
  if (S == 0) return PA_OK;
  if (out_dtype != c.dtype && out_dtype != PA_F32)
    return fail(PA_ERR_INVALID_ARG, "%s: out_dtype must be the cache dtype or PA_F32", fn);
  if (!out || !query || !block_tables || !cu_q_lens || !context_lens)
    return fail(PA_ERR_INVALID_ARG, "%s: NULL out/query/block_tables/cu_q_lens/context_lens", fn);
  if (!aligned(out, 16) || !aligned(query, 16))
    return fail(PA_ERR_INVALID_ARG, "%s: out/query must be 16-byte aligned", fn);
  if (!aligned(block_tables, 4) || !aligned(context_lens, 4) || !aligned(cu_q_lens, 4))
    return fail(PA_ERR_INVALID_ARG, "%s: index arrays must be 4-byte aligned", fn);
  if (max_q_len < 1 || max_context_len < max_q_len)
    return fail(PA_ERR_INVALID_ARG, "%s: need 1 <= max_q_len (%d) <= max_context_len (%d)", fn, max_q_len,
                max_context_len);
  if (max_blocks_per_seq < 1 || (int64_t)max_blocks_per_seq * c.block_size < max_context_len)
    return fail(PA_ERR_INVALID_ARG, "%s: max_blocks_per_seq = %d cannot hold %d tokens of block %d", fn,
                max_blocks_per_seq, max_context_len, c.block_size);
  if (!std::isfinite(scale) || !(scale > 0.f))
    return fail(PA_ERR_INVALID_ARG, "%s: scale must be finite and > 0", fn);
  if (!pa::prefill_supported(c.dtype, c.head_dim, c.block_size))
    return fail(PA_ERR_UNSUPPORTED, "%s: (dtype %d, head_dim %d, block_size %d) not built", fn, (int)c.dtype,
                c.head_dim, c.block_size);
  // the launch's work-items (S x heads x query tiles or rows) must fit 32 bits
  const int64_t items = pa::prefill_work_items(c, S, max_q_len);
  if (items > (int64_t)UINT32_MAX)
    return fail(PA_ERR_INVALID_ARG, "%s: %lld work-items (S x heads x queries) exceed the launch limit", fn,
                (long long)items);
  if (g_debug.load()) {
    st = debug_tables(fn, c, block_tables, max_blocks_per_seq, context_lens, S, max_context_len, (hipStream_t)stream);
    std::vector<int32_t> cu, l;
    if (st == PA_OK) st = fetch(fn, cu_q_lens, (int64_t)S + 1, (hipStream_t)stream, &cu);
    if (st == PA_OK) st = fetch(fn, context_lens, S, (hipStream_t)stream, &l);
    if (st == PA_OK) st = pa_check_prefill_rows(cu.data(), l.data(), S, max_q_len);
    if (st != PA_OK) return st;
  }
  return launched(fn, pa::launch_paged_prefill(c, out, out_dtype, query, block_tables, max_blocks_per_seq,
                                               cu_q_lens, context_lens, S, max_q_len, max_context_len, scale,
                                               (hipStream_t)stream));
}

pa_status pa_read_stream(const void* buf, int64_t bytes, void* sink, void* stream) {
  const char* fn = "pa_read_stream";
  if (bytes < 0 || bytes % 16) return fail(PA_ERR_INVALID_ARG, "%s: bytes = %lld must be >= 0 and a multiple of 16", fn,
                                           (long long)bytes);
  if (bytes == 0) return PA_OK;
  if (!buf || !sink) return fail(PA_ERR_INVALID_ARG, "%s: NULL buffer or sink", fn);
  if (!aligned(buf, 16) || !aligned(sink, 16)) return fail(PA_ERR_INVALID_ARG, "%s: pointers must be 16-byte aligned", fn);
  return launched(fn, pa::launch_read_stream(buf, bytes, sink, (hipStream_t)stream));
}

pa_status pa_read_tiles(const void* buf, int64_t tile_bytes, int32_t num_tiles, const int32_t* tiles, int32_t n,
                        void* sink, void* stream) {
  const char* fn = "pa_read_tiles";
  if (tile_bytes <= 0 || tile_bytes % 16)
    return fail(PA_ERR_INVALID_ARG, "%s: tile_bytes = %lld must be > 0 and a multiple of 16", fn, (long long)tile_bytes);
  if (n < 0 || num_tiles < 0) return fail(PA_ERR_INVALID_ARG, "%s: negative size", fn);
  if (n == 0) return PA_OK;
  if (!buf || !tiles || !sink) return fail(PA_ERR_INVALID_ARG, "%s: NULL buffer, tiles or sink", fn);
  if (!aligned(buf, 16) || !aligned(sink, 16) || !aligned(tiles, 4))
    return fail(PA_ERR_INVALID_ARG, "%s: misaligned pointer", fn);
  return launched(fn, pa::launch_read_tiles(buf, tile_bytes, num_tiles, tiles, n, sink, (hipStream_t)stream));
}

const char* pa_status_string(pa_status status) {
  switch (status) {
    case PA_OK: return "PA_OK";
    case PA_ERR_INVALID_ARG: return "PA_ERR_INVALID_ARG";
    case PA_ERR_UNSUPPORTED: return "PA_ERR_UNSUPPORTED";
    case PA_ERR_WORKSPACE: return "PA_ERR_WORKSPACE";
    case PA_ERR_LAUNCH: return "PA_ERR_LAUNCH";
  }
  return "PA_ERR_UNKNOWN";
}

const char* pa_last_error(void) { return g_last_error.c_str(); }

int32_t pa_abi_version(void) { return PA_ABI_VERSION; }

}  // extern "C"
