// Internal declarations shared by the HIP translation units of libpagedattn.
// Nothing here is part of the C-ABI; the public contract is include/pagedattn.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/pagedattn.h"

namespace pa {

// A validated copy of pa_kv_cache with sizes widened for address arithmetic.
struct Cache {
  void* k;
  void* v;
  int32_t num_blocks;
  int32_t num_heads;
  int32_t head_dim;
  int32_t block_size;
  pa_dtype dtype;
};

inline int dtype_bytes(pa_dtype t) { return t == PA_F32 ? 4 : 2; }

// ---- cache writes and copies (cache_ops.hip) ---------------------------------
// The cache write launches T x ceil(H * vectors per row / kWriteThreads)
// workgroups of kWriteThreads threads.
constexpr int kWriteThreads = 256;
// Launch shape of the copy and swap kernels: grid.x = 2 * pairs (keys and
// values), grid.y = copy_grid_y(c) chunks per block, kCopyThreads threads.
constexpr int kCopyThreads = 256;
constexpr int kCopyUnroll = 4;
inline int64_t copy_grid_y(const Cache& c) {
  const int64_t vec_per_block = (int64_t)c.num_heads * c.block_size * c.head_dim * dtype_bytes(c.dtype) / 16;
  const int64_t per_wg = kCopyThreads * kCopyUnroll;
  return (vec_per_block + per_wg - 1) / per_wg;
}
hipError_t launch_reshape_and_cache(const Cache& c, const void* key, const void* value,
                                    const int64_t* slot_mapping, int32_t T, hipStream_t stream);
hipError_t launch_copy_blocks(const Cache& c, const int64_t* pairs, int32_t n, hipStream_t stream);
// host_k / host_v are device-accessible addresses of pinned host pools of
// host_blocks blocks; to_host: device -> host (pairs = (device, host)).
hipError_t launch_swap_blocks(const Cache& c, void* host_k, void* host_v, int32_t host_blocks,
                              const int64_t* pairs, int32_t n, bool to_host, hipStream_t stream);
// Swap staging for pa_swap_blocks_dma: pairs i0 .. i0 + count - 1 between
// their device blocks and consecutive staging slots (gather: device ->
// staging; otherwise staging -> device).
hipError_t launch_stage_blocks(const Cache& c, void* stage_k, void* stage_v, const int64_t* pairs, int64_t i0,
                               int32_t count, int64_t src_blocks, int64_t dst_blocks, bool gather,
                               hipStream_t stream);

// ---- decode (paged_decode.hip) ------------------------------------------------
// Tokens per context partition for this cache shape, or 0 if the shape is
// not built.
int decode_partition_tokens(pa_dtype dtype, int head_dim, int block_size);
// bytes to allocate (serves every launch of at most S sequences and
// max_context_len tokens) and bytes one such launch uses
size_t decode_workspace_bytes(const Cache& c, int32_t S, int32_t max_context_len);
size_t decode_workspace_needed(const Cache& c, int32_t S, int32_t max_context_len);
// The most work-items a decode launch of this shape may take (0 when the
// shape is not built).
int64_t decode_work_items(const Cache& c, int32_t S, int32_t max_context_len, int32_t group_size, bool append);
// key_new / value_new ([S][H][D], cache dtype): an appending decode, which
// first stores each row's newest token (position context_lens[s] - 1) into
// the cache slot its table maps; NULL for a plain decode.  cow_src ([S] or
// NULL): the copy-on-write source of each row's newest-token block (-1: none).
hipError_t launch_paged_decode(const Cache& c, void* out, pa_dtype out_dtype, const void* query,
                               const int32_t* block_tables, int32_t max_blocks_per_seq,
                               const int32_t* context_lens, int32_t S, int32_t max_context_len,
                               float scale, void* workspace, hipStream_t stream,
                               const void* key_new = nullptr, const void* value_new = nullptr,
                               const int32_t* cow_src = nullptr);

// Device address of the allocation-free decode's scratch array on the
// current device (looked up once per device, then cached).
hipError_t noalloc_scratch(void** ptr);

// Grouped decode: rows taken group_size at a time read shared blocks once.
// Shapes without a grouped build are served by launch_paged_decode.
bool decode_grouped_built(pa_dtype dtype, int head_dim, int block_size, int group_size);
size_t decode_grouped_workspace_bytes(const Cache& c, int32_t S, int32_t max_context_len, int32_t group_size);
hipError_t launch_paged_decode_grouped(const Cache& c, void* out, pa_dtype out_dtype, const void* query,
                                       const int32_t* block_tables, int32_t max_blocks_per_seq,
                                       const int32_t* context_lens, int32_t S, int32_t max_context_len,
                                       float scale, int32_t group_size, void* workspace, hipStream_t stream,
                                       const void* key_new = nullptr, const void* value_new = nullptr,
                                       const int32_t* cow_src = nullptr);

// ---- prefill (paged_prefill.hip) ----------------------------------------------
bool prefill_supported(pa_dtype dtype, int head_dim, int block_size);
// work-items of the prefill launch for this cache description (32-bit limit)
int64_t prefill_work_items(const Cache& c, int32_t S, int32_t max_q_len);
hipError_t launch_paged_prefill(const Cache& c, void* out, pa_dtype out_dtype, const void* query,
                                const int32_t* block_tables, int32_t max_blocks_per_seq,
                                const int32_t* cu_q_lens, const int32_t* context_lens, int32_t S,
                                int32_t max_q_len, int32_t max_context_len, float scale,
                                hipStream_t stream);

// ---- measurement reads (read_bench.hip) -----------------------------------------
hipError_t launch_read_stream(const void* buf, int64_t bytes, void* sink, hipStream_t stream);
hipError_t launch_read_tiles(const void* buf, int64_t tile_bytes, int32_t num_tiles, const int32_t* tiles,
                             int32_t n, void* sink, hipStream_t stream);

}  // namespace pa
