/*
 * libpagedattn — paged KV-cache attention for AMD Instinct MI355X (gfx950).
 *
 * The data-parallel hot path of vLLM's PagedAttention as three web pages
 * describe it: every sequence keeps its key/value history in fixed-size KV
 * blocks that need not be adjacent in memory, a per-sequence block table
 * translates logical block j to a physical block id, and attention reads the
 * history through that table.  Cache writes and copy-on-write block copies
 * keep the blocks consistent.
 *
 * Sources cited below by page and section:
 *   [P1] "vLLM / PagedAttention — 把 LLM 服务的瓶颈从显存碎片里救出来"
 *        (awesome.papernotes.org), "方法详解", key designs 1-5.
 *   [P2] "vLLM" notes (formulaic.cloudchewie.com), "PagedAttention 原理" and
 *        "在不同解码策略下的效果".
 *   [P3] "vLLM / PagedAttention (SOSP 2023)" guide (upskillscore),
 *        sections 03-05.
 *
 * Conventions shared by every call
 * --------------------------------
 * - All data pointers are DEVICE pointers owned by the caller (the one
 *   exception: the pinned host pools of pa_swap_blocks); the library never
 *   allocates or frees memory, never synchronises (debug mode aside, below),
 *   and keeps no global mutable state except a thread-local "last error"
 *   string and the process-wide debug switch.
 * - Every compute call is asynchronous on `stream` (a hipStream_t passed as
 *   void*; NULL is the default stream).  Buffers must stay alive until the
 *   stream has executed the call.
 * - Cache layout: separate key and value pools, each
 *   [num_blocks][num_heads][block_size][head_dim], row-major, elements of
 *   `dtype`.  Token offset o of head h in physical block b lives at
 *   pool[b][h][o][:].  A slot is b * block_size + o (int64).
 * - Token rows (keys, values, queries, outputs) are contiguous
 *   [rows][num_heads][head_dim].
 * - Data pointers (pools, rows, outputs) must be 16-byte aligned, and
 *   head_dim * sizeof(dtype) must be a multiple of 16.
 * - Argument checks happen on the host before any launch and return
 *   PA_ERR_INVALID_ARG / PA_ERR_UNSUPPORTED / PA_ERR_WORKSPACE with a message
 *   in pa_last_error().  A failed launch returns PA_ERR_LAUNCH.
 * - Index CONTENTS (slots, block ids, lengths) are preconditions.  The kernels
 *   skip a slot, a pair or a block id outside the pool instead of touching
 *   memory outside it, but the numerical result of such a call is undefined.
 *   In debug mode (pa_set_debug(1), or PA_DEBUG=1 in the environment when the
 *   library loads) every compute call first copies its index arrays to the
 *   host -- synchronously, on its stream -- and checks them with the
 *   pa_check_* functions below; a violated precondition returns
 *   PA_ERR_INVALID_ARG and launches nothing.
 */
#ifndef PAGEDATTN_H
#define PAGEDATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PA_ABI_VERSION 1

typedef enum {
  PA_OK = 0,
  PA_ERR_INVALID_ARG = 1,  /* null pointer, negative size, misalignment, bad dtype */
  PA_ERR_UNSUPPORTED = 2,  /* valid but not built: (dtype, head_dim, block_size) */
  PA_ERR_WORKSPACE = 3,    /* workspace missing or smaller than required */
  PA_ERR_LAUNCH = 4        /* the HIP runtime refused a launch */
} pa_status;

typedef enum { PA_F32 = 0, PA_F16 = 1, PA_BF16 = 2 } pa_dtype;

/* A description of caller-owned cache memory (not owned by the library). */
typedef struct {
  void* k;             /* key pool   [num_blocks][num_heads][block_size][head_dim] */
  void* v;             /* value pool, same shape and dtype                         */
  int32_t num_blocks;  /* physical blocks in each pool, >= 1                       */
  int32_t num_heads;   /* attention heads (keys and values have the same count)    */
  int32_t head_dim;    /* d                                                        */
  int32_t block_size;  /* B, tokens per block, a power of two                      */
  pa_dtype dtype;      /* element type of both pools                               */
} pa_kv_cache;

/*
 * pa_reshape_and_cache — write new tokens' keys and values into their slots.
 * [P1] key design 5 (the new K/V of a layer are reshaped into the block-read
 * layout and written to their positions in one fused operation); [P2]
 * "PagedAttention 原理" (the K/V of the prompt and of each decoded token go
 * into the physical-block slots the block table maps to).
 *
 *   key, value    [T][num_heads][head_dim], cache dtype, 16-byte aligned.
 *   slot_mapping  int64 [T]: slot of token t; a negative slot skips the token.
 *                 Slots are unique within a call (precondition).
 *   T             number of token rows, >= 0; T == 0 is a no-op.
 * Effect: k[slot/B][h][slot%B][:] = key[t][h][:] (same for v), bit-exact.
 */
pa_status pa_reshape_and_cache(const pa_kv_cache* cache, const void* key, const void* value,
                               const int64_t* slot_mapping, int32_t T, void* stream);

/*
 * pa_copy_blocks — batched whole-block copies for copy-on-write.
 * [P1] key design 3 (a write into a block whose reference count exceeds one
 * first copies the block into a newly allocated one) and key design 5 (the
 * many small copies this causes are batched into one kernel instead of one
 * memcpy per block); [P3] section 04 (copy-on-write copies only one block).
 *
 *   pairs  int64 [n][2] = (src, dst) physical ids.  Destinations are distinct
 *          and no destination is also a source (precondition).
 *   n      number of pairs, >= 0; n == 0 is a no-op.
 * Effect: k[dst] = k[src] and v[dst] = v[src] (all heads, all slots), bit-exact.
 */
pa_status pa_copy_blocks(const pa_kv_cache* cache, const int64_t* pairs, int32_t n, void* stream);

/*
 * pa_swap_blocks — move whole blocks between the device pools and a pinned
 * host pool, in one batched call.
 * [P2] 调度和抢占 (a preempted request's KV blocks, all of them, are swapped
 * to CPU memory and brought back when memory frees up); [P3] section 05
 * (all-or-nothing eviction of a sequence's blocks; the swap space lives in
 * CPU RAM); [P1] key design 4.
 *
 *   host_k, host_v   pinned host memory the device can address (hipHostMalloc,
 *                    or a torch tensor with pin_memory=True), each
 *                    [host_num_blocks][num_heads][block_size][head_dim] of the
 *                    cache dtype.  Anything else is rejected (PA_ERR_INVALID_ARG)
 *                    before any launch.
 *   pairs            int64 [n][2] on the device: (src, dst).  PA_SWAP_OUT:
 *                    src = device block, dst = host block; PA_SWAP_IN: src =
 *                    host block, dst = device block.  Destinations distinct.
 * Effect: dst block = src block for keys and values, bit-exact.
 */
typedef enum { PA_SWAP_OUT = 0, PA_SWAP_IN = 1 } pa_swap_dir;
pa_status pa_swap_blocks(const pa_kv_cache* cache, void* host_k, void* host_v, int32_t host_num_blocks,
                         const int64_t* pairs, int32_t n, pa_swap_dir dir, void* stream);

/*
 * pa_swap_blocks_dma — the moves of pa_swap_blocks with the host link driven
 * by the copy engines instead of a kernel.  Swap-out: a short kernel gathers
 * the device blocks into consecutive staging slots (device to device), then
 * one DMA copy per pool moves every run of pairs whose host ids are
 * consecutive; swap-in: the DMA copies first, then a kernel scatters the
 * staging slots into their device blocks.  No compute unit then waits on the
 * host link, which matters when the swap runs beside decode launches
 * (measured at the OPT-13B shape: the kernel form slows a concurrent decode
 * by ~50 %).  [P2] 调度和抢占, [P3] section 05, [P1] key design 4, as
 * pa_swap_blocks.
 *
 *   host_k, host_v   as pa_swap_blocks (pinned host memory, checked).
 *   pairs            int64 [n][2] on the device, (src, dst) as for
 *                    pa_swap_blocks; destinations distinct.  A pair with an
 *                    id outside its pool moves nothing.
 *   pairs_host       the same pairs in host memory (the copies are planned on
 *                    the host); reusable once the call returns.  Debug mode
 *                    checks that the two agree.
 *   staging          device memory, 16-byte aligned, caller-owned: slots of
 *                    one key and one value block (pa_swap_staging_bytes);
 *                    a swap larger than the staging runs in chunks of its
 *                    size, in order on `stream`.  Too small for one block:
 *                    PA_ERR_WORKSPACE.
 * Effect: as pa_swap_blocks, bit-exact; everything is queued on `stream`.
 */
size_t pa_swap_staging_bytes(const pa_kv_cache* cache, int32_t blocks);
pa_status pa_swap_blocks_dma(const pa_kv_cache* cache, void* host_k, void* host_v, int32_t host_num_blocks,
                             const int64_t* pairs, const int64_t* pairs_host, int32_t n, pa_swap_dir dir,
                             void* staging, size_t staging_bytes, void* stream);

/*
 * Workspace of pa_paged_decode, in bytes: enough for every call with at most
 * S sequences whose contexts are at most max_context_len tokens (the size
 * never decreases as S or max_context_len grow).  0 means "no workspace
 * needed".  Returns (size_t)-1 for an unsupported cache description.
 */
size_t pa_decode_workspace_bytes(const pa_kv_cache* cache, int32_t S, int32_t max_context_len);

/*
 * pa_paged_decode — one decode step of attention over paged histories.
 * [P1] key design 1: o = sum_j a_j v_j with a_j = exp(q.k_j * scale) /
 * sum_t exp(q.k_t * scale), evaluated block by block (eq. 2) with blocks
 * gathered through the block table; key design 5 (block reads are fused into
 * the attention kernel).
 *
 *   out            [S][num_heads][head_dim] of out_dtype (cache dtype or PA_F32).
 *   query          [S][num_heads][head_dim], cache dtype.
 *   block_tables   int32 [S][max_blocks_per_seq]; entry j of row s is the
 *                  physical id of logical block j.  Entries at or beyond
 *                  ceil(context_lens[s]/B) are never read.
 *   context_lens   int32 [S], 1 <= context_lens[s] <= max_context_len; counts
 *                  the token being decoded (its K/V are already in the cache).
 *   max_context_len  host-side upper bound of context_lens (sizes the grid).
 *   scale          score scale, usually 1/sqrt(head_dim).
 *   workspace      device scratch of >= pa_decode_workspace_bytes() bytes
 *                  (any content; may be NULL when that size is 0).
 * Accumulation is fp32; the softmax is exact (no approximation).
 */
pa_status pa_paged_decode(const pa_kv_cache* cache, void* out, pa_dtype out_dtype, const void* query,
                          const int32_t* block_tables, int32_t max_blocks_per_seq,
                          const int32_t* context_lens, int32_t S, int32_t max_context_len,
                          float scale, void* workspace, size_t workspace_bytes, void* stream);

/*
 * pa_paged_decode_noalloc — pa_paged_decode for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc.  It computes exactly what pa_paged_decode computes
 * (the same kernels, bit-identical results) but keeps the partial results of
 * long contexts in a scratch array of PA_NOALLOC_SCRATCH_BYTES that the
 * library holds in device memory, one per GPU, until the process ends,
 * instead of in a caller workspace.  It calls no allocator of any kind (debug
 * mode does not apply to it: its checks copy indices into host buffers).
 *   Every argument is as for pa_paged_decode, without the workspace.
 *   A call whose partials need more than PA_NOALLOC_SCRATCH_BYTES (the size
 *   pa_decode_workspace_bytes reports bounds it) returns PA_ERR_WORKSPACE and
 *   launches nothing.
 *   Calls on one GPU share that GPU's array: calls that overlap in time on
 *   one GPU (several streams or threads) race and must be serialised by the
 *   caller.  Calls in one stream are ordered and safe.
 */
#define PA_NOALLOC_SCRATCH_BYTES (32u << 20)
pa_status pa_paged_decode_noalloc(const pa_kv_cache* cache, void* out, pa_dtype out_dtype, const void* query,
                                  const int32_t* block_tables, int32_t max_blocks_per_seq,
                                  const int32_t* context_lens, int32_t S, int32_t max_context_len,
                                  float scale, void* stream);

/*
 * pa_paged_decode_grouped — pa_paged_decode for batches whose rows share
 * blocks (parallel samples or beam candidates over a common prefix).
 * [P1] key design 3 (several logical blocks map to one physical block) and
 * key design 1 (the attention computed is unchanged).
 *
 * Rows are taken group_size at a time (rows 0..g-1, g..2g-1, ...; the last
 * group may be short).  Wherever all rows of a group map a logical block to
 * the same physical block, that block is read from HBM once for the whole
 * group.  The result is the same as pa_paged_decode's for any grouping and
 * any table contents; only the traffic depends on the actual sharing.
 *   group_size  1, 2 or 4 (1, or a shape without a grouped build, runs the
 *               ungrouped kernel).
 *   workspace   >= pa_decode_grouped_workspace_bytes(...) bytes.
 * Every other argument is as for pa_paged_decode.
 */
size_t pa_decode_grouped_workspace_bytes(const pa_kv_cache* cache, int32_t S, int32_t max_context_len,
                                         int32_t group_size);
pa_status pa_paged_decode_grouped(const pa_kv_cache* cache, void* out, pa_dtype out_dtype, const void* query,
                                  const int32_t* block_tables, int32_t max_blocks_per_seq,
                                  const int32_t* context_lens, int32_t S, int32_t max_context_len,
                                  float scale, int32_t group_size, void* workspace, size_t workspace_bytes,
                                  void* stream);

/*
 * pa_paged_decode_append — a decode step that also stores the step's new
 * tokens.  For every row s, key[s] and value[s] (the K/V of its newest token,
 * at position context_lens[s] - 1) are written into the cache slot the row's
 * table maps that position to, and the row's attention over its whole
 * context, that token included, is computed from them.  [P2] "PagedAttention
 * 原理" (a new token's K/V are stored in their block, then attention reads
 * the blocks) with [P1] key design 1 and eq. 2: pa_reshape_and_cache and the
 * decode in one launch instead of two.
 *   key, value   [S][num_heads][head_dim], cache dtype, 16-byte aligned.
 *   cow_src      int32 [S] or NULL.  cow_src[s] >= 0: the block that holds
 *                row s's newest token is a copy-on-write copy of block
 *                cow_src[s] ([P1] key design 3); the call makes it one
 *                before the newest token lands in it, so no separate copy
 *                launch is needed: every head's slots before the newest
 *                token's offset are copied (the row's tokens in that block);
 *                the slots after it hold no token of any row and keep what
 *                they held.  -1: no copy.  Ids outside the pool copy
 *                nothing, as in pa_copy_blocks.
 *   group_size   1 (pa_paged_decode's kernels) or 2 / 4 (pa_paged_decode_grouped's).
 *   workspace    >= pa_decode_grouped_workspace_bytes(cache, S,
 *                max_context_len, group_size) bytes.
 * Every other argument is as for pa_paged_decode.
 * Precondition (the copy-on-write rule of [P1] key design 3): the rows'
 * newest slots are distinct, and no other row of the call reads them (no
 * other row's context reaches that offset of that block); otherwise the
 * result depends on the order in which workgroups run.  With cow_src: a
 * block that receives a copy is mapped by its row alone, no copy reads from
 * a block that receives one, and no write of the call lands in a slot a copy
 * reads (rows that write into a copy's source write at or past the copying
 * row's offset, as siblings over a shared block do).  Debug mode checks all
 * of it (pa_check_append_slots).  Copy-on-write copies not passed in cow_src
 * (pa_copy_blocks) go before this call on the same stream.
 * Cache contents equal pa_copy_blocks with the cow_src pairs, then
 * pa_reshape_and_cache with the slot of position context_lens[s] - 1 for
 * row s, bit for bit, in every slot but those after a copied block's newest
 * token (no row holds a token there); the output equals pa_paged_decode
 * (group_size 1) or pa_paged_decode_grouped after them up to rounding (the
 * newest token is added last).  The writes are made by extra workgroups at
 * the end of the decode's grid (ceil(S * num_heads / waves) of them);
 * the launch's work-items must fit 32 bits (PA_ERR_INVALID_ARG otherwise).
 */
pa_status pa_paged_decode_append(const pa_kv_cache* cache, void* out, pa_dtype out_dtype, const void* query,
                                 const void* key, const void* value, const int32_t* cow_src,
                                 const int32_t* block_tables,
                                 int32_t max_blocks_per_seq, const int32_t* context_lens, int32_t S,
                                 int32_t max_context_len, float scale, int32_t group_size, void* workspace,
                                 size_t workspace_bytes, void* stream);

/*
 * pa_paged_prefill — causal attention for the prompt tokens of S sequences.
 * [P1] key design 1, eq. 1 (query i attends to positions t <= i, itself
 * included) with keys/values read through the block table as in eq. 2;
 * [P2] "PagedAttention 原理" (the prompt's K/V are first written into the
 * mapped slots — call pa_reshape_and_cache before this).
 *
 *   query, out     [sum_s q_len_s][num_heads][head_dim]; rows of sequence s
 *                  are cu_q_lens[s] .. cu_q_lens[s+1]-1.  The call is not
 *                  given their row count: both must hold cu_q_lens[S] rows
 *                  (a precondition; the Python binding checks it in debug
 *                  mode).
 *   block_tables   int32 [S][max_blocks_per_seq] as for pa_paged_decode, except
 *                  that entries at or beyond ceil(context_lens[s]/B) may be
 *                  read (the first tiles' entries are fetched before the
 *                  length is known) but are never used: the whole array must
 *                  be readable.
 *   cu_q_lens      int32 [S+1], cu_q_lens[0] = 0, non-decreasing.
 *   context_lens   int32 [S]; q_len_s <= context_lens[s]; the queries are the
 *                  last q_len_s logical positions of the sequence.
 *   max_q_len, max_context_len  host-side upper bounds.
 *   scale          score scale, finite and > 0 (PA_ERR_INVALID_ARG otherwise).
 *   out_dtype      the cache dtype or PA_F32.
 * head_dim 128 with bf16 or fp16 caches and block_size 16, 32, 64 or 128
 * runs on MFMA (tiles of 128 queries x 64 keys; S * num_heads *
 * ceil(max_q_len / 128) workgroups of 256 threads).  Every other description
 * with head_dim <= 512 (fp32 included, any block size) runs a generic kernel
 * made for correctness rather than speed (one wave per query row and head:
 * S * num_heads * max_q_len workgroups of 64 threads); head_dim > 512 returns
 * PA_ERR_UNSUPPORTED.  The launch's work-items must fit 32 bits
 * (PA_ERR_INVALID_ARG otherwise).  Queries whose q_len is 0 produce no rows.
 */
pa_status pa_paged_prefill(const pa_kv_cache* cache, void* out, pa_dtype out_dtype, const void* query,
                           const int32_t* block_tables, int32_t max_blocks_per_seq,
                           const int32_t* cu_q_lens, const int32_t* context_lens, int32_t S,
                           int32_t max_q_len, int32_t max_context_len, float scale, void* stream);

/*
 * Measurement helpers (not part of the method; the pages define no such
 * operation).  Plain reads with no arithmetic, whose rates are the
 * achievable HBM bandwidth the kernels above are measured against.  Both
 * fold what they read into 16 bytes and write `sink` only if the fold equals
 * a fixed value, so the reads cannot be optimised away; the contents of
 * `sink` afterwards are unspecified.
 *
 * pa_read_stream — read bytes of device memory at buf once, front to back,
 * with 16-byte non-temporal loads.
 *   buf    device, 16-byte aligned; bytes a multiple of 16, >= 0 (0: no-op).
 *   sink   device, 16 bytes, 16-byte aligned.
 *
 * pa_read_tiles — the paged access pattern without its arithmetic: read the
 * n tiles buf + tiles[i] * tile_bytes (i = 0 .. n-1), each tile_bytes long,
 * with 16-byte non-temporal loads.
 *   buf         device, 16-byte aligned, num_tiles * tile_bytes bytes.
 *   tile_bytes  > 0, a multiple of 16.
 *   tiles       device int32 [n], 4-byte aligned; an id outside
 *               [0, num_tiles) is skipped.
 *   n           >= 0 (0: no-op).
 */
pa_status pa_read_stream(const void* buf, int64_t bytes, void* sink, void* stream);
pa_status pa_read_tiles(const void* buf, int64_t tile_bytes, int32_t num_tiles, const int32_t* tiles, int32_t n,
                        void* sink, void* stream);

/*
 * Index-precondition checks (host only: every pointer below is HOST memory;
 * nothing touches a device).  Each returns PA_OK or PA_ERR_INVALID_ARG with
 * the first violation in pa_last_error().
 *
 * pa_check_copy_pairs — the pairs of pa_copy_blocks (same_pool = 1) or of
 * pa_swap_blocks (same_pool = 0, sources and destinations in different
 * pools).  [P1] key design 3 (a copy-on-write copy goes to a newly allocated
 * block) and key design 5 (a step's copies run as one batch): every source in
 * [0, src_blocks), every destination in [0, dst_blocks), destinations
 * distinct, and with same_pool no destination is also a source -- otherwise
 * the batch's result would depend on the order its copies run in.
 *   pairs  int64 [n][2] = (src, dst).
 */
pa_status pa_check_copy_pairs(const int64_t* pairs, int32_t n, int32_t src_blocks, int32_t dst_blocks,
                              int32_t same_pool);
/*
 * pa_check_slot_mapping — the slots of pa_reshape_and_cache ([P2]
 * "PagedAttention 原理": each new token's K/V go to its own slot): every
 * non-negative slot below num_slots (= num_blocks * block_size), no slot
 * written by two tokens.  Negative slots (skipped tokens) may repeat.
 */
pa_status pa_check_slot_mapping(const int64_t* slot_mapping, int32_t T, int64_t num_slots);
/*
 * pa_check_block_tables — the tables and lengths of the attention calls
 * ([P1] key design 2: logical block j of a sequence maps to a physical
 * block): 1 <= context_lens[s] <= max_context_len, ceil(context_lens[s] /
 * block_size) <= max_blocks_per_seq, and each of those entries of row s in
 * [0, num_blocks).  Entries past them are not looked at.
 *   block_tables  int32 [S][max_blocks_per_seq];  context_lens  int32 [S].
 */
pa_status pa_check_block_tables(const int32_t* block_tables, int32_t S, int32_t max_blocks_per_seq,
                                const int32_t* context_lens, int32_t max_context_len, int32_t block_size,
                                int32_t num_blocks);
/*
 * pa_check_append_slots — the tables, lengths and copy sources of
 * pa_paged_decode_append: the slot of each row's newest token (position
 * context_lens[s] - 1) is distinct from every other row's and lies outside
 * every other row's context ([P1] key design 3: a block that receives a
 * token belongs to that sequence alone, the writer of a shared block copies
 * it first); with cow_src (NULL: no copies), each copy's source is in
 * [0, num_blocks) and is not its destination, the destination (the row's
 * newest-token block) is mapped by no other row and receives no other copy,
 * no copy's source receives a copy, and every write into a copy's source
 * lands at or past the copying row's newest offset (the copy reads the
 * slots before it).  Each
 * row needs 1 <= context_lens[s] <= block_size * max_blocks_per_seq.
 *   block_tables  int32 [S][max_blocks_per_seq];  context_lens, cow_src  int32 [S].
 */
pa_status pa_check_append_slots(const int32_t* block_tables, int32_t S, int32_t max_blocks_per_seq,
                                const int32_t* context_lens, int32_t block_size, const int32_t* cow_src,
                                int32_t num_blocks);
/*
 * pa_check_prefill_rows — the query ranges of pa_paged_prefill: cu_q_lens[0]
 * = 0, 0 <= q_len_s = cu_q_lens[s+1] - cu_q_lens[s] <= max_q_len, and q_len_s
 * <= context_lens[s] (the queries are the last q_len_s positions).
 *   cu_q_lens  int32 [S+1];  context_lens  int32 [S].
 */
pa_status pa_check_prefill_rows(const int32_t* cu_q_lens, const int32_t* context_lens, int32_t S,
                                int32_t max_q_len);
/* Debug mode on (non-zero) or off; process-wide. */
void pa_set_debug(int32_t on);
/* 1 when debug mode is on. */
int32_t pa_get_debug(void);

/* Human-readable name of a status code (static storage). */
const char* pa_status_string(pa_status status);
/* Detail of the last non-OK status returned on this thread ("" if none). */
const char* pa_last_error(void);
/* PA_ABI_VERSION of the built library. */
int32_t pa_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDATTN_H */
