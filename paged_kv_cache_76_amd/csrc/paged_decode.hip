// Paged decode attention: one query token per sequence attends to the
// sequence's whole key/value history, read block by block through its block
// table.
//
// What is computed ("vLLM / PagedAttention", awesome.papernotes.org, key
// design 1): o = sum_j a_j v_j, a_j = exp(q.k_j * scale) / sum_t exp(q.k_t *
// scale) over the logical history, eq. 2 of the same section evaluating it one
// KV block at a time with each block found through the block table (key
// design 5 fuses that block read into the attention kernel).
//
// gfx950 design (HBM-bound: ~1 flop per byte of K/V):
// * Work item = (head, sequence, context partition of P tokens).  A
//   workgroup of NW wave64s owns one item; its waves take interleaved steps of
//   G tokens.  Long contexts therefore spread over many workgroups, and the
//   partitions are merged exactly (max-rescaled sums) afterwards.
// * Within a wave, LPT = head_dim*bytes/16 lanes hold one token's key or value
//   row (16 bytes each), so one load instruction moves TPL = 64/LPT whole rows:
//   1 KiB of consecutive bytes for a (block, head) tile at fp16/d=128.
// * q.k is a 16-byte dot (v_dot2_f32_f16 / v_dot2_f32_bf16 / fma) followed by
//   a DPP all-reduce across the LPT lanes of the row.  Each row of the wave
//   keeps its own running max / sum / output (a log2-domain online softmax),
//   so no cross-row traffic happens until the partition ends.
// * A wave keeps a 64-entry window of the block table in one register (one
//   entry per lane) and broadcasts entries with readlane, so the dependent
//   table read sits off the per-block critical path.
// * Entries of the table at or beyond ceil(ctx/B) are never read; a block id
//   outside the pool contributes nothing (memory stays in bounds).
#include <algorithm>
#include <mutex>

#include <type_traits>

#include "pa_device.h"
#include "pa_internal.h"

// Tuning knobs.  Defaults are the measured best on MI355X at head_dim 128,
// B=16: non-temporal K/V loads are worth ~14% (the K/V stream is read once
// and must not evict the table, q and partials from L2).  Two partitionings
// are built and picked per launch: the wide one (16 waves x 4096-token
// partitions) beats 8 x 1024 by 1-3% on the OPT-13B step (contexts
// U[1,2048]), a serving mix (lognormal around 400) and 32K contexts, and
// leaves no merge at all for contexts up to 4096; when it would give the
// GPU fewer than kWideMinWorkgroups workgroups (a few long sequences: one
// 32K sequence at 40 heads is 320 of them) the narrow one (8 x 1024) runs,
// 17% faster there.  FUSED (the last partition merges the others after a
// device-scope fence) is kept as a knob only: the fence costs milliseconds
// on this part.
#ifndef PA_DECODE_NW
#define PA_DECODE_NW 16  // waves per workgroup, wide partitioning (head_dim >= 64)
#endif
#ifndef PA_DECODE_PT
#define PA_DECODE_PT 4096  // tokens per context partition, wide partitioning (head_dim >= 64)
#endif
#ifndef PA_DECODE_NW_NARROW
#define PA_DECODE_NW_NARROW 8
#endif
#ifndef PA_DECODE_PT_NARROW
#define PA_DECODE_PT_NARROW 1024
#endif
#ifndef PA_DECODE_WIDE_MIN_WG
#define PA_DECODE_WIDE_MIN_WG 1024  // four per CU of an MI355X
#endif
#ifndef PA_DECODE_NT
#define PA_DECODE_NT 1  // 1: non-temporal K/V loads
#endif
#ifndef PA_DECODE_FUSED
#define PA_DECODE_FUSED 0  // 1: the last partition of a (sequence, head) merges all of them
#endif
#ifndef PA_DECODE_FAST_MERGE
#define PA_DECODE_FAST_MERGE 1  // 1: one-round-trip merge for up to kFastParts partitions
#endif
#ifndef PA_DECODE_MINW
#define PA_DECODE_MINW 0  // >0: ask for at least this many waves per SIMD (caps VGPRs)
#endif
#if PA_DECODE_MINW > 0
#define PA_DECODE_OCC __attribute__((amdgpu_waves_per_eu(PA_DECODE_MINW)))
#else
#define PA_DECODE_OCC
#endif

namespace pa {
namespace {

constexpr float kNegBig = -1e30f;  // finite "minus infinity": keeps exp2 free of NaN
constexpr float kLog2e = 1.44269504088896340736f;

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ u32x4 load_kv(const u32x4* p) {
#if PA_DECODE_NT
  return __builtin_nontemporal_load(p);
#else
  return *p;
#endif
}

struct DecodeArgs {
  const u32x4* q;      // [S][H][D] as 16-byte chunks
  const u32x4* kpool;  // [N][H][B][D]
  const u32x4* vpool;
  const int32_t* tables;
  const int32_t* lens;
  void* out;     // [S][H][D] of out_dtype
  float* ws_o;   // [S][H][max_parts][D]   unnormalised partial outputs
  float* ws_ml;  // [S][H][max_parts][2]   (running max in log2 units, sum)
  int32_t* counters;  // [S][H] arrivals per (sequence, head); zero between calls
  int32_t S, H, N, max_blocks, max_parts;
  float scale_log2;  // scale * log2(e)
  pa_dtype out_dtype;
  // Appending decode: [S][H][D] keys/values of each row's newest token
  // (position lens[s] - 1); NULL for a plain decode, whose tokens are all in
  // the cache already.
  const u32x4* knew;
  const u32x4* vnew;
  // Appending decode with copy-on-write folded in: cow_src[s] >= 0 names the
  // block whose copy the row's newest-token block must first receive (whole
  // block, every head); NULL when there are no copies.
  const int32_t* cow_src;
};

constexpr int cmin(int a, int b) { return a < b ? a : b; }
constexpr int cmax(int a, int b) { return a > b ? a : b; }

template <typename E, int D, int BS, bool WIDE = true>
struct DecodeCfg {
  static constexpr int VEC = 16 / E::bytes;               // elements per 16-byte chunk
  static constexpr int LPT = D / VEC;                     // lanes per token row
  static constexpr int TPL = 64 / LPT;                    // token rows per wave-wide load
  static constexpr int G = cmax(TPL, cmin(BS, 4 * TPL));  // tokens per step
  static constexpr int NCH = G / TPL;                     // loads per lane per step, per pool
  static constexpr bool SMALL = D < 64;
  static constexpr int NW = SMALL ? 1 : (WIDE ? PA_DECODE_NW : PA_DECODE_NW_NARROW);  // waves per workgroup
  static constexpr int PT = SMALL ? 64 : (WIDE ? PA_DECODE_PT : PA_DECODE_PT_NARROW);  // target tokens per partition
  static constexpr int STEPS = cmax(1, PT / G);           // steps per partition
  static constexpr int P = STEPS * G;                     // tokens per partition
  static_assert(D % VEC == 0 && LPT >= 1 && LPT <= 64, "unsupported head_dim");
  static_assert(G % TPL == 0 && (BS >= G ? BS % G == 0 : G % BS == 0), "step/block mismatch");
  static_assert(P % BS == 0, "a partition holds whole blocks");
  static_assert(BS >= G || P / BS <= 64, "multi-block steps keep the partition's table in one register");
};

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) x = fmaxf(x, __shfl_xor(x, off));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) x += __shfl_xor(x, off);
  return x;
}

// Merge of the partitions of one (sequence, head) split into several:
// o = sum_p 2^(m_p - M) o_p / sum_p 2^(m_p - M) l_p with M = max_p m_p.
// Every thread of the block computes M and L (the pairs are few and shared
// through the cache); thread t then owns dims t, t + nthreads, ...
__device__ __forceinline__ void merge_partitions(const DecodeArgs& a, int64_t sh, int nparts, int D,
                                                 int tid, int nthreads) {
  const float* ml = a.ws_ml + sh * a.max_parts * 2;
  const float* po = a.ws_o + sh * a.max_parts * D;
  float M = kNegBig;
  for (int q = 0; q < nparts; ++q) M = fmaxf(M, ml[2 * q]);
  float L = 0.f;
  for (int q = 0; q < nparts; ++q) L += ml[2 * q + 1] * fast_exp2(ml[2 * q] - M);
  const float inv_L = 1.f / L;
  for (int d = tid; d < D; d += nthreads) {
    float O = 0.f;
#pragma unroll 4
    for (int q = 0; q < nparts; ++q) O += po[(int64_t)q * D + d] * fast_exp2(ml[2 * q] - M);
    store_out(a.out, sh * D + d, O * inv_L, a.out_dtype);
  }
}

// An appending decode's newest tokens are fetched at the start of the kernel
// straight into LDS (per row 2 x 64 chunks, K then V, lane k holding chunk
// k % LPT; then 64 copies of the partition kernel's block id), so no
// register is held across the loop, nothing waits for them before it, and
// their latency hides behind it.
template <int ROWS>
struct NewTokenStage {
  u32x4 kv[ROWS][2][64];
  int32_t phys[64];
};
template <int ROWS>
__device__ __forceinline__ NewTokenStage<ROWS>* new_token_stage() {
  __shared__ NewTokenStage<ROWS> stage;
  return &stage;
}

// The cache writes of an appending decode are made by writer workgroups
// appended to the decode grid: each takes NW (row, head) items (item =
// row * H + head), one per wave for the copies, and stores the row's newest
// token of that head into its slot and, for a row with a copy-on-write
// source, copies the row's tokens before the newest (slots [0, off) of the
// head's slice) from the source into the newest-token block.  Dispatched
// last, they run while the decode workgroups drain: measured, the same
// stores issued by the decode workgroups, spread through the read stream,
// cost several times as much.  (One item per wave rather than four: a
// beam-search step 75.8 -> 70.9 us, the copies of a workgroup no longer
// queue behind each other in one wave.)
// Nothing the decode workgroups read is written: a row reads its copied
// block's older tokens from the source (its table entry is patched) and its
// newest token from the inputs, and no other row maps either slot.
__host__ __device__ constexpr int writer_items(int nw) { return nw; }
inline int64_t writer_groups(int64_t S, int64_t H, int nw) {
  return (S * H + writer_items(nw) - 1) / writer_items(nw);
}
// Writer workgroup `wid`; `max_len`: the longest context whose newest token
// the decode adds (longer ones were clipped: nothing is written for them).
// (S * H and the item ids fit 32 bits: the launch's work-items do.)
template <int BS, int LPT, int NW>
__device__ __forceinline__ void write_step(const DecodeArgs& a, int wid, int64_t max_len) {
  constexpr int IPW = writer_items(NW), NT = NW * 64;
  __shared__ int32_t lds_dst[IPW], lds_off[IPW], lds_src[IPW];
  const int item0 = wid * IPW;
  if (threadIdx.x < IPW) {
    const int item = item0 + threadIdx.x;
    int dst = -1, off = 0, src = -1;
    if (item < a.S * a.H) {
      const int row = item / a.H;
      const int len = a.lens[row];
      if (len >= 1 && len <= max_len && (len - 1) / BS < a.max_blocks) {
        const int d = a.tables[(int64_t)row * a.max_blocks + (len - 1) / BS];
        if (d >= 0 && d < a.N) {
          dst = d;
          off = (len - 1) % BS;
          // a source outside the pool copies nothing, like pa_copy_blocks
          if (a.cow_src) {
            const int c = a.cow_src[row];
            src = c >= 0 && c < a.N ? c : -1;
          }
        }
      }
    }
    lds_dst[threadIdx.x] = dst;
    lds_off[threadIdx.x] = off;
    lds_src[threadIdx.x] = src;
  }
  __syncthreads();
  // the newest tokens: (item, pool, chunk) spread over the threads, all
  // loads first, then the stores
  constexpr int TOK = IPW * 2 * LPT, KT = (TOK + NT - 1) / NT;
  u32x4 val[KT];
  int64_t at[KT];
#pragma unroll
  for (int k = 0; k < KT; ++k) {
    const int e = threadIdx.x + k * NT;
    const int i = e / (2 * LPT), pool = (e / LPT) % 2, c = e % LPT;
    at[k] = -1;
    if (e < TOK && lds_dst[i] >= 0) {
      const int item = item0 + i;
      const int h = item % a.H;
      val[k] = (pool ? a.vnew : a.knew)[(int64_t)item * LPT + c];
      at[k] = ((((int64_t)lds_dst[i] * a.H + h) * BS + lds_off[i]) * LPT + c) * 2 + pool;
    }
  }
#pragma unroll
  for (int k = 0; k < KT; ++k) {
    if (at[k] >= 0)
      __builtin_nontemporal_store(val[k], &const_cast<u32x4*>((at[k] & 1) ? a.vpool : a.kpool)[at[k] >> 1]);
  }
  // the copies: one item per wave at a time; a slice's tokens before the
  // newest are one contiguous run of off * LPT chunks per pool
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  for (int i = w; i < IPW; i += NW) {
    const int src = __builtin_amdgcn_readfirstlane(lds_src[i]);
    if (src < 0) continue;
    const int dst = __builtin_amdgcn_readfirstlane(lds_dst[i]);
    const int per_pool = __builtin_amdgcn_readfirstlane(lds_off[i]) * LPT;
    const int h = (item0 + i) % a.H;
    const int64_t s0 = ((int64_t)src * a.H + h) * BS * LPT, d0 = ((int64_t)dst * a.H + h) * BS * LPT;
    constexpr int KC = 8;  // loads in flight per lane
    for (int b = 0; b < 2 * per_pool; b += KC * 64) {
      u32x4 v[KC];
#pragma unroll
      for (int k = 0; k < KC; ++k) {
        const int e = b + k * 64 + lane;
        if (e < 2 * per_pool) v[k] = (e < per_pool ? a.kpool : a.vpool)[s0 + (e < per_pool ? e : e - per_pool)];
      }
#pragma unroll
      for (int k = 0; k < KC; ++k) {
        const int e = b + k * 64 + lane;
        if (e < 2 * per_pool)
          __builtin_nontemporal_store(v[k], &const_cast<u32x4*>(e < per_pool ? a.kpool : a.vpool)
                                                [d0 + (e < per_pool ? e : e - per_pool)]);
      }
    }
  }
}

// The calling wave starts the fetch of element row_h (= row * H + head) of
// knew/vnew into `stage`.
template <int LPT>
__device__ __forceinline__ void fetch_new_token(const DecodeArgs& a, int64_t row_h, int lane, u32x4* stage) {
  const int64_t src = row_h * LPT + lane % LPT;
  load_to_lds(a.knew + src, lds_addr(stage));
  load_to_lds(a.vnew + src, lds_addr(stage + 64));
}

// After the loop, the wave that fetched it: the newest token from `stage`,
// scored against q and folded into token row 0 of the wave's running
// (m, l, o) state (skipped for a block id outside the pool, like every read).
// Every lane scores it (the dot product's lane reduction needs whole lane
// groups); only token row 0 keeps it.
template <typename E, int D, int BS>
__device__ __forceinline__ void add_new_token(const DecodeArgs& a, const u32x4* stage, int lane, int phys,
                                              const u32x4& qc, int r, float& m, float& l, float* o) {
  using C = DecodeCfg<E, D, BS>;
  constexpr int VEC = C::VEC, LPT = C::LPT;
  wait_vmem();  // the fetch into LDS has landed
  const u32x4 kn = stage[lane];
  const u32x4 vn = stage[64 + lane];
  const float d = group_sum<LPT>(dot_chunk(E{}, qc, kn)) * a.scale_log2;
  if (phys < 0 || phys >= a.N) return;  // uniform
  if (r == 0) {
    const float m_new = fmaxf(m, d);
    const float alpha = fast_exp2(m - m_new);
    const float pn = fast_exp2(d - m_new);
    l = l * alpha + pn;
    float vf[VEC];
    widen(E{}, vn, vf);
#pragma unroll
    for (int e = 0; e < VEC; ++e) o[e] = __builtin_fmaf(pn, vf[e], o[e] * alpha);
    m = m_new;
  }
}

// APPEND: the appending decode (knew/vnew set), built apart from the plain
// decode, whose loop it shares unchanged.
template <typename E, int D, int BS, bool WIDE, bool APPEND>
__global__ __launch_bounds__((DecodeCfg<E, D, BS, WIDE>::NW * 64)) PA_DECODE_OCC void decode_partition_kernel(
    DecodeArgs a) {
  using C = DecodeCfg<E, D, BS, WIDE>;
  constexpr int VEC = C::VEC, LPT = C::LPT, TPL = C::TPL, G = C::G, NCH = C::NCH;
  constexpr int NW = C::NW, STEPS = C::STEPS, P = C::P;
  __shared__ float lds_o[NW][D];
  __shared__ float lds_m[NW];
  __shared__ float lds_l[NW];

  const int bid = blockIdx.x;
  if constexpr (APPEND) {
    // the writer workgroups follow the S * H * max_parts decode workgroups
    const int64_t ndec = (int64_t)a.S * a.H * a.max_parts;
    if (__builtin_expect(bid >= ndec, 0)) {
      write_step<BS, LPT, NW>(a, (int)(bid - ndec), (int64_t)a.max_parts * P);
      return;
    }
  }
  const int h = bid % a.H;
  const int rest = bid / a.H;
  const int s = rest % a.S;
  const int p = rest / a.S;
  // a length beyond the grid's partitions is clipped (memory stays in bounds)
  // (an appending decode also reads the row's copy-on-write source, in the
  // same round trip: the lengths again when there is none)
  int len, cow_in = -1;
  if constexpr (APPEND) {
    scalar_load2(a.lens + s, a.cow_src ? a.cow_src + s : a.lens + s, len, cow_in);
    if (!a.cow_src) cow_in = -1;
  } else {
    len = a.lens[s];
  }
  const int ctx = min(len, a.max_parts * P);
  const int nparts = (ctx + P - 1) / P;
  if (p >= nparts) return;  // uniform for the whole workgroup (also ctx < 1)
  // An appending decode reads ctx - 1 tokens from the pools and takes the
  // newest one from its inputs after the loop (not when the length was
  // clipped: then no token is known to be the newest and nothing is written;
  // the writer workgroups make the same choice).
  const bool add_new = APPEND && len <= a.max_parts * P;
  const int kv_ctx = add_new ? ctx - 1 : ctx;

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane / LPT;  // token row within a wave-wide load
  const int c = lane % LPT;  // 16-byte column within the row

  // wave 0 of the partition holding the newest token adds it
  const bool new_part = add_new && (ctx - 1) / P == p;  // this partition holds the newest token
  const bool new_here = new_part && w == 0;
  const int new_blk = (ctx - 1) / BS;  // logical block of the newest token
  NewTokenStage<1>* stage = nullptr;
  // copy-on-write: the newest token's block receives a copy of `cow` (made
  // by a writer workgroup); the row reads that block's older tokens from
  // `cow` itself (an id outside the pool copies nothing, like pa_copy_blocks)
  const int cow = new_part && cow_in >= 0 && cow_in < a.N ? cow_in : -1;
  if constexpr (APPEND) {
    stage = new_token_stage<1>();
    if (new_here) {
      fetch_new_token<LPT>(a, (int64_t)s * a.H + h, lane, &stage->kv[0][0][0]);
      if (new_blk < a.max_blocks)
        load_dword_to_lds(&a.tables[(int64_t)s * a.max_blocks + new_blk], lds_addr(stage->phys));
    }
  }

  const int nblk = (kv_ctx + BS - 1) / BS;  // logical blocks read from the pools
  const int jb = p * (P / BS);           // first logical block of the partition
  const int64_t trow = (int64_t)s * a.max_blocks;
  // table window: lane k holds logical block jb + wbase + k (-1 past the end)
  auto window = [&](int wbase) {
    const int j = jb + wbase + lane;
    int e = (j < nblk && j < a.max_blocks) ? a.tables[trow + j] : -1;
    if (APPEND && j == new_blk && cow >= 0) e = cow;
    return e;
  };
  int wbase = 0;
  int tbl = window(0);

  const u32x4 qc = a.q[((int64_t)s * a.H + h) * LPT + c];

  float m = kNegBig, l = 0.f;
  float o[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) o[e] = 0.f;

  const int nsteps = min(STEPS, (kv_ctx - p * P + G - 1) / G);  // kv_ctx >= p * P
  for (int step = w; step < nsteps; step += NW) {
    const int tb = p * P + step * G;  // first logical token of the step
    const bool full = tb + G <= kv_ctx;

    u32x4 kc[NCH], vc[NCH];
    bool valid[NCH];
    if constexpr (BS >= G) {
      // the whole step lies in one block: a wave-uniform physical id
      const int jl = (step * G) / BS;
      if (jl >= wbase + 64) {
        wbase = jl;
        tbl = window(wbase);
      }
      const int phys = __builtin_amdgcn_readlane(tbl, jl - wbase);
      const bool in_pool = phys >= 0 && phys < a.N;
      const int off0 = (step * G) % BS;
      const int64_t base = (((int64_t)phys * a.H + h) * BS + off0 + r) * LPT + c;
      if (full && in_pool) {
#pragma unroll
        for (int i = 0; i < NCH; ++i) {
          kc[i] = load_kv(&a.kpool[base + i * TPL * LPT]);
          vc[i] = load_kv(&a.vpool[base + i * TPL * LPT]);
          valid[i] = true;
        }
      } else {
#pragma unroll
        for (int i = 0; i < NCH; ++i) {
          valid[i] = in_pool && (tb + i * TPL + r < kv_ctx);
          kc[i] = valid[i] ? load_kv(&a.kpool[base + i * TPL * LPT]) : u32x4{0, 0, 0, 0};
          vc[i] = valid[i] ? load_kv(&a.vpool[base + i * TPL * LPT]) : u32x4{0, 0, 0, 0};
        }
      }
    } else {
      // several blocks per wave-wide load (B < TPL): per-row physical ids
      static_assert(NCH == 1, "multi-block steps use one load per pool");
      const int t = tb + r;
      const int phys = __shfl(tbl, (t - p * P) / BS);
      valid[0] = t < kv_ctx && phys >= 0 && phys < a.N;
      const int64_t idx = (((int64_t)phys * a.H + h) * BS + (t % BS)) * LPT + c;
      kc[0] = valid[0] ? load_kv(&a.kpool[idx]) : u32x4{0, 0, 0, 0};
      vc[0] = valid[0] ? load_kv(&a.vpool[idx]) : u32x4{0, 0, 0, 0};
    }

    float sc[NCH];
    float mblk = kNegBig;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const float d = group_sum<LPT>(dot_chunk(E{}, qc, kc[i])) * a.scale_log2;
      sc[i] = valid[i] ? d : -__builtin_inff();
      mblk = fmaxf(mblk, sc[i]);
    }
    const float m_new = fmaxf(m, mblk);
    const float alpha = fast_exp2(m - m_new);
    l *= alpha;
#pragma unroll
    for (int e = 0; e < VEC; ++e) o[e] *= alpha;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const float pi = fast_exp2(sc[i] - m_new);
      l += pi;
      float vf[VEC];
      widen(E{}, vc[i], vf);
#pragma unroll
      for (int e = 0; e < VEC; ++e) o[e] = __builtin_fmaf(pi, vf[e], o[e]);
    }
    m = m_new;
  }

  if constexpr (APPEND) {
    if (new_here) {
      wait_vmem();  // the fetches into LDS have landed
      const int new_phys = new_blk < a.max_blocks ? __builtin_amdgcn_readfirstlane(stage->phys[0]) : -1;
      add_new_token<E, D, BS>(a, &stage->kv[0][0][0], lane, new_phys, qc, r, m, l, o);
    }
  }

  // Merge the TPL row streams of the wave (lanes with equal column c).
#pragma unroll
  for (int off = LPT; off < 64; off <<= 1) {
    const float m2 = __shfl_xor(m, off);
    const float l2 = __shfl_xor(l, off);
    const float M = fmaxf(m, m2);
    const float f1 = fast_exp2(m - M), f2 = fast_exp2(m2 - M);
    l = l * f1 + l2 * f2;
#pragma unroll
    for (int e = 0; e < VEC; ++e) o[e] = o[e] * f1 + __shfl_xor(o[e], off) * f2;
    m = M;
  }
  if (lane < LPT) {
#pragma unroll
    for (int e = 0; e < VEC; ++e) lds_o[w][c * VEC + e] = o[e];
  }
  if (lane == 0) {
    lds_m[w] = m;
    lds_l[w] = l;
  }
  __syncthreads();

  // Merge the waves and write either the final row or this partition's part.
  float M = kNegBig;
#pragma unroll
  for (int k = 0; k < NW; ++k) M = fmaxf(M, lds_m[k]);
  float L = 0.f;
  float fw[NW];
#pragma unroll
  for (int k = 0; k < NW; ++k) {
    fw[k] = fast_exp2(lds_m[k] - M);
    L += lds_l[k] * fw[k];
  }
  const int64_t sh = (int64_t)s * a.H + h;
  for (int d = threadIdx.x; d < D; d += NW * 64) {
    float O = 0.f;
#pragma unroll
    for (int k = 0; k < NW; ++k) O += lds_o[k][d] * fw[k];
    if (nparts == 1) {
      store_out(a.out, sh * D + d, O / L, a.out_dtype);
    } else {
      a.ws_o[(sh * a.max_parts + p) * D + d] = O;
    }
  }
  if (nparts > 1 && threadIdx.x == 0) {
    a.ws_ml[(sh * a.max_parts + p) * 2] = M;
    a.ws_ml[(sh * a.max_parts + p) * 2 + 1] = L;
  }
#if PA_DECODE_FUSED
  if (nparts > 1) {
    // publish this partition, count arrivals; the last one merges them all
    __shared__ int lds_last;
    __threadfence();
    __syncthreads();
    if (threadIdx.x == 0) lds_last = atomicAdd(&a.counters[sh], 1) == nparts - 1;
    __syncthreads();
    if (!lds_last) return;
    __threadfence();
    merge_partitions(a, sh, nparts, D, threadIdx.x, NW * 64);
    if (threadIdx.x == 0) atomicExch(&a.counters[sh], 0);  // ready for the next call
  }
#endif
}

// ---- grouped decode: rows that share blocks read them once ----------------------
// Consecutive batch rows are taken W at a time.  A workgroup serves one
// (group, head, partition of kGroupTokens tokens); at every block position
// where all W rows map the same physical block (parallel samples or beams
// over a common prefix: "vLLM / PagedAttention", key design 3), the
// (block, head) tile is loaded once and scored against all W queries.
// Anywhere else each row loads its own block.  Each row keeps its own online
// softmax, so the result equals pa_paged_decode's for any grouping; only the
// HBM traffic depends on the sharing.
#ifndef PA_GROUP_NW
#define PA_GROUP_NW 8  // waves per workgroup of the grouped kernel
#endif
#ifndef PA_GROUP_PT
#define PA_GROUP_PT 1024  // tokens per partition of the grouped kernel (a 64-entry table window)
#endif
constexpr int kGroupWaves = PA_GROUP_NW;
constexpr float kGroupSlack = 8.0f;  // lazy-rescale slack of the grouped kernel, log2 units
constexpr int kGroupTokens = PA_GROUP_PT;

template <typename E, int D, int BS, int W, bool APPEND>
// (at B = 16 the W = 4 build fits 4 waves per SIMD without spills; at B = 32 it
// would spill, so it keeps 3)
__global__ __launch_bounds__(kGroupWaves * 64) __attribute__((amdgpu_waves_per_eu(BS <= 16 ? 4 : 3)))
void decode_grouped_kernel(DecodeArgs a, int32_t ngroups) {
  using C = DecodeCfg<E, D, BS>;
  constexpr int VEC = C::VEC, LPT = C::LPT, TPL = C::TPL, G = C::G, NCH = C::NCH;
  constexpr int NW = kGroupWaves, P = kGroupTokens, STEPS = P / G;
  static_assert(BS >= G && P % BS == 0 && P / BS <= 64, "grouped decode needs whole-block steps");
  __shared__ float lds_o[NW][W][D];
  __shared__ float lds_m[NW][W];
  __shared__ float lds_l[NW][W];

  const int bid = blockIdx.x;
  if constexpr (APPEND) {
    // the writer workgroups follow the ngroups * H * max_parts decode workgroups
    const int64_t ndec = (int64_t)ngroups * a.H * a.max_parts;
    if (__builtin_expect(bid >= ndec, 0)) {
      write_step<BS, C::LPT, NW>(a, (int)(bid - ndec), (int64_t)a.max_parts * P);
      return;
    }
  }
  const int h = bid % a.H;
  const int rest = bid / a.H;
  const int grp = rest % ngroups;
  const int p = rest / ngroups;
  const int r0 = grp * W;
  // ctx: the row's tokens; kv_ctx: those read from the pools (an appending
  // decode takes each row's newest token from its inputs after the loops,
  // unless the length was clipped)
  // (the W lengths come in one vector load, lane r holding row r's, instead
  // of one scalar round trip per row)
  const int lens_w = a.lens[min(r0 + min((int)(threadIdx.x & 63), W - 1), a.S - 1)];
  // copy-on-write sources of the rows, loaded the same way
  const int cow_w = (APPEND && a.cow_src) ? a.cow_src[min(r0 + min((int)(threadIdx.x & 63), W - 1), a.S - 1)] : -1;
  int ctx[W], kv_ctx[W];
  int maxctx = 0, max_kv = 0;
#pragma unroll
  for (int r = 0; r < W; ++r) {
    const int len = __builtin_amdgcn_readlane(lens_w, r);
    ctx[r] = (r0 + r < a.S) ? min(len, a.max_parts * P) : 0;
    const bool add_new = APPEND && r0 + r < a.S && len > 0 && len <= a.max_parts * P;
    kv_ctx[r] = add_new ? ctx[r] - 1 : ctx[r];
    maxctx = max(maxctx, ctx[r]);
    max_kv = max(max_kv, kv_ctx[r]);
  }
  if (p * P >= maxctx) return;  // uniform for the whole workgroup

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int tr = lane / LPT;  // token row within a wave-wide load
  const int c = lane % LPT;   // 16-byte column within the row
  const int jb = p * (P / BS);

  // row r's newest token: wave r % NW of the partition that holds it
  NewTokenStage<W>* stage = nullptr;
  if constexpr (APPEND) {
    stage = new_token_stage<W>();
#pragma unroll
    for (int r = 0; r < W; ++r) {
      if (kv_ctx[r] < ctx[r] && (ctx[r] - 1) / P == p && w == r % NW)
        fetch_new_token<LPT>(a, (int64_t)(r0 + r) * a.H + h, lane, &stage->kv[r][0][0]);
    }
  }

  int tbl[W];
  u32x4 qc[W];
  float m[W], l[W], o[W][VEC];
#pragma unroll
  for (int r = 0; r < W; ++r) {
    const int nblk = (ctx[r] + BS - 1) / BS;
    const int j = jb + lane;
    tbl[r] = (lane < P / BS && j < nblk && j < a.max_blocks) ? a.tables[(int64_t)(r0 + r) * a.max_blocks + j] : -1;
    qc[r] = ctx[r] > 0 ? a.q[((int64_t)(r0 + r) * a.H + h) * LPT + c] : u32x4{0, 0, 0, 0};
    m[r] = kNegBig;
    l[r] = 0.f;
#pragma unroll
    for (int e = 0; e < VEC; ++e) o[r][e] = 0.f;
  }

  // Rows whose newest token is in this partition: the block that receives
  // it (new_dst, from the table) and, with copy-on-write folded in, the
  // block it receives a copy of (made by a writer workgroup): the row reads
  // that block's older tokens from the copy's source (its table lane is
  // patched).
  int new_dst[W];
#pragma unroll
  for (int r = 0; r < W; ++r) {
    new_dst[r] = -1;
    if (APPEND && kv_ctx[r] < ctx[r] && (ctx[r] - 1) / P == p) {
      const int jn = (ctx[r] - 1) / BS - jb;  // lane of the newest token's block (< P / BS <= 64)
      new_dst[r] = __builtin_amdgcn_readlane(tbl[r], jn);
      const int src = __builtin_amdgcn_readlane(cow_w, r);
      // an id outside the pool copies nothing, like pa_copy_blocks
      if (src >= 0 && src < a.N && lane == jn) tbl[r] = src;
    }
  }

  // Online-softmax update of row r with one step's chunks; the value
  // chunks are widened one at a time (a shared tile's chunk once for all its
  // rows, below), which keeps the W = 4 kernel at 4 waves per SIMD without
  // spills at B = 16.  Lazy rescale: a lane's reference max only moves when
  // its max grows by more than kGroupSlack (log2 units), so weights stay
  // below 2^kGroupSlack and most steps skip the rescale; numerator and
  // denominator share the reference.
  auto update = [&](const int r, const u32x4* kc, const u32x4* vc, const bool* valid) {
    float sc[NCH];
    float mblk = kNegBig;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const float d = group_sum<LPT>(dot_chunk(E{}, qc[r], kc[i])) * a.scale_log2;
      sc[i] = valid[i] ? d : -__builtin_inff();
      mblk = fmaxf(mblk, sc[i]);
    }
    const bool raise = mblk > m[r] + kGroupSlack;
    if (__any(raise)) {
      const float m_new = raise ? mblk : m[r];
      const float alpha = fast_exp2(m[r] - m_new);
      l[r] *= alpha;
#pragma unroll
      for (int e = 0; e < VEC; ++e) o[r][e] *= alpha;
      m[r] = m_new;
    }
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const float pi = fast_exp2(sc[i] - m[r]);
      l[r] += pi;
      float vf[VEC];
      widen(E{}, vc[i], vf);
#pragma unroll
      for (int e = 0; e < VEC; ++e) o[r][e] = __builtin_fmaf(pi, vf[e], o[r][e]);
    }
  };

  // Steps [0, n_sh): every row of the group maps the step's block to one
  // physical block and has all of the step's tokens -- read once for all
  // rows.  Sharing that comes from forks forms such a prefix; the steps after
  // it (the rows' private tails) are split into one unit per (step, row) and
  // continue the round-robin where the shared steps left off, so a tail step
  // (W loads) does not land on a single wave.  Any step past the prefix is
  // read per row even if it happens to be shared, which is always correct.
  const int nsteps = min(STEPS, (max_kv - p * P + G - 1) / G);  // max_kv >= maxctx - 1 >= p * P
  int n_sh = 0;
  {
    constexpr int NM = (STEPS + 63) / 64;  // steps judged 64 at a time, one per lane
    bool prefix = true;
#pragma unroll
    for (int q = 0; q < NM; ++q) {
      const int st = 64 * q + lane;
      const int tb = p * P + st * G;
      const int jl = (st * G) / BS;  // block of step st within the window (< P / BS <= 64)
      bool sh = st < nsteps;
      int ph0 = 0;
#pragma unroll
      for (int r = 0; r < W; ++r) {
        const int ph = __shfl(tbl[r], jl);
        if (r == 0) ph0 = ph;
        sh = sh && (tb + G <= kv_ctx[r]) && (ph == ph0);
      }
      const uint64_t mask = __ballot(sh && ph0 >= 0 && ph0 < a.N);
      if (prefix) {
        const int run = (~mask) ? __builtin_ctzll(~mask) : 64;  // leading shared steps of this group of 64
        n_sh += run;
        prefix = run == 64;
      }
    }
  }
  for (int step = w; step < n_sh; step += NW) {
    const int jl = (step * G) / BS;
    const int off0 = (step * G) % BS;
    const int phys = __builtin_amdgcn_readlane(tbl[0], jl);
    const int64_t base = (((int64_t)phys * a.H + h) * BS + off0 + tr) * LPT + c;
    u32x4 kc[NCH], vc[NCH];
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      kc[i] = load_kv(&a.kpool[base + i * TPL * LPT]);
      vc[i] = load_kv(&a.vpool[base + i * TPL * LPT]);
    }
    // scores of every row first (the key chunks die here), then one value
    // chunk widened at a time for all rows
    float sc[W][NCH];
#pragma unroll
    for (int r = 0; r < W; ++r) {
      float mblk = kNegBig;
#pragma unroll
      for (int i = 0; i < NCH; ++i) {
        sc[r][i] = group_sum<LPT>(dot_chunk(E{}, qc[r], kc[i])) * a.scale_log2;
        mblk = fmaxf(mblk, sc[r][i]);
      }
      const bool raise = mblk > m[r] + kGroupSlack;
      if (__any(raise)) {
        const float m_new = raise ? mblk : m[r];
        const float alpha = fast_exp2(m[r] - m_new);
        l[r] *= alpha;
#pragma unroll
        for (int e = 0; e < VEC; ++e) o[r][e] *= alpha;
        m[r] = m_new;
      }
    }
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      float vf[VEC];
      widen(E{}, vc[i], vf);
#pragma unroll
      for (int r = 0; r < W; ++r) {
        const float pi = fast_exp2(sc[r][i] - m[r]);
        l[r] += pi;
#pragma unroll
        for (int e = 0; e < VEC; ++e) o[r][e] = __builtin_fmaf(pi, vf[e], o[r][e]);
      }
    }
  }
  // Tail units u = (step - n_sh) * W + row go to wave (n_sh + u) % NW.  As
  // NW is a multiple of W, every unit of a wave has the same row: R below.
  static_assert(NW % W == 0, "the tail split gives each wave one row");
  const int n_units = (nsteps - n_sh) * W;
  const int u0 = ((w - n_sh) % NW + NW) % NW;  // this wave's first unit
  auto tail = [&](auto row_tag) {
    constexpr int R = decltype(row_tag)::value;
    for (int u = u0; u < n_units; u += NW) {
      const int step = n_sh + u / W;
      const int tb = p * P + step * G;
      if (tb >= kv_ctx[R]) continue;  // uniform: the row has no token in this step
      const int jl = (step * G) / BS;
      const int off0 = (step * G) % BS;
      const int phys = __builtin_amdgcn_readlane(tbl[R], jl);
      const bool in_pool = phys >= 0 && phys < a.N;
      const int64_t base = (((int64_t)(in_pool ? phys : 0) * a.H + h) * BS + off0 + tr) * LPT + c;
      u32x4 kc[NCH], vc[NCH];
      bool valid[NCH];
#pragma unroll
      for (int i = 0; i < NCH; ++i) {
        valid[i] = in_pool && (tb + i * TPL + tr < kv_ctx[R]);
        kc[i] = valid[i] ? load_kv(&a.kpool[base + i * TPL * LPT]) : u32x4{0, 0, 0, 0};
        vc[i] = valid[i] ? load_kv(&a.vpool[base + i * TPL * LPT]) : u32x4{0, 0, 0, 0};
      }
      update(R, kc, vc, valid);
    }
  };
  if (n_units > u0) {
    switch (u0 % W) {
      case 0: tail(std::integral_constant<int, 0>{}); break;
      case 1: tail(std::integral_constant<int, 1 % W>{}); break;
      case 2: tail(std::integral_constant<int, 2 % W>{}); break;
      default: tail(std::integral_constant<int, 3 % W>{}); break;
    }
  }

  if constexpr (APPEND) {
#pragma unroll
    for (int r = 0; r < W; ++r) {
      const int pos = ctx[r] - 1;
      if (kv_ctx[r] < ctx[r] && pos / P == p && w == r % NW)
        add_new_token<E, D, BS>(a, &stage->kv[r][0][0], lane, new_dst[r], qc[r], tr, m[r], l[r], o[r]);
    }
  }

  // per row: merge the token rows of the wave, then the waves
#pragma unroll
  for (int r = 0; r < W; ++r) {
#pragma unroll
    for (int off = LPT; off < 64; off <<= 1) {
      const float m2 = __shfl_xor(m[r], off);
      const float l2 = __shfl_xor(l[r], off);
      const float M = fmaxf(m[r], m2);
      const float f1 = fast_exp2(m[r] - M), f2 = fast_exp2(m2 - M);
      l[r] = l[r] * f1 + l2 * f2;
#pragma unroll
      for (int e = 0; e < VEC; ++e) o[r][e] = o[r][e] * f1 + __shfl_xor(o[r][e], off) * f2;
      m[r] = M;
    }
    if (lane < LPT) {
#pragma unroll
      for (int e = 0; e < VEC; ++e) lds_o[w][r][c * VEC + e] = o[r][e];
    }
    if (lane == 0) {
      lds_m[w][r] = m[r];
      lds_l[w][r] = l[r];
    }
  }
  __syncthreads();
#pragma unroll
  for (int r = 0; r < W; ++r) {
    if (p * P >= ctx[r]) continue;  // this row has no token in the partition
    const int nparts = (ctx[r] + P - 1) / P;
    float M = kNegBig;
#pragma unroll
    for (int k = 0; k < NW; ++k) M = fmaxf(M, lds_m[k][r]);
    float L = 0.f;
    float fw[NW];
#pragma unroll
    for (int k = 0; k < NW; ++k) {
      fw[k] = fast_exp2(lds_m[k][r] - M);
      L += lds_l[k][r] * fw[k];
    }
    const int64_t sh = (int64_t)(r0 + r) * a.H + h;
    for (int d = threadIdx.x; d < D; d += NW * 64) {
      float O = 0.f;
#pragma unroll
      for (int k = 0; k < NW; ++k) O += lds_o[k][r][d] * fw[k];
      if (nparts == 1) {
        store_out(a.out, sh * D + d, O / L, a.out_dtype);
      } else {
        a.ws_o[(sh * a.max_parts + p) * D + d] = O;
      }
    }
    if (nparts > 1 && threadIdx.x == 0) {
      a.ws_ml[(sh * a.max_parts + p) * 2] = M;
      a.ws_ml[(sh * a.max_parts + p) * 2 + 1] = L;
    }
  }
}

// Merge of the partitions of each (sequence, head) split into several:
// o = sum_p 2^(m_p - M) o_p / sum_p 2^(m_p - M) l_p with M = max_p m_p.
// One wave per (sequence, head): the (m_p, l_p) pairs are read in parallel,
// one per lane, and the weights go through LDS to the lanes owning the dims.
constexpr int kReduceChunk = 256;  // partitions whose weights sit in LDS at once

constexpr int kFastParts = 4;
__global__ __launch_bounds__(64) void decode_reduce_kernel(DecodeArgs a, int32_t D, int32_t P) {
  __shared__ float lds_w[kReduceChunk];
  const int bid = blockIdx.x;
  const int h = bid % a.H;
  const int s = bid / a.H;
  const int ctx = min(a.lens[s], a.max_parts * P);
  const int nparts = (ctx + P - 1) / P;
  if (nparts <= 1) return;
  const int lane = threadIdx.x;
  const int64_t sh = (int64_t)s * a.H + h;
  const float* ml = a.ws_ml + sh * a.max_parts * 2;
  const float* po = a.ws_o + sh * a.max_parts * D;
  constexpr int kMaxDimsPerLane = 4;  // head_dim <= 256
#if PA_DECODE_FAST_MERGE
  if (nparts <= kFastParts) {
    // few partitions: every lane reads all the (max, sum) pairs and its own
    // dims of every partial output at once (they do not depend on each
    // other), so the merge is one round trip instead of a chain
    float mq[kFastParts], lq[kFastParts], pq[kFastParts][kMaxDimsPerLane];
#pragma unroll
    for (int q = 0; q < kFastParts; ++q) {
      mq[q] = kNegBig;
      lq[q] = 0.f;
      if (q < nparts) {
        mq[q] = ml[2 * q];
        lq[q] = ml[2 * q + 1];
      }
#pragma unroll
      for (int k = 0; k < kMaxDimsPerLane; ++k) {
        const int d = lane + 64 * k;
        pq[q][k] = (q < nparts && d < D) ? po[(int64_t)q * D + d] : 0.f;
      }
    }
    float M = mq[0];
#pragma unroll
    for (int q = 1; q < kFastParts; ++q) M = fmaxf(M, mq[q]);
    float L = 0.f, wq[kFastParts];
#pragma unroll
    for (int q = 0; q < kFastParts; ++q) {
      wq[q] = q < nparts ? fast_exp2(mq[q] - M) : 0.f;
      L += lq[q] * wq[q];
    }
    const float inv_L = 1.f / L;
#pragma unroll
    for (int k = 0; k < kMaxDimsPerLane; ++k) {
      const int d = lane + 64 * k;
      if (d >= D) break;
      float O = 0.f;
#pragma unroll
      for (int q = 0; q < kFastParts; ++q) O += pq[q][k] * wq[q];
      store_out(a.out, sh * D + d, O * inv_L, a.out_dtype);
    }
    return;
  }
#endif
  float mloc = kNegBig;
  for (int q = lane; q < nparts; q += 64) mloc = fmaxf(mloc, ml[2 * q]);
  const float M = wave_max(mloc);
  float lloc = 0.f;
  for (int q = lane; q < nparts; q += 64) lloc += ml[2 * q + 1] * fast_exp2(ml[2 * q] - M);
  const float inv_L = 1.f / wave_sum(lloc);
  float O[kMaxDimsPerLane] = {0.f, 0.f, 0.f, 0.f};
  for (int q0 = 0; q0 < nparts; q0 += kReduceChunk) {
    const int nq = min(kReduceChunk, nparts - q0);
    __syncthreads();
    for (int q = lane; q < nq; q += 64) lds_w[q] = fast_exp2(ml[2 * (q0 + q)] - M);
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kMaxDimsPerLane; ++k) {
      const int d = lane + 64 * k;
      if (d < D) {
        float acc = 0.f;
#pragma unroll 8
        for (int q = 0; q < nq; ++q) acc += po[(int64_t)(q0 + q) * D + d] * lds_w[q];
        O[k] += acc;
      }
    }
  }
#pragma unroll
  for (int k = 0; k < kMaxDimsPerLane; ++k) {
    const int d = lane + 64 * k;
    if (d < D) store_out(a.out, sh * D + d, O[k] * inv_L, a.out_dtype);
  }
}

// ---- instantiation table -------------------------------------------------------
struct Partitioning {
  int P, NW;
  void (*kernel)(DecodeArgs);
  void (*append_kernel)(DecodeArgs);
};
struct Variant {
  pa_dtype dtype;
  int D, BS;
  Partitioning wide, narrow;
};

#define PA_DECODE_PARTITIONING(E, D, BS, WIDE) \
  Partitioning {                                                                                       \
    DecodeCfg<E, D, BS, WIDE>::P, DecodeCfg<E, D, BS, WIDE>::NW, decode_partition_kernel<E, D, BS, WIDE, false>, \
        decode_partition_kernel<E, D, BS, WIDE, true>                                                    \
  }
#define PA_DECODE_VARIANT(E, D, BS) \
  Variant { E::id, D, BS, PA_DECODE_PARTITIONING(E, D, BS, true), PA_DECODE_PARTITIONING(E, D, BS, false) }

#define PA_DECODE_ALL_TYPES(D, BS) \
  PA_DECODE_VARIANT(F32, D, BS), PA_DECODE_VARIANT(F16, D, BS), PA_DECODE_VARIANT(BF16, D, BS)

const Variant kVariants[] = {
    PA_DECODE_ALL_TYPES(8, 4),    PA_DECODE_ALL_TYPES(8, 8),    PA_DECODE_ALL_TYPES(8, 16),
    PA_DECODE_ALL_TYPES(64, 16),  PA_DECODE_ALL_TYPES(64, 32),
    PA_DECODE_ALL_TYPES(128, 8),  PA_DECODE_ALL_TYPES(128, 16), PA_DECODE_ALL_TYPES(128, 32),
    PA_DECODE_ALL_TYPES(128, 64), PA_DECODE_ALL_TYPES(128, 128),
    PA_DECODE_ALL_TYPES(256, 16), PA_DECODE_ALL_TYPES(256, 32),
};

const Variant* find_variant(pa_dtype dtype, int D, int BS) {
  for (const Variant& v : kVariants)
    if (v.dtype == dtype && v.D == D && v.BS == BS) return &v;
  return nullptr;
}

size_t counter_bytes(int32_t S, int32_t H) {
  return ((size_t)S * H * sizeof(int32_t) + 255) / 256 * 256;
}

struct GroupedVariant {
  pa_dtype dtype;
  int D, BS, W;
  void (*kernel)(DecodeArgs, int32_t);
  void (*append_kernel)(DecodeArgs, int32_t);
};

#define PA_GROUPED_VARIANT(E, D, BS, W) \
  GroupedVariant { E::id, D, BS, W, decode_grouped_kernel<E, D, BS, W, false>, decode_grouped_kernel<E, D, BS, W, true> }
#define PA_GROUPED_ALL(BS, W) \
  PA_GROUPED_VARIANT(F32, 128, BS, W), PA_GROUPED_VARIANT(F16, 128, BS, W), PA_GROUPED_VARIANT(BF16, 128, BS, W)

const GroupedVariant kGroupedVariants[] = {PA_GROUPED_ALL(16, 2), PA_GROUPED_ALL(16, 4), PA_GROUPED_ALL(32, 2),
                                           PA_GROUPED_ALL(32, 4)};

const GroupedVariant* find_grouped(pa_dtype dtype, int D, int BS, int W) {
  for (const GroupedVariant& v : kGroupedVariants)
    if (v.dtype == dtype && v.D == D && v.BS == BS && v.W == W) return &v;
  return nullptr;
}

int64_t max_parts_for(const Partitioning& p, int32_t max_context_len) {
  return ((int64_t)max_context_len + p.P - 1) / p.P;
}

// the wide partitioning unless its grid would leave most of the GPU idle
constexpr int64_t kWideMinWorkgroups = PA_DECODE_WIDE_MIN_WG;
const Partitioning& pick_partitioning(const Variant& v, int32_t S, int32_t H, int32_t max_context_len) {
  return (int64_t)S * H * max_parts_for(v.wide, max_context_len) >= kWideMinWorkgroups ? v.wide : v.narrow;
}

}  // namespace

int decode_partition_tokens(pa_dtype dtype, int head_dim, int block_size) {
  const Variant* v = find_variant(dtype, head_dim, block_size);
  return v ? v->wide.P : 0;
}

namespace {
size_t partials_bytes(const Cache& c, int32_t S, int64_t mp) {
  if (mp <= 1) return 0;
  return counter_bytes(S, c.num_heads) + (size_t)S * c.num_heads * mp * (c.head_dim + 2) * sizeof(float);
}
}  // namespace

// What the caller allocates: enough for the narrow partitioning (the one
// with more partitions), so that one workspace serves every launch with at
// most S sequences and max_context_len tokens, whichever partitioning each
// launch picks.
size_t decode_workspace_bytes(const Cache& c, int32_t S, int32_t max_context_len) {
  const Variant* v = find_variant(c.dtype, c.head_dim, c.block_size);
  if (!v) return (size_t)-1;
  return partials_bytes(c, S, max_parts_for(v->narrow, max_context_len));
}

// The most work-items a decode launch of this shape may take (whichever
// partitioning it picks, the grouped kernel's for group_size > 1, plus an
// appending decode's writer workgroups): the caller refuses launches whose
// count does not fit the 32-bit grid size.
int64_t decode_work_items(const Cache& c, int32_t S, int32_t max_context_len, int32_t group_size, bool append) {
  const Variant* v = find_variant(c.dtype, c.head_dim, c.block_size);
  if (!v) return 0;
  int64_t most = 0;
  for (const Partitioning* pt : {&v->wide, &v->narrow}) {
    const int64_t wg = (int64_t)S * c.num_heads * max_parts_for(*pt, max_context_len) +
                       (append ? writer_groups(S, c.num_heads, pt->NW) : 0);
    most = std::max(most, wg * pt->NW * 64);
  }
  if (group_size > 1 && find_grouped(c.dtype, c.head_dim, c.block_size, group_size)) {
    const int64_t mp = ((int64_t)max_context_len + kGroupTokens - 1) / kGroupTokens;
    const int64_t wg = (int64_t)(S + group_size - 1) / group_size * c.num_heads * mp +
                       (append ? writer_groups(S, c.num_heads, kGroupWaves) : 0);
    most = std::max(most, wg * kGroupWaves * 64);
  }
  return most;
}

// What one launch uses (its own partitioning), at most the size above.
size_t decode_workspace_needed(const Cache& c, int32_t S, int32_t max_context_len) {
  const Variant* v = find_variant(c.dtype, c.head_dim, c.block_size);
  if (!v) return (size_t)-1;
  return partials_bytes(c, S, max_parts_for(pick_partitioning(*v, S, c.num_heads, max_context_len),
                                            max_context_len));
}

namespace {

DecodeArgs make_args(const Cache& c, void* out, pa_dtype out_dtype, const void* query,
                     const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* context_lens,
                     int32_t S, int64_t mp, float scale, void* workspace, const void* key_new,
                     const void* value_new, const int32_t* cow_src) {
  DecodeArgs a;
  a.q = (const u32x4*)query;
  a.kpool = (const u32x4*)c.k;
  a.vpool = (const u32x4*)c.v;
  a.tables = block_tables;
  a.lens = context_lens;
  a.out = out;
  // workspace: [counters S*H int32, padded to 256 B][partial o][partial (m, l)]
  const size_t cbytes = counter_bytes(S, c.num_heads);
  a.counters = workspace ? (int32_t*)workspace : nullptr;
  a.ws_o = workspace ? (float*)((char*)workspace + cbytes) : nullptr;
  a.ws_ml = workspace ? a.ws_o + (size_t)S * c.num_heads * mp * c.head_dim : nullptr;
  a.S = S;
  a.H = c.num_heads;
  a.N = c.num_blocks;
  a.max_blocks = max_blocks_per_seq;
  a.max_parts = (int32_t)mp;
  a.scale_log2 = scale * kLog2e;
  a.out_dtype = out_dtype;
  a.knew = (const u32x4*)key_new;
  a.vnew = (const u32x4*)value_new;
  a.cow_src = cow_src;
  return a;
}

}  // namespace

hipError_t launch_paged_decode(const Cache& c, void* out, pa_dtype out_dtype, const void* query,
                               const int32_t* block_tables, int32_t max_blocks_per_seq,
                               const int32_t* context_lens, int32_t S, int32_t max_context_len,
                               float scale, void* workspace, hipStream_t stream, const void* key_new,
                               const void* value_new, const int32_t* cow_src) {
  const Variant* v = find_variant(c.dtype, c.head_dim, c.block_size);
  if (!v) return hipErrorInvalidValue;
  const Partitioning& pt = pick_partitioning(*v, S, c.num_heads, max_context_len);
  const int64_t mp = max_parts_for(pt, max_context_len);
  DecodeArgs a = make_args(c, out, out_dtype, query, block_tables, max_blocks_per_seq, context_lens, S, mp, scale,
                           workspace, key_new, value_new, cow_src);
  // an appending decode's writer workgroups come after the decode's
  const int64_t grid = (int64_t)S * c.num_heads * mp + (key_new ? writer_groups(S, c.num_heads, pt.NW) : 0);
  hipLaunchKernelGGL(key_new ? pt.append_kernel : pt.kernel, dim3((unsigned)grid), dim3(pt.NW * 64), 0, stream, a);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || mp <= 1 || PA_DECODE_FUSED) return err;
  hipLaunchKernelGGL(decode_reduce_kernel, dim3((unsigned)(S * c.num_heads)), dim3(64), 0, stream, a,
                     (int32_t)c.head_dim, (int32_t)pt.P);
  return hipGetLastError();
}

bool decode_grouped_built(pa_dtype dtype, int head_dim, int block_size, int group_size) {
  return find_grouped(dtype, head_dim, block_size, group_size) != nullptr;
}

size_t decode_grouped_workspace_bytes(const Cache& c, int32_t S, int32_t max_context_len, int32_t group_size) {
  if (!find_grouped(c.dtype, c.head_dim, c.block_size, group_size))
    return decode_workspace_bytes(c, S, max_context_len);  // served by the ungrouped kernel
  const int64_t mp = ((int64_t)max_context_len + kGroupTokens - 1) / kGroupTokens;
  if (mp <= 1) return 0;
  return counter_bytes(S, c.num_heads) + (size_t)S * c.num_heads * mp * (c.head_dim + 2) * sizeof(float);
}

hipError_t launch_paged_decode_grouped(const Cache& c, void* out, pa_dtype out_dtype, const void* query,
                                       const int32_t* block_tables, int32_t max_blocks_per_seq,
                                       const int32_t* context_lens, int32_t S, int32_t max_context_len,
                                       float scale, int32_t group_size, void* workspace, hipStream_t stream,
                                       const void* key_new, const void* value_new, const int32_t* cow_src) {
  const GroupedVariant* v = find_grouped(c.dtype, c.head_dim, c.block_size, group_size);
  if (!v)  // no grouped build for this shape: the ungrouped kernel gives the same result
    return launch_paged_decode(c, out, out_dtype, query, block_tables, max_blocks_per_seq, context_lens, S,
                               max_context_len, scale, workspace, stream, key_new, value_new, cow_src);
  const int64_t mp = ((int64_t)max_context_len + kGroupTokens - 1) / kGroupTokens;
  const int32_t ngroups = (S + group_size - 1) / group_size;
  DecodeArgs a = make_args(c, out, out_dtype, query, block_tables, max_blocks_per_seq, context_lens, S, mp, scale,
                           workspace, key_new, value_new, cow_src);
  const int64_t grid =
      (int64_t)ngroups * c.num_heads * mp + (key_new ? writer_groups(S, c.num_heads, kGroupWaves) : 0);
  hipLaunchKernelGGL(key_new ? v->append_kernel : v->kernel, dim3((unsigned)grid), dim3(kGroupWaves * 64), 0,
                     stream, a, ngroups);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || mp <= 1) return err;
  hipLaunchKernelGGL(decode_reduce_kernel, dim3((unsigned)(S * c.num_heads)), dim3(64), 0, stream, a,
                     (int32_t)c.head_dim, (int32_t)kGroupTokens);
  return hipGetLastError();
}

// ---- allocation-free decode: partials in a library-owned device array ---------
// For callers that cannot allocate (graph capture, serving loops, harnesses
// that forbid hipMalloc).  The array exists once per GPU (every device that
// loads this code object holds its own copy) for the life of the process.
// Host code never passes its name to a kernel: on the host the name is a
// stand-in, not the device address.  Each device's address is looked up once,
// with that device current, and kept.  Nothing in the array needs to start at
// zero: every partial the merge kernel reads was written earlier in the same
// call, in stream order, by the partition kernel (the arrival counters are
// used only by the off-by-default fused merge, which this path never runs).
static __device__ __align__(256) unsigned char scratch[PA_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t noalloc_scratch(void** ptr) {
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (err != hipSuccess) return err;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace pa
