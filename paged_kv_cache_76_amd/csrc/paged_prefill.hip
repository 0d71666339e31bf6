// Paged causal prefill: every prompt token attends to the positions up to and
// including its own, with keys and values read through the block table.
//
// What is computed ("vLLM / PagedAttention", awesome.papernotes.org, key
// design 1): for query i, o_i = sum_{j<=i} a_ij v_j with a_ij = softmax over
// t <= i of q_i.k_t * scale (eq. 1), the keys/values being gathered block by
// block through the sequence's block table (eq. 2).  The queries of sequence s
// are its last q_len_s logical positions; q_len_s = context_len_s is the plain
// prompt case.
//
// gfx950 design (a dense contraction, so MFMA; 128 queries x 64 keys tiles):
// * Workgroup = 4 wave64s = 128 queries of one (sequence, head); wave w owns
//   queries 32w..32w+31.  Key and value tiles of 64 tokens go from their
//   physical blocks straight into LDS (global_load_lds_dwordx4: no registers,
//   no LDS write instructions), both as [token][d] rows of 256 bytes whose
//   16-byte chunks are XOR-swizzled by token so the operand reads below do
//   not conflict on LDS banks.
// * Scores are formed transposed, S^T = K Q^T, with
//   v_mfma_f32_32x32x16_{bf16,f16}: the result layout puts one query per lane
//   column, so the online softmax of a query is in-lane except for one
//   exchange between the two half-waves.
// * O^T += V^T P^T with the same MFMA: the B operand P^T for a 16-key step is
//   exactly 8 of the lane's own score registers (rounded to 16 bits), so P
//   never leaves the registers; the A operand V^T is read from the [token][d]
//   tile with two transposing LDS reads (ds_read_b64_tr_b16).
// * Tiles entirely above the diagonal are never loaded; the diagonal ones are
//   masked per element.  Workgroups are issued heaviest-first (last query tile
//   first), XCD-aware.
// * Software pipeline: keys run one tile ahead of values, so the MFMAs of
//   S(j+1) = K(j+1) Q^T are in flight while the exponentials of S(j) are
//   computed, and P(j) V(j) follows.  LDS holds two key and two value tiles;
//   the loads of K(j+2) and V(j+1) are issued at the start of step j into the
//   buffers the previous barrier released, each wave waits for its own loads
//   at the end of the step, and one barrier per step publishes them.  The
//   block-table entries the workgroup needs are copied to LDS once, and a
//   step reads the entries of the next step's loads.
// * Queries come in and outputs go out as whole 256-byte rows through LDS:
//   the operand layout would otherwise make every load or store instruction
//   touch 16 bytes in each of 32 rows that lie H * 256 bytes apart.
#include <type_traits>

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4_t;

// x combined with the same register of lane (l ^ 32) by a commutative op:
// v_permlane32_swap exchanges the upper half-wave of one register with the
// lower half-wave of another, so with both operands = x the two results hold
// x of lanes l % 32 and 32 + l % 32.  (The result is taken by value as a
// 2-vector: this clang mis-reads element 1 of an `auto` result.)
__device__ __forceinline__ float halves_max(float x) {
  const u32x2 r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, x), __builtin_bit_cast(uint32_t, x),
                                                   false, false);
  const uint32_t lo = r.x, hi = r.y;
  return fmaxf(__builtin_bit_cast(float, lo), __builtin_bit_cast(float, hi));
}
__device__ __forceinline__ float halves_sum(float x) {
  const u32x2 r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, x), __builtin_bit_cast(uint32_t, x),
                                                   false, false);
  const uint32_t lo = r.x, hi = r.y;
  return __builtin_bit_cast(float, lo) + __builtin_bit_cast(float, hi);
}

// Workgroup barrier that orders LDS accesses only.  __syncthreads() also
// releases global memory, which makes every wave wait for all its in-flight
// global loads at each barrier; the waits this kernel needs are explicit.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}
// (wait_vmem, load_to_lds and lds_addr: the device helpers header; this
// kernel orders its direct-to-LDS loads itself: wait_vmem, then a barrier,
// before any wave reads the buffer)
// Four such loads of consecutive 1 KiB global pieces from one address
// register: the immediate offset k * 1024 advances both the global address
// and the LDS address; M0 takes m[k] (so the LDS pieces may have gaps).
__device__ __forceinline__ void load4_to_lds(const void* src, uint32_t m0, uint32_t m1, uint32_t m2, uint32_t m3) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "{m0}"(m0) : "memory");
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off offset:1024" ::"v"(src), "{m0}"(m1) : "memory");
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off offset:2048" ::"v"(src), "{m0}"(m2) : "memory");
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off offset:3072" ::"v"(src), "{m0}"(m3) : "memory");
}

constexpr int kD = 128;         // head_dim
constexpr int kRowBytes = kD * 2;
constexpr int kXcds = 8;        // accelerator complex dies of an MI355X
#ifndef PA_PREFILL_PAIR_GROUP
#define PA_PREFILL_PAIR_GROUP 4
#endif
constexpr int kPairGroup = PA_PREFILL_PAIR_GROUP;  // (sequence, head) pairs ordered together
constexpr float kNegBig = -1e30f;
constexpr float kRescaleLog2 = 8.0f;
constexpr float kLog2e = 1.44269504088896340736f;

// LDS tile layouts.  A token row is 256 bytes; its 16-byte chunk c sits at
// chunk position c ^ swz(t), and the swizzles depend only on t % 4 (a
// token's place within the four a load instruction brings), so all the
// loads of a wave can share one address register.  Keys: rows in groups of
// four, groups 1024 + 64 bytes apart; with chunk ^ (t % 4) the QK operand
// read (one chunk of 16 consecutive tokens per group of lanes) hits all 64
// banks once.  Values: rows 256 bytes apart, chunk ^ 4(t % 4): a transposing
// read takes two adjacent chunks of four consecutive tokens per 16 lanes,
// conflict-free for 32 lanes.
constexpr int kKGroupBytes = 4 * kRowBytes + 64;
__device__ __forceinline__ int k_off(const int t, const int chunk) {
  return (t >> 2) * kKGroupBytes + (t & 3) * kRowBytes + 16 * (chunk ^ (t & 3));
}
__device__ __forceinline__ int v_off(const int t, const int chunk) {
  return t * kRowBytes + 16 * (chunk ^ (4 * (t & 3)));
}

__device__ __forceinline__ f32x16 mfma32(BF16, u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma32(F16, u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0,
                                                0, 0);
}

// two fp32 -> one dword of two 16-bit floats (round to nearest even)
__device__ __forceinline__ uint32_t pack2(BF16, float x, float y) {
  bf16x2 v = {(__bf16)x, (__bf16)y};
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ uint32_t pack2(F16, float x, float y) {
  f16x2 v = {(_Float16)x, (_Float16)y};
  return __builtin_bit_cast(uint32_t, v);
}

// acc + the sum of the eight 16-bit floats of a 16-byte operand: a dot
// product with (1, 1) pairs (products exact, fp32 accumulation)
__device__ __forceinline__ float sum_unpacked(BF16, u32x4 v, float acc) {
  const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
  acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(v.x), one, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(v.y), one, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(v.z), one, acc, false);
  return __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(v.w), one, acc, false);
}
__device__ __forceinline__ float sum_unpacked(F16, u32x4 v, float acc) {
  const f16x2 one = {(_Float16)1.0f, (_Float16)1.0f};
  acc = __builtin_amdgcn_fdot2(as_f16x2(v.x), one, acc, false);
  acc = __builtin_amdgcn_fdot2(as_f16x2(v.y), one, acc, false);
  acc = __builtin_amdgcn_fdot2(as_f16x2(v.z), one, acc, false);
  return __builtin_amdgcn_fdot2(as_f16x2(v.w), one, acc, false);
}

struct PrefillArgs {
  const u32x4* q;  // [sum q][H][D] 16-byte chunks
  const u32x4* kpool;
  const u32x4* vpool;
  const int32_t* tables;
  const int32_t* cu_q;
  const int32_t* lens;
  void* out;
  int32_t S, H, N, max_blocks, ntiles;  // ntiles = ceil(max_q_len / queries per workgroup)
  float scale_log2;
  pa_dtype out_dtype;
};

// One workgroup = NW waves of 32 queries each; key tiles of BN tokens (MB
// blocks of 32).  BN = 32 halves the LDS of a workgroup so that more of them
// share a CU.
template <typename E, int BS, int NW, int BN>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(BN == 32 ? 3 : 2))) void prefill_kernel(
    PrefillArgs a) {
  constexpr int kBM = NW * 32;   // queries per workgroup
  constexpr int MB = BN / 32;    // 32-key blocks per tile
  constexpr int KPW = BN / NW;   // tile keys each wave loads, four per load instruction
  constexpr int kKTileBytes = BN / 4 * kKGroupBytes;
  constexpr int kVTileBytes = BN * kRowBytes;
  constexpr int kTabCache = BN == 32 ? 1024 : 2048;  // block-table entries a workgroup keeps in LDS
  static_assert((BN == 32 || BN == 64) && KPW % 4 == 0 && BS >= 4 && (BN % BS == 0 || BS % BN == 0),
                "block size must tile the key step");
  static_assert(NW % 2 == 0 && NW / 2 * 32 * kRowBytes <= (int)sizeof(uint8_t[2][kVTileBytes]) &&
                    NW / 2 * 32 * kRowBytes <= (int)sizeof(uint8_t[2][kKTileBytes]),
                "the output staging of half the waves fits each tile buffer pair");
  __shared__ __attribute__((aligned(16))) uint8_t lds_k[2][kKTileBytes];
  __shared__ __attribute__((aligned(16))) uint8_t lds_v[2][kVTileBytes];
  __shared__ int32_t lds_tab[kTabCache];

  // XCD-aware order: workgroups are handed to the 8 XCDs round-robin, so
  // XCD x runs blocks x, x+8, ...; give each XCD a contiguous range of the
  // work list, so the key/value tiles every query tile of a (sequence, head)
  // pair re-reads stay in that XCD's L2.  The list takes pairs in groups of
  // kPairGroup (their keys/values fit an XCD's L2 together) and, within a
  // group, query tiles heaviest first across the group's pairs, so the last
  // workgroups dispatched are the short ones.
  const int total = a.ntiles * a.S * a.H;
  const int xcd = blockIdx.x % kXcds;
  const int q8 = total / kXcds, r8 = total % kXcds;
  const int lin = xcd * q8 + min(xcd, r8) + (int)(blockIdx.x / kXcds);
  const int grp0 = lin / (kPairGroup * a.ntiles) * kPairGroup;       // first pair of this group
  const int gn = min(kPairGroup, a.S * a.H - grp0);                 // pairs in this group
  const int gr = lin - grp0 * a.ntiles;
  const int pair = grp0 + gr % gn;
  const int tile = a.ntiles - 1 - gr / gn;
  const int s = pair / a.H;
  const int h = pair % a.H;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);

  // Everything the first tile loads depend on -- the query range, the
  // context length and the block-table entries of the first two tiles and of
  // token 0 -- is read in one batch with a single wait: these reads do not
  // depend on each other, and a chain of dependent reads at the start of
  // every workgroup would leave it idle for several memory round trips.
  constexpr int KPW0 = BN / NW;
  constexpr int NE0 = BS >= KPW0 ? 1 : KPW0 / 4;
  const int64_t trow = (int64_t)s * a.max_blocks;
  const int q_begin = a.cu_q[s];
  const int q_end = a.cu_q[s + 1];
  const int ctx = a.lens[s];
  const int raw_first = a.tables[trow];
  int raw_e0[NE0], raw_e1[NE0];
#pragma unroll
  for (int i = 0; i < NE0; ++i) {
    raw_e0[i] = a.tables[trow + min((KPW0 * w + 4 * i) / BS, a.max_blocks - 1)];
    raw_e1[i] = a.tables[trow + min((BN + KPW0 * w + 4 * i) / BS, a.max_blocks - 1)];
  }
  // keeps the compiler from sinking the reads above past the early exit
  // below (which would serialise them again), and from placing a use of one
  // of them between the reads (which would wait for the first before issuing
  // the rest)
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("" ::"s"(q_begin), "s"(q_end), "s"(ctx), "s"(raw_first));
#pragma unroll
  for (int i = 0; i < NE0; ++i) asm volatile("" ::"s"(raw_e0[i]), "s"(raw_e1[i]));

  const int qlen = q_end - q_begin;
  const int q0 = tile * kBM;  // first query row of this workgroup (within the sequence)
  if (q0 >= qlen || qlen > ctx) return;
  const int pos0 = ctx - qlen;  // logical position of query row 0

  const int g = lane >> 5;     // half-wave
  const int col = lane & 31;   // this lane's query column
  const int qrow = q0 + 32 * w + col;
  const int qpos = pos0 + qrow;

  // B operands of S^T = K Q^T: Q[query][16ks + 8g .. +8] for k-steps ks = 0..7
  // Queries go through LDS when the two value buffers hold the workgroup's
  // query tile: loaded into a lane's operand layout directly, each
  // instruction would fetch 16 bytes from each of 32 rows (rows of [H][d]
  // are 18 KiB apart at 72 heads), which measured ~4 % slower than moving
  // whole rows and redistributing them through LDS.
  constexpr bool kStageQ = NW * 32 * kRowBytes <= 2 * kVTileBytes;
  u32x4 qop[8];
  if constexpr (!kStageQ) {
    const bool valid = qrow < qlen;
    const int64_t qbase = ((int64_t)(q_begin + (valid ? qrow : 0)) * a.H + h) * (kD / 8);
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) qop[ks] = valid ? a.q[qbase + 2 * ks + g] : u32x4{0, 0, 0, 0};
  }

  f32x16 acc_o[4];
#pragma unroll
  for (int dm = 0; dm < 4; ++dm)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc_o[dm][i] = 0.f;
  // running max (raw units) and the denominator as four partial sums, so the
  // per-tile additions form four short dependency chains instead of one
  float m = kNegBig;
  float lp[4] = {0.f, 0.f, 0.f, 0.f};

  // keys needed by the workgroup: positions 0 .. pos0 + min(q0 + kBM, qlen) - 1
  const int last_pos = pos0 + min(q0 + kBM, qlen) - 1;
  const int nkt = last_pos / BN + 1;

  // tiles whose keys all precede every query of the workgroup need no mask
  const int n_full = min(nkt, (pos0 + q0 + 1) / BN);
  const int wave_max_pos = pos0 + min(q0 + 32 * w + 31, qlen - 1);  // last query of this wave
  const int wave_tiles = min(nkt, wave_max_pos / BN + 1);         // tiles with keys this wave needs
  const float c = a.scale_log2;
  // Lazy rescale: the running max used for the weights is only raised (and
  // the accumulators rescaled) when some query's max grows by more than
  // kRescaleLog2 in log2 units.  Weights are then at most 2^kRescaleLog2,
  // and numerator and denominator share the same reference, so the result is
  // unchanged up to rounding; after the first tiles the rescale is rare.
  const float slack = kRescaleLog2 / c;  // in raw score units (c > 0)

  // ---- block table: the entries of the tokens the tiles cover (up to
  // kTabCache of them) are copied to LDS once; entries are clamped into the
  // pool.  Entries past those are never used for a load (tokens at or past
  // the context length are redirected below).
  auto clamp_phys = [&](const int e) { return (e >= 0 && e < a.N) ? e : 0; };
  const int n_tab = min(min(nkt * BN, ctx) - 1, (a.max_blocks - 1) * BS) / BS + 1;
  auto entry = [&](const int blk) -> int {
    const int b = min(blk, a.max_blocks - 1);
    return b < kTabCache ? lds_tab[b] : clamp_phys(a.tables[trow + b]);
  };
  const int64_t first_row = ((int64_t)clamp_phys(raw_first) * a.H + h) * BS;  // token 0 (ctx >= 1)

  // ---- tile loads: wave w brings tokens KPW*w .. KPW*w + KPW-1 of a tile,
  // four (1 KiB) per instruction; lane -> token 4i + lane/16, chunk position
  // lane % 16.  Tokens at or past the context length load the sequence's
  // token 0 instead: finite data, whose scores the causal mask removes and
  // whose weights are then exactly zero.
  const int tok_in_inst = lane >> 4;
  const int chunk_pos = lane & 15;
  // physical blocks of this wave's tokens in tile kt (one per four tokens;
  // a single one when a block holds all of them)
  constexpr int NI = KPW / 4;
  constexpr int NE = BS >= KPW ? 1 : NI;
  auto entries = [&](const int kt, int* ent) {
#pragma unroll
    for (int i = 0; i < NE; ++i) ent[i] = entry((kt * BN + KPW * w + 4 * i) / BS);
  };
  static_assert(NE == NE0 && KPW == KPW0, "early table reads cover the first tiles");
  // LDS byte offset of the first row of tile token t0 (a multiple of 4)
  auto row_base = [&](const int t0, const bool is_v) { return is_v ? t0 * kRowBytes : t0 / 4 * kKGroupBytes; };
  auto issue = [&](const u32x4* pool, uint8_t* dst, const int kt, const int* ent, const bool is_v) {
    const int cpos = is_v ? chunk_pos ^ (4 * tok_in_inst) : chunk_pos ^ tok_in_inst;  // t % 4 == tok_in_inst
    if (NE == 1 && NI == 4 && kt * BN + KPW * (w + 1) <= ctx) {
      // the wave's 16 tokens are consecutive rows of one block, all in the
      // context: one address, four loads with immediate offsets
      const int64_t row = ((int64_t)ent[0] * a.H + h) * BS + (kt * BN + KPW * w) % BS + tok_in_inst;
      const uint32_t m = lds_addr(dst + row_base(KPW * w, is_v));
      const uint32_t gap = is_v ? 0 : kKGroupBytes - 4 * kRowBytes;  // LDS bytes between pieces beyond 1 KiB
      load4_to_lds(pool + row * (kD / 8) + cpos, m, m + gap, m + 2 * gap, m + 3 * gap);
      return;
    }
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int t0 = KPW * w + 4 * i;  // first tile token of this instruction (wave-uniform)
      const int phys = ent[NE == 1 ? 0 : i];
      const int jk = kt * BN + t0 + tok_in_inst;
      const int64_t row = jk < ctx ? ((int64_t)phys * a.H + h) * BS + jk % BS : first_row;
      load_to_lds(pool + row * (kD / 8) + cpos, lds_addr(dst + row_base(t0, is_v)));
    }
  };

  // ---- the three stages of a tile
  // S^T = K Q^T for one key tile (key operand: token 32mb + col, chunk 2ks + g)
  auto qk = [&](const uint8_t* __restrict__ tk, f32x16* acc_s) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc_s[mb][i] = 0.f;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const int t = 32 * mb + col;
        const u32x4 ka = *(const u32x4*)&tk[k_off(t, 2 * ks + g)];
        acc_s[mb] = mfma32(E{}, ka, qop[ks], acc_s[mb]);
      }
  };
  // mask (diagonal tiles), running max, lazy rescale
  auto softmax_max = [&](f32x16* acc_s, const int j0, auto masked_tag) {
    constexpr bool MASKED = decltype(masked_tag)::value;
    float mt[4] = {kNegBig, kNegBig, kNegBig, kNegBig};  // four independent max chains
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        if constexpr (MASKED) {
          const int kpos = j0 + 32 * mb + 8 * (i / 4) + 4 * g + (i % 4);
          if (kpos > qpos) acc_s[mb][i] = -__builtin_inff();
        }
        mt[i & 3] = fmaxf(mt[i & 3], acc_s[mb][i]);
      }
    const float mtile = fmaxf(fmaxf(mt[0], mt[1]), fmaxf(mt[2], mt[3]));
    const float m_new = fmaxf(m, halves_max(mtile));  // raw units (scale > 0 keeps the order)
    if (__any(m_new > m + slack)) {
      const float alpha = __builtin_amdgcn_exp2f((m - m_new) * c);
#pragma unroll
      for (int k = 0; k < 4; ++k) lp[k] *= alpha;
#pragma unroll
      for (int dm = 0; dm < 4; ++dm)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc_o[dm][i] *= alpha;
      m = m_new;
    }
  };
  // P^T operands: k-step (mb, t) takes result elements 8t .. 8t+7 of block mb;
  // the denominator sums the same rounded weights the MFMA multiplies
  auto weights = [&](const f32x16* acc_s, u32x4 (*pb)[2]) {
    const float mc = -m * c;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        float p[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) p[j] = __builtin_amdgcn_exp2f(__builtin_fmaf(acc_s[mb][8 * t + j], c, mc));
        pb[mb][t] = u32x4{pack2(E{}, p[0], p[1]), pack2(E{}, p[2], p[3]), pack2(E{}, p[4], p[5]),
                          pack2(E{}, p[6], p[7])};
        lp[2 * mb + t] = sum_unpacked(E{}, pb[mb][t], lp[2 * mb + t]);
      }
  };
  // O^T += V^T P^T; k-slot (g, j) of step (mb, t) is key 32mb + 16t + 8(j/4) + 4g + j%4.
  // Transposing read: in each 16-lane group, lane r points at 4 dims of
  // token k0 + r/4 and receives the 4 tokens k0 .. k0+3 of one dim.
  const int grp = lane >> 4, r16 = lane & 15;
  auto pv = [&](const uint8_t* __restrict__ tv, u32x4 (*pb)[2]) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int dm = 0; dm < 4; ++dm) {
          const int d = 32 * dm + 16 * (grp & 1) + 4 * (r16 & 3);
          uint32_t va[4];
#pragma unroll
          for (int half = 0; half < 2; ++half) {
            const int tok = 32 * mb + 16 * t + 8 * half + 4 * (grp >> 1) + (r16 >> 2);
            const uint8_t* p = &tv[v_off(tok, d >> 3) + 2 * (d & 7)];
            const s16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)p);
            const u32x2 xw = __builtin_bit_cast(u32x2, x);
            va[2 * half] = xw.x;
            va[2 * half + 1] = xw.y;
          }
          acc_o[dm] = mfma32(E{}, u32x4{va[0], va[1], va[2], va[3]}, pb[mb][t], acc_o[dm]);
        }
  };

  // ---- software pipeline: keys run one tile ahead of values.  Step j
  // holds S(j) (scores of key tile j) on entry, and K(j+1), V(j) in LDS.
  // It starts the loads of K(j+2) and V(j+1) (into the buffers released by
  // the barrier that ended step j-1), finishes the softmax of S(j), forms
  // S(j+1) on the MFMAs while the exponentials of S(j) run, accumulates
  // P(j) V(j), then waits for its loads and ends with a barrier.
  // Query staging (kStageQ): wave w's 32 rows sit where its own share of the
  // value tiles goes -- rows 0-15 in bytes [4 KiB w, 4 KiB (w+1)) of value
  // buffer 0, rows 16-31 at the same place in buffer 1 -- so a wave's value
  // loads overwrite only its own staged queries, after it has read them.
  // Row r is 256 bytes with chunk c at position c ^ (r % 16).  Rows past the
  // query count load the sequence's first query row (finite; their outputs
  // are never stored).
  auto q_stage = [&](const int r) { return &lds_v[r >> 4][KPW * w * kRowBytes + (r & 15) * kRowBytes]; };
  int e0[NE];
#pragma unroll
  for (int i = 0; i < NE; ++i) e0[i] = __builtin_amdgcn_readfirstlane(clamp_phys(raw_e0[i]));
  {
    int e1[NE];
#pragma unroll
    for (int i = 0; i < NE; ++i) e1[i] = __builtin_amdgcn_readfirstlane(clamp_phys(raw_e1[i]));
    if constexpr (kStageQ) {
      static_assert(KPW == 16, "a wave's share of a value tile holds 16 staged query rows");
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int r = 4 * i + tok_in_inst;  // this lane's row; four rows per instruction
        const int row = q0 + 32 * w + r;
        const int64_t src = ((int64_t)(q_begin + (row < qlen ? row : 0)) * a.H + h) * (kD / 8);
        load_to_lds(a.q + src + (chunk_pos ^ (r & 15)), lds_addr(q_stage(4 * i)));
      }
    } else {
      issue(a.vpool, lds_v[0], 0, e0, true);
    }
    issue(a.kpool, lds_k[0], 0, e0, false);
    if (nkt > 1) issue(a.kpool, lds_k[1], 1, e1, false);
  }
  // the LDS copy of the block table, published by the barrier below: all of
  // a thread's entries are requested before the first is stored, so the copy
  // costs one memory round trip whatever its length
  {
    constexpr int kTabRounds = kTabCache / (NW * 64);
    const int nt = min(n_tab, kTabCache);
    int tv[kTabRounds];
#pragma unroll
    for (int r = 0; r < kTabRounds; ++r) {
      const int i = tid + r * NW * 64;
      tv[r] = i < nt ? a.tables[trow + i] : 0;
    }
#pragma unroll
    for (int r = 0; r < kTabRounds; ++r) {
      const int i = tid + r * NW * 64;
      if (i < nt) lds_tab[i] = clamp_phys(tv[r]);
    }
  }
  wait_vmem();
  lds_barrier();  // K(0), K(1), the block-table copy (and V(0) or the staged queries) are visible
  if constexpr (kStageQ) {
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) qop[ks] = *(const u32x4*)(q_stage(col) + 16 * ((2 * ks + g) ^ (col & 15)));
    // the value loads below overwrite this wave's staged rows: its reads
    // must have returned first
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    issue(a.vpool, lds_v[0], 0, e0, true);
  }
  f32x16 s_cur[MB];
  qk(lds_k[0], s_cur);
  lds_barrier();  // every wave has read K(0): its buffer can take K(2)

  // Block-table entries run one step ahead: step j reads (from the LDS
  // copy) the entries of the tiles step j + 1 loads, so the read's latency
  // is spent under step j's arithmetic rather than in front of its loads.
  int ek_next[NE], ev_next[NE];
  entries(2, ek_next);
  entries(1, ev_next);
  auto step = [&](const int j, auto masked_tag, auto has_next_tag, auto first_tag) {
    constexpr bool HAS_NEXT = decltype(has_next_tag)::value;
    {
      int ek[NE], ev[NE];
#pragma unroll
      for (int i = 0; i < NE; ++i) {
        ek[i] = __builtin_amdgcn_readfirstlane(ek_next[i]);
        ev[i] = __builtin_amdgcn_readfirstlane(ev_next[i]);
      }
      if (j + 2 < nkt) issue(a.kpool, lds_k[j & 1], j + 2, ek, false);
      if (j + 1 < nkt) issue(a.vpool, lds_v[(j + 1) & 1], j + 1, ev, true);
      entries(j + 3, ek_next);
      entries(j + 2, ev_next);
    }
    if constexpr (decltype(first_tag)::value) {
      // Step 0 with staged queries: V(0) was requested after the query
      // reads, so P(0) V(0) waits for it.  Every wave takes part (tile 0
      // precedes every query); the step is built masked and with S(1), which
      // is correct for any tile (an unmasked tile masks nothing; S(1) from a
      // buffer never loaded when there is no tile 1 is never used).
      softmax_max(s_cur, 0, masked_tag);
      f32x16 s_next[MB];
      qk(lds_k[1], s_next);
      u32x4 pb[MB][2];
      weights(s_cur, pb);
      // the loads this wave issued after V(0): K(2) and V(1), NI each
      if (nkt > 2) __builtin_amdgcn_s_waitcnt(0x0F70 | (2 * NI));
      else if (nkt > 1) __builtin_amdgcn_s_waitcnt(0x0F70 | NI);
      else wait_vmem();
      lds_barrier();  // V(0) from every wave is visible
      pv(lds_v[0], pb);
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) s_cur[mb] = s_next[mb];
    } else if (j < wave_tiles) {
      softmax_max(s_cur, j * BN, masked_tag);
      f32x16 s_next[MB];
      if constexpr (HAS_NEXT) qk(lds_k[(j + 1) & 1], s_next);
      u32x4 pb[MB][2];
      weights(s_cur, pb);
      pv(lds_v[j & 1], pb);
      if constexpr (HAS_NEXT) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) s_cur[mb] = s_next[mb];
      }
    }
    wait_vmem();
    lds_barrier();
  };
  // unmasked steps whose next tile exists, then masked ones, then the last
  // (with staged queries, step 0 is its own form)
  int j = 0;
  const int last = nkt - 1;
  constexpr std::false_type no;
  constexpr std::true_type yes;
  if constexpr (kStageQ) {
    step(0, yes, yes, yes);
    j = 1;
  }
  for (; j < min(n_full, last); ++j) step(j, no, yes, no);
  for (; j < min(last, wave_tiles - 1); ++j) step(j, yes, yes, no);
  for (; j < last; ++j) step(j, yes, no, no);  // this wave's last tile, then none
  if (j == last) {
    if (last < n_full) step(last, no, no, no);
    else step(last, yes, no, no);
  }

  // normalise and store: result element i of block dm is dim 32dm + 8(i/4) + 4g + i%4
  const float l = halves_sum((lp[0] + lp[1]) + (lp[2] + lp[3]));
  const float inv_l = 1.f / l;
  if (a.out_dtype == E::id) {
    // In the cache dtype the rows go out whole: a lane holds 4 dims of one
    // query per result block, so storing from registers would touch 32 rows
    // (18 KiB apart) per instruction, 16 bytes each.  Each wave instead puts
    // its 32 x 128 tile into LDS (free after the last barrier; wave-private
    // regions, so no further barrier), rows 256 bytes apart with 16-byte
    // chunk c at position c ^ (row % 16), and reads it back as 4 whole rows
    // per instruction.
    uint8_t* const stage = (w < NW / 2 ? &lds_k[0][0] : &lds_v[0][0]) + (w % (NW / 2)) * (32 * kRowBytes);
#pragma unroll
    for (int dm = 0; dm < 4; ++dm)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const float o0 = acc_o[dm][4 * r4] * inv_l, o1 = acc_o[dm][4 * r4 + 1] * inv_l;
        const float o2 = acc_o[dm][4 * r4 + 2] * inv_l, o3 = acc_o[dm][4 * r4 + 3] * inv_l;
        const u32x2 v = {pack2(E{}, o0, o1), pack2(E{}, o2, o3)};
        *(u32x2*)&stage[col * kRowBytes + 16 * ((4 * dm + r4) ^ (col & 15)) + 8 * g] = v;
      }
    const int c = lane & 15;
    u32x4 rows[8];  // all eight reads in flight before the first store
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int r = 4 * j + (lane >> 4);
      rows[j] = *(const u32x4*)&stage[r * kRowBytes + 16 * (c ^ (r & 15))];
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int row = q0 + 32 * w + 4 * j + (lane >> 4);
      if (row < qlen) *(u32x4*)((uint16_t*)a.out + ((int64_t)(q_begin + row) * a.H + h) * kD + 8 * c) = rows[j];
    }
    return;
  }
  if (qrow >= qlen || a.out_dtype != PA_F32) return;
  const int64_t obase = ((int64_t)(q_begin + qrow) * a.H + h) * kD;
#pragma unroll
  for (int dm = 0; dm < 4; ++dm)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const int d = 32 * dm + 8 * r4 + 4 * g;
      float4 v = {acc_o[dm][4 * r4] * inv_l, acc_o[dm][4 * r4 + 1] * inv_l, acc_o[dm][4 * r4 + 2] * inv_l,
                  acc_o[dm][4 * r4 + 3] * inv_l};
      *(float4*)((float*)a.out + obase + d) = v;
    }
}


// ---- generic path --------------------------------------------------------------
// Every cache description the MFMA kernel is not built for (fp32, other head
// dims, small blocks) takes this kernel: one wave per (query row, head).  A
// query row is the decode of its own position over the keys t <= position
// (the same sum as above, [P1] key design 1 eq. 1, read through the table as
// in eq. 2).  Lanes take 64 keys at a time for the scores (fp32 dot products
// against the query held in LDS), the running max and sum are wave-wide, and
// for P V the lanes take head dims.  Made for correctness on small shapes,
// not for speed; a block id outside the pool contributes nothing.
constexpr int kGenericMaxD = 512;

__device__ __forceinline__ float load_elem(F32, const void* p, int64_t i) { return ((const float*)p)[i]; }
__device__ __forceinline__ float load_elem(F16, const void* p, int64_t i) {
  return (float)((const _Float16*)p)[i];
}
__device__ __forceinline__ float load_elem(BF16, const void* p, int64_t i) {
  return __uint_as_float((uint32_t)((const uint16_t*)p)[i] << 16);
}
__device__ __forceinline__ float wave_max64(float x) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) x = fmaxf(x, __shfl_xor(x, off));
  return x;
}
__device__ __forceinline__ float wave_sum64(float x) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) x += __shfl_xor(x, off);
  return x;
}

template <typename E>
__global__ __launch_bounds__(64) void prefill_generic_kernel(PrefillArgs a, int32_t D, int32_t BS,
                                                              int32_t max_q_len) {
  constexpr int kSlots = kGenericMaxD / 64;  // head dims per lane
  __shared__ float q_lds[kGenericMaxD];
  __shared__ float p_lds[64];
  __shared__ int64_t row_lds[64];
  const int lane = threadIdx.x;
  const int64_t bid = blockIdx.x;
  const int h = (int)(bid % a.H);
  const int64_t rest = bid / a.H;
  const int i = (int)(rest % max_q_len);
  const int s = (int)(rest / max_q_len);
  const int q_begin = a.cu_q[s];
  const int qlen = a.cu_q[s + 1] - q_begin;
  const int ctx = a.lens[s];
  if (i >= qlen || qlen > ctx) return;  // uniform for the wave
  const int nkeys = ctx - qlen + i + 1;  // causal: positions 0 .. the query's own
  const int64_t qrow = (int64_t)(q_begin + i) * a.H + h;
  for (int d = lane; d < D; d += 64) q_lds[d] = load_elem(E{}, a.q, qrow * D + d);
  __syncthreads();

  float o[kSlots];
#pragma unroll
  for (int k = 0; k < kSlots; ++k) o[k] = 0.f;
  float m = kNegBig, l = 0.f;  // running max (log2 units) and sum
  const int64_t trow = (int64_t)s * a.max_blocks;
  for (int t0 = 0; t0 < nkeys; t0 += 64) {
    const int t = t0 + lane;
    float sc = -__builtin_inff();
    int64_t row = -1;
    // a key whose logical block lies past the table row (a context length
    // beyond max_blocks * B) is treated like one outside the pool
    if (t < nkeys && t / BS < a.max_blocks) {
      const int phys = a.tables[trow + t / BS];
      if (phys >= 0 && phys < a.N) {
        row = ((int64_t)phys * a.H + h) * BS + t % BS;
        float acc = 0.f;
        for (int d = 0; d < D; ++d) acc = __builtin_fmaf(q_lds[d], load_elem(E{}, a.kpool, row * D + d), acc);
        sc = acc * a.scale_log2;
      }
    }
    const float m_new = fmaxf(m, wave_max64(sc));
    const float alpha = __builtin_amdgcn_exp2f(m - m_new);
    const float p = row >= 0 ? __builtin_amdgcn_exp2f(sc - m_new) : 0.f;
    l = l * alpha + wave_sum64(p);
    p_lds[lane] = p;
    row_lds[lane] = row;
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kSlots; ++k) o[k] *= alpha;
    const int nj = min(64, nkeys - t0);
    for (int j = 0; j < nj; ++j) {
      const int64_t rj = row_lds[j];
      if (rj < 0) continue;  // uniform: every lane reads the same entry
      const float pj = p_lds[j];
#pragma unroll
      for (int k = 0; k < kSlots; ++k) {
        const int d = lane + 64 * k;
        if (d < D) o[k] = __builtin_fmaf(pj, load_elem(E{}, a.vpool, rj * D + d), o[k]);
      }
    }
    m = m_new;
    __syncthreads();
  }
  // no usable key at all (every block outside the pool): zeros, not 0/0
  const float inv_l = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
  for (int k = 0; k < kSlots; ++k) {
    const int d = lane + 64 * k;
    if (d < D) store_out(a.out, qrow * D + d, o[k] * inv_l, a.out_dtype);
  }
}

#ifndef PA_PREFILL_BN
#define PA_PREFILL_BN 64  // keys per tile
#endif
#ifndef PA_PREFILL_NW
#define PA_PREFILL_NW 4  // waves per workgroup
#endif
constexpr int kNW = PA_PREFILL_NW;
constexpr int kTileQ = kNW * 32;  // queries per workgroup

struct Variant {
  pa_dtype dtype;
  int BS;
  void (*kernel)(PrefillArgs);
};

#define PA_PREFILL_VARIANTS(BS)                                    \
  Variant{PA_BF16, BS, prefill_kernel<BF16, BS, kNW, PA_PREFILL_BN>}, Variant { \
    PA_F16, BS, prefill_kernel<F16, BS, kNW, PA_PREFILL_BN>                     \
  }

const Variant kVariants[] = {PA_PREFILL_VARIANTS(16), PA_PREFILL_VARIANTS(32), PA_PREFILL_VARIANTS(64),
                             PA_PREFILL_VARIANTS(128)};

const Variant* find_variant(pa_dtype dtype, int head_dim, int block_size) {
  if (head_dim != kD) return nullptr;
  for (const Variant& v : kVariants)
    if (v.dtype == dtype && v.BS == block_size) return &v;
  return nullptr;
}

}  // namespace

bool prefill_supported(pa_dtype dtype, int head_dim, int block_size) {
  return find_variant(dtype, head_dim, block_size) != nullptr || (head_dim >= 1 && head_dim <= kGenericMaxD &&
                                                                  block_size >= 1);
}

int64_t prefill_work_items(const Cache& c, int32_t S, int32_t max_q_len) {
  if (find_variant(c.dtype, c.head_dim, c.block_size))
    return ((int64_t)max_q_len + kTileQ - 1) / kTileQ * S * c.num_heads * (kNW * 64);
  return (int64_t)max_q_len * S * c.num_heads * 64;
}

hipError_t launch_paged_prefill(const Cache& c, void* out, pa_dtype out_dtype, const void* query,
                                const int32_t* block_tables, int32_t max_blocks_per_seq,
                                const int32_t* cu_q_lens, const int32_t* context_lens, int32_t S,
                                int32_t max_q_len, int32_t max_context_len, float scale,
                                hipStream_t stream) {
  (void)max_context_len;
  const Variant* v = find_variant(c.dtype, c.head_dim, c.block_size);
  if (!v && !prefill_supported(c.dtype, c.head_dim, c.block_size)) return hipErrorInvalidValue;
  PrefillArgs a;
  a.q = (const u32x4*)query;
  a.kpool = (const u32x4*)c.k;
  a.vpool = (const u32x4*)c.v;
  a.tables = block_tables;
  a.cu_q = cu_q_lens;
  a.lens = context_lens;
  a.out = out;
  a.S = S;
  a.H = c.num_heads;
  a.N = c.num_blocks;
  a.max_blocks = max_blocks_per_seq;
  a.ntiles = (max_q_len + kTileQ - 1) / kTileQ;
  a.scale_log2 = scale * kLog2e;
  a.out_dtype = out_dtype;
  if (!v) {
    const int64_t grid = (int64_t)max_q_len * S * c.num_heads;
    void (*k)(PrefillArgs, int32_t, int32_t, int32_t) =
        c.dtype == PA_F32 ? prefill_generic_kernel<F32>
                          : (c.dtype == PA_F16 ? prefill_generic_kernel<F16> : prefill_generic_kernel<BF16>);
    hipLaunchKernelGGL(k, dim3((unsigned)grid), dim3(64), 0, stream, a, (int32_t)c.head_dim,
                       (int32_t)c.block_size, max_q_len);
    return hipGetLastError();
  }
  const int64_t grid = (int64_t)a.ntiles * S * c.num_heads;
  hipLaunchKernelGGL(v->kernel, dim3((unsigned)grid), dim3(kNW * 64), 0, stream, a);
  return hipGetLastError();
}

}  // namespace pa
