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
//   queries 32w..32w+31.  Key/value tiles of 64 tokens are gathered from their
//   physical blocks (16-byte loads) into LDS: keys as [token][d] rows, values
//   transposed to [d][token] rows (registers do the 4x8 transpose with
//   v_perm_b32), both row-padded, and the value rows' key units XOR-swizzled,
//   so neither the tile writes nor the MFMA operand reads conflict on LDS
//   banks.
// * Scores are formed transposed, S^T = K Q^T, with
//   v_mfma_f32_32x32x16_{bf16,f16}: the result layout puts one query per lane
//   column, so the online softmax of a query is in-lane except for one
//   exchange between the two half-waves.
// * O^T += V^T P^T with the same MFMA: the B operand P^T for a 16-key step is
//   exactly 8 of the lane's own score registers (rounded to 16 bits), so P
//   never leaves the registers; the A operand is two 8-byte LDS reads of V^T.
// * Tiles entirely above the diagonal are never loaded; the diagonal ones are
//   masked per element.  Workgroups are issued heaviest-first (last query tile
//   first).
// * Pipeline: LDS holds two key/value tiles.  After tile j is computed from
//   one buffer, tile j+1 (loaded into registers during tile j-1) is written to
//   the other and the global loads of tile j+2 are issued; the block-table
//   entry of tile j+2 is read before tile j's compute, so no load waits on a
//   table read.  One barrier per tile, ordering LDS only.
#include <type_traits>

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

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
// releases global memory, which makes every wave wait for its in-flight global
// loads (the next tiles) at each barrier; the tiles need only LDS ordering.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

constexpr int kD = 128;        // head_dim
constexpr int kBN = 64;        // keys per tile
constexpr int kXcds = 8;       // accelerator complex dies of an MI355X
constexpr int kKRow = kD + 8;  // padded LDS row of a key (elements)
constexpr int kVRow = kBN + 4; // padded LDS row of a transposed value (elements)
constexpr float kNegBig = -1e30f;
constexpr float kRescaleLog2 = 8.0f;

// V^T rows hold 64 keys as 16 units of four; dimension block dm (rows
// 32dm .. 32dm+31) stores key unit u at position u ^ 4dm.  The transposing
// tile writes (rows 8 apart across lanes) then spread over all 64 banks
// (two lanes per bank, the minimum for 8-byte writes) instead of a quarter of
// them, and an operand read's two halves stay 16 bytes apart.
__device__ __forceinline__ int vt_unit(const int u, const int dm) { return u ^ (4 * dm); }
constexpr float kLog2e = 1.44269504088896340736f;

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
  int32_t S, H, N, max_blocks, ntiles;  // ntiles = ceil(max_q_len / kBM)
  float scale_log2;
  pa_dtype out_dtype;
};

// One workgroup = NW waves; a wave owns QB blocks of 32 queries.  With QB = 2
// every key/value operand read from LDS feeds two MFMAs, and the exponentials
// of one query block overlap the MFMAs of the other.
template <typename E, int BS, int NW, int QB>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(QB == 2 || NW == 8 ? 1 : 2))) void prefill_kernel(
    PrefillArgs a) {
  constexpr int kBM = NW * QB * 32;  // queries per workgroup
  constexpr int KPT = 16 / NW;       // keys per thread in a tile load (16-byte chunk dc of each)
  static_assert(KPT == 2 || KPT % 4 == 0, "tile loads take 2 or a multiple of 4 keys per thread");
  static_assert(BS >= KPT && (kBN % BS == 0 || BS % kBN == 0), "block size must tile the 64-key step");
  __shared__ __attribute__((aligned(16))) uint16_t lds_k[2][kBN * kKRow];
  __shared__ __attribute__((aligned(16))) uint16_t lds_vt[2][kD * kVRow];

  // XCD-aware order: workgroups are handed to the 8 XCDs round-robin, so
  // XCD x runs blocks x, x+8, ...; give each XCD a contiguous range of
  // (sequence, head) pairs with all their query tiles (heaviest first), so the
  // key/value tiles every query tile of a pair re-reads stay in that XCD's L2.
  const int total = a.ntiles * a.S * a.H;
  const int xcd = blockIdx.x % kXcds;
  const int q8 = total / kXcds, r8 = total % kXcds;
  const int lin = xcd * q8 + min(xcd, r8) + (int)(blockIdx.x / kXcds);
  const int pair = lin / a.ntiles;
  const int tile = a.ntiles - 1 - lin % a.ntiles;
  const int s = pair / a.H;
  const int h = pair % a.H;
  const int q_begin = a.cu_q[s];
  const int qlen = a.cu_q[s + 1] - q_begin;
  const int ctx = a.lens[s];
  const int q0 = tile * kBM;  // first query row of this workgroup (within the sequence)
  if (q0 >= qlen || qlen > ctx) return;
  const int pos0 = ctx - qlen;  // logical position of query row 0

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int g = lane >> 5;     // half-wave
  const int col = lane & 31;   // this lane's query column within a block
  int qrow[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) qrow[qb] = q0 + 32 * (QB * w + qb) + col;

  // B operands of S^T = K Q^T: Q[query][16ks + 8g .. +8] for k-steps ks = 0..7
  u32x4 qop[QB][8];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const bool valid = qrow[qb] < qlen;
    const int64_t qbase = ((int64_t)(q_begin + (valid ? qrow[qb] : 0)) * a.H + h) * (kD / 8);
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) qop[qb][ks] = valid ? a.q[qbase + 2 * ks + g] : u32x4{0, 0, 0, 0};
  }

  f32x16 acc_o[QB][4];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int dm = 0; dm < 4; ++dm)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc_o[qb][dm][i] = 0.f;
  float m[QB], l[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m[qb] = kNegBig;
    l[qb] = 0.f;
  }

  // keys needed by the workgroup: positions 0 .. pos0 + min(q0 + kBM, qlen) - 1
  const int last_pos = pos0 + min(q0 + kBM, qlen) - 1;
  const int nkt = last_pos / kBN + 1;

  // cooperative tile load: thread -> keys KPT*kg .. +KPT-1, dims 8*dc .. 8*dc+7
  const int kg = tid >> 4;
  const int dc = tid & 15;
  const int64_t trow = (int64_t)s * a.max_blocks;

  // tiles whose keys all precede every query of the workgroup need no mask
  const int n_full = min(nkt, (pos0 + q0 + 1) / kBN);
  const int wave_max_pos = pos0 + min(q0 + 32 * QB * w + 32 * QB - 1, qlen - 1);  // last query of this wave
  const float c = a.scale_log2;
  // Lazy rescale: the running max used for the weights is only raised (and
  // the accumulators rescaled) when some query's max grows by more than
  // kRescaleLog2 in log2 units.  Weights are then at most 2^kRescaleLog2,
  // and numerator and denominator share the same reference, so the result is
  // unchanged up to rounding; after the first tiles the rescale is rare.
  const float slack = kRescaleLog2 / c;  // in raw score units (c > 0)

  // Softmax of one query block's scores: mask, new running max, rescale.
  // Returns the per-lane max (raw units) in m_new.
  auto block_max = [&](f32x16* acc_s, const int j0, const int qb, auto masked_tag) -> float {
    constexpr bool MASKED = decltype(masked_tag)::value;
    const int qpos = pos0 + qrow[qb];
    float mt = kNegBig;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        if constexpr (MASKED) {
          const int kpos = j0 + 32 * mb + 8 * (i / 4) + 4 * g + (i % 4);
          if (kpos > qpos) acc_s[mb][i] = -__builtin_inff();
        }
        mt = fmaxf(mt, acc_s[mb][i]);
      }
    return fmaxf(m[qb], halves_max(mt));  // raw units (scale > 0 keeps the order)
  };
  auto rescale = [&](const int qb, const float m_new) {
    const float alpha = __builtin_amdgcn_exp2f((m[qb] - m_new) * c);
    l[qb] *= alpha;
#pragma unroll
    for (int dm = 0; dm < 4; ++dm)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc_o[qb][dm][i] *= alpha;
    m[qb] = m_new;
  };
  // P^T operands: k-step (mb, t) takes result elements 8t .. 8t+7 of block mb;
  // the denominator sums the same rounded weights the MFMA multiplies
  auto weights = [&](const f32x16* acc_s, const int qb, u32x4 (*pb)[2]) {
    const float mc = -m[qb] * c;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        float p[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) p[j] = __builtin_amdgcn_exp2f(__builtin_fmaf(acc_s[mb][8 * t + j], c, mc));
        pb[mb][t] = u32x4{pack2(E{}, p[0], p[1]), pack2(E{}, p[2], p[3]), pack2(E{}, p[4], p[5]),
                          pack2(E{}, p[6], p[7])};
        l[qb] = sum_unpacked(E{}, pb[mb][t], l[qb]);
      }
  };

  // One key tile: S^T = K Q^T, online softmax, O^T += V^T P^T.  MASKED tiles
  // straddle the diagonal; scores of keys after the query become -inf.
  auto compute_tile = [&](const int j0, const uint16_t* __restrict__ tk, const uint16_t* __restrict__ tvt,
                          auto masked_tag) {
    f32x16 acc_s[QB][2];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc_s[qb][mb][i] = 0.f;
    u32x4 pb[QB][2][2];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      // key operands are re-read per query block (holding all sixteen would
      // not fit beside two blocks' accumulators)
#pragma unroll
      for (int ks = 0; ks < 8; ++ks)
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
          const u32x4 ka = *(const u32x4*)&tk[(32 * mb + col) * kKRow + 16 * ks + 8 * g];
          acc_s[qb][mb] = mfma32(E{}, ka, qop[qb][ks], acc_s[qb][mb]);
        }
      // the previous block's weights overlap this block's MFMAs
      if (qb > 0) weights(acc_s[qb - 1], qb - 1, pb[qb - 1]);
      const float m_new = block_max(acc_s[qb], j0, qb, masked_tag);
      if (__any(m_new > m[qb] + slack)) rescale(qb, m_new);
    }
    weights(acc_s[QB - 1], QB - 1, pb[QB - 1]);
    // O^T += V^T P^T; k-slot (g, j) of step (mb, t) is key 32mb + 16t + 8(j/4) + 4g + j%4
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int dm = 0; dm < 4; ++dm) {
          const uint16_t* vrow = &tvt[(32 * dm + col) * kVRow + 4 * vt_unit(8 * mb + 4 * t + g, dm)];
          const u32x2 v0 = *(const u32x2*)vrow;
          const u32x2 v1 = *(const u32x2*)(vrow + 8);
          const u32x4 va = {v0.x, v0.y, v1.x, v1.y};
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) acc_o[qb][dm] = mfma32(E{}, va, pb[qb][mb][t], acc_o[qb][dm]);
        }
  };

  // Physical block of this thread's keys in key tile kt.  The read is
  // unconditional (index clamped into the table row) so the compiler keeps
  // no predicated definition of it alive across the loop; load_tile ignores
  // the entry for keys at or past the context length.
  auto table_entry = [&](const int kt) -> int {
    const int blk = min((kt * kBN + KPT * kg) / BS, a.max_blocks - 1);
    return a.tables[trow + blk];
  };
  // Global -> register loads of one key tile (thread: KPT keys x 8 dims of K and V)
  auto load_tile = [&](const int kt, const int phys, u32x4* kr, u32x4* vr) {
    const int jk = kt * kBN + KPT * kg;  // first of this thread's keys (one block: BS >= KPT)
    const bool ok = phys >= 0 && phys < a.N;
    const int off = jk % BS;
    const int64_t base = (((int64_t)(ok ? phys : 0) * a.H + h) * BS + off) * (kD / 8) + dc;
#pragma unroll
    for (int u = 0; u < KPT; ++u) {
      const bool valid = ok && (jk + u < ctx);
      kr[u] = valid ? a.kpool[base + u * (kD / 8)] : u32x4{0, 0, 0, 0};
      vr[u] = valid ? a.vpool[base + u * (kD / 8)] : u32x4{0, 0, 0, 0};
    }
  };
  // Registers -> one LDS buffer: K rows as they are, V transposed (4 keys x 8
  // dims -> 8 rows of V^T, per group of four keys)
  auto store_tile = [&](const int buf, const u32x4* kr, const u32x4* vr) {
#pragma unroll
    for (int u = 0; u < KPT; ++u) *(u32x4*)&lds_k[buf][(KPT * kg + u) * kKRow + 8 * dc] = kr[u];
    if constexpr (KPT == 2) {  // two keys x 8 dims -> 8 rows of V^T, 4 bytes each
      const uint32_t w0[4] = {vr[0].x, vr[0].y, vr[0].z, vr[0].w};
      const uint32_t w1[4] = {vr[1].x, vr[1].y, vr[1].z, vr[1].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int e = 4 * vt_unit(kg >> 1, dc >> 2) + 2 * (kg & 1);  // rows 8dc.. lie in dim block dc / 4
        *(uint32_t*)&lds_vt[buf][(8 * dc + 2 * i) * kVRow + e] = __builtin_amdgcn_perm(w1[i], w0[i], 0x05040100u);
        *(uint32_t*)&lds_vt[buf][(8 * dc + 2 * i + 1) * kVRow + e] = __builtin_amdgcn_perm(w1[i], w0[i], 0x07060302u);
      }
    }
#pragma unroll
    for (int q4 = 0; q4 < KPT / 4; ++q4) {
      const u32x4* v4 = vr + 4 * q4;
      const uint32_t w0[4] = {v4[0].x, v4[0].y, v4[0].z, v4[0].w};
      const uint32_t w1[4] = {v4[1].x, v4[1].y, v4[1].z, v4[1].w};
      const uint32_t w2[4] = {v4[2].x, v4[2].y, v4[2].z, v4[2].w};
      const uint32_t w3[4] = {v4[3].x, v4[3].y, v4[3].z, v4[3].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        u32x2 lo, hi;  // dims 8dc+2i (low halves) and 8dc+2i+1 (high halves)
        lo.x = __builtin_amdgcn_perm(w1[i], w0[i], 0x05040100u);
        lo.y = __builtin_amdgcn_perm(w3[i], w2[i], 0x05040100u);
        hi.x = __builtin_amdgcn_perm(w1[i], w0[i], 0x07060302u);
        hi.y = __builtin_amdgcn_perm(w3[i], w2[i], 0x07060302u);
        const int e = 4 * vt_unit(KPT / 4 * kg + q4, dc >> 2);
        *(u32x2*)&lds_vt[buf][(8 * dc + 2 * i) * kVRow + e] = lo;
        *(u32x2*)&lds_vt[buf][(8 * dc + 2 * i + 1) * kVRow + e] = hi;
      }
    }
  };

  // prologue: tile 0 in LDS buffer 0, tile 1 in flight
  u32x4 kr[KPT], vr[KPT];
  load_tile(0, table_entry(0), kr, vr);
  const int phys1 = table_entry(1);
  store_tile(0, kr, vr);
  if (nkt > 1) load_tile(1, phys1, kr, vr);
  lds_barrier();
  // After tile kt: write tile kt + 1 into the other buffer (last read during
  // tile kt - 1, before the previous barrier), start the loads of tile kt + 2.
  auto advance = [&](const int kt, const int phys2) {
    if (kt + 1 < nkt) {
      store_tile((kt & 1) ^ 1, kr, vr);
      if (kt + 2 < nkt) load_tile(kt + 2, phys2, kr, vr);
    }
    lds_barrier();
  };
  // Two loops, so each has one compute path and the accumulators stay in
  // place (a join of two inlined paths makes the compiler copy them).
  int kt = 0;
  for (; kt < n_full; ++kt) {
    const int phys2 = table_entry(kt + 2);  // issued before the compute, used after it
    compute_tile(kt * kBN, lds_k[kt & 1], lds_vt[kt & 1], std::false_type{});
    advance(kt, phys2);
  }
  for (; kt < nkt; ++kt) {
    const int phys2 = table_entry(kt + 2);
    const int j0 = kt * kBN;
    if (j0 <= wave_max_pos)  // a wave skips tiles wholly after its queries
      compute_tile(j0, lds_k[kt & 1], lds_vt[kt & 1], std::true_type{});
    advance(kt, phys2);
  }

  // normalise and store: result element i of block dm is dim 32dm + 8(i/4) + 4g + i%4
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float lsum = halves_sum(l[qb]);
    if (qrow[qb] >= qlen) continue;
    const float inv_l = 1.f / lsum;
    const int64_t obase = ((int64_t)(q_begin + qrow[qb]) * a.H + h) * kD;
#pragma unroll
    for (int dm = 0; dm < 4; ++dm)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int d = 32 * dm + 8 * r4 + 4 * g;
        const float o0 = acc_o[qb][dm][4 * r4] * inv_l, o1 = acc_o[qb][dm][4 * r4 + 1] * inv_l;
        const float o2 = acc_o[qb][dm][4 * r4 + 2] * inv_l, o3 = acc_o[qb][dm][4 * r4 + 3] * inv_l;
        if (a.out_dtype == PA_F32) {
          float4 v = {o0, o1, o2, o3};
          *(float4*)((float*)a.out + obase + d) = v;
        } else if (a.out_dtype == E::id) {
          u32x2 v = {pack2(E{}, o0, o1), pack2(E{}, o2, o3)};
          *(u32x2*)((uint16_t*)a.out + obase + d) = v;
        }
      }
  }
}

#ifndef PA_PREFILL_NW
#define PA_PREFILL_NW 4  // waves per workgroup
#endif
#ifndef PA_PREFILL_QB
#define PA_PREFILL_QB 1  // 32-query blocks per wave
#endif
constexpr int kNW = PA_PREFILL_NW;
constexpr int kQB = PA_PREFILL_QB;
constexpr int kTileQ = kNW * kQB * 32;  // queries per workgroup

struct Variant {
  pa_dtype dtype;
  int BS;
  void (*kernel)(PrefillArgs);
};

#define PA_PREFILL_VARIANTS(BS)                                    \
  Variant{PA_BF16, BS, prefill_kernel<BF16, BS, kNW, kQB>}, Variant { \
    PA_F16, BS, prefill_kernel<F16, BS, kNW, kQB>                     \
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
  return find_variant(dtype, head_dim, block_size) != nullptr;
}

hipError_t launch_paged_prefill(const Cache& c, void* out, pa_dtype out_dtype, const void* query,
                                const int32_t* block_tables, int32_t max_blocks_per_seq,
                                const int32_t* cu_q_lens, const int32_t* context_lens, int32_t S,
                                int32_t max_q_len, int32_t max_context_len, float scale,
                                hipStream_t stream) {
  (void)max_context_len;
  const Variant* v = find_variant(c.dtype, c.head_dim, c.block_size);
  if (!v) return hipErrorInvalidValue;
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
  const int64_t grid = (int64_t)a.ntiles * S * c.num_heads;
  hipLaunchKernelGGL(v->kernel, dim3((unsigned)grid), dim3(kNW * 64), 0, stream, a);
  return hipGetLastError();
}

}  // namespace pa
