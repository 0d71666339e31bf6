// Device helpers for gfx950: 16-byte chunk arithmetic per element type,
// 16-lane row reductions with DPP, and output rounding.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/pagedattn.h"

namespace pa {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;

// s_waitcnt vmcnt(0) only: this wave's global loads (including those that
// write LDS directly) have completed
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x3f70); }
// 16 bytes per lane from global memory straight into LDS at lds_base + 16 *
// lane (global_load_lds_dwordx4; the LDS address is wave-uniform and comes
// from M0, which the "{m0}" operand makes the compiler set before the
// instruction, so it knows M0's value; one wait state follows the M0 write).
// Issued as inline assembly so the compiler does not hold every later LDS
// read back until these loads complete: the caller orders them (wait_vmem
// before this wave reads the data, plus a barrier before other waves do).
__device__ __forceinline__ void load_to_lds(const void* src, uint32_t lds_base) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "{m0}"(lds_base) : "memory");
}
// 4 bytes per lane into LDS at lds_base + 4 * lane (global_load_lds_dword).
__device__ __forceinline__ void load_dword_to_lds(const void* src, uint32_t lds_base) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dword %0, off" ::"v"(src), "{m0}"(lds_base) : "memory");
}
// A wave-uniform 32-bit value read through the scalar data cache (a load;
// the kernel that uses this never writes `p`).  The compiler picks scalar
// loads by itself only when it can prove that no store of the kernel reaches
// the address; kernels that also write the pools lose that proof, and their
// vector loads of such metadata queue behind the wave's streaming loads.
// Returns after the value has arrived.
__device__ __forceinline__ int32_t scalar_load(const int32_t* p) {
  int32_t v;
  asm volatile("s_load_dword %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(v) : "s"(p) : "memory");
  return v;
}
// Two such values in one round trip.
__device__ __forceinline__ void scalar_load2(const int32_t* p, const int32_t* q, int32_t& x, int32_t& y) {
  asm volatile("s_load_dword %0, %2, 0x0\n\ts_load_dword %1, %3, 0x0\n\ts_waitcnt lgkmcnt(0)"
               : "=&s"(x), "=&s"(y)
               : "s"(p), "s"(q)
               : "memory");
}
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(lds_void_t*)p;
}
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Storage element tags; the arithmetic is always fp32.
struct F32 { static constexpr int bytes = 4; static constexpr pa_dtype id = PA_F32; };
struct F16 { static constexpr int bytes = 2; static constexpr pa_dtype id = PA_F16; };
struct BF16 { static constexpr int bytes = 2; static constexpr pa_dtype id = PA_BF16; };

template <typename E>
struct Chunk {
  static constexpr int elems = 16 / E::bytes;  // elements in 16 bytes
};

// fp32 sum of the elementwise products of two 16-byte chunks.
__device__ __forceinline__ float dot_chunk(F32, const u32x4& a, const u32x4& b) {
  float acc = __uint_as_float(a.x) * __uint_as_float(b.x);
  acc = __builtin_fmaf(__uint_as_float(a.y), __uint_as_float(b.y), acc);
  acc = __builtin_fmaf(__uint_as_float(a.z), __uint_as_float(b.z), acc);
  acc = __builtin_fmaf(__uint_as_float(a.w), __uint_as_float(b.w), acc);
  return acc;
}
// Reinterpret one 32-bit word as two 16-bit floats.  The word is taken by
// value: a bit-cast applied directly to an ext_vector element (``v.y``) is
// compiled as a read of element 0 by this clang, so callers pass ``v.x`` etc.
// through these helpers instead.
__device__ __forceinline__ f16x2 as_f16x2(uint32_t u) { return __builtin_bit_cast(f16x2, u); }
__device__ __forceinline__ bf16x2 as_bf16x2(uint32_t u) { return __builtin_bit_cast(bf16x2, u); }

__device__ __forceinline__ float dot_chunk(F16, const u32x4& a, const u32x4& b) {
  // v_dot2_f32_f16: products of 16-bit floats are exact in fp32
  float acc = __builtin_amdgcn_fdot2(as_f16x2(a.x), as_f16x2(b.x), 0.f, false);
  acc = __builtin_amdgcn_fdot2(as_f16x2(a.y), as_f16x2(b.y), acc, false);
  acc = __builtin_amdgcn_fdot2(as_f16x2(a.z), as_f16x2(b.z), acc, false);
  acc = __builtin_amdgcn_fdot2(as_f16x2(a.w), as_f16x2(b.w), acc, false);
  return acc;
}
__device__ __forceinline__ float dot_chunk(BF16, const u32x4& a, const u32x4& b) {
  float acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(a.x), as_bf16x2(b.x), 0.f, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(a.y), as_bf16x2(b.y), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(a.z), as_bf16x2(b.z), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(a.w), as_bf16x2(b.w), acc, false);
  return acc;
}

// Widen the 16-byte chunk to fp32 elements (exact).
__device__ __forceinline__ void widen(F32, const u32x4& v, float* f) {
  f[0] = __uint_as_float(v.x); f[1] = __uint_as_float(v.y);
  f[2] = __uint_as_float(v.z); f[3] = __uint_as_float(v.w);
}
__device__ __forceinline__ void widen(F16, const u32x4& v, float* f) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const f16x2 h = as_f16x2(w[i]);
    f[2 * i] = (float)h.x;
    f[2 * i + 1] = (float)h.y;
  }
}
__device__ __forceinline__ void widen(BF16, const u32x4& v, float* f) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(w[i] << 16);
    f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}

// ---- DPP lane exchange -------------------------------------------------------
// Control codes of the GCN/CDNA DPP encoding.
constexpr int kDppQuadXor1 = 0xB1;       // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;       // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141; // lane i <-> 7-i within each 8
constexpr int kDppRowMirror = 0x140;     // lane i <-> 15-i within each 16

template <int Ctrl>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), Ctrl, 0xf, 0xf, false));
}

// Sum over each aligned group of N lanes (N a power of two <= 64); every lane
// of the group receives the same value (each step adds two operands in an
// order-independent way, so all lanes agree bit for bit).
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  if constexpr (N >= 2) x += dpp<kDppQuadXor1>(x);
  if constexpr (N >= 4) x += dpp<kDppQuadXor2>(x);
  if constexpr (N >= 8) x += dpp<kDppRowHalfMirror>(x);
  if constexpr (N >= 16) x += dpp<kDppRowMirror>(x);
  if constexpr (N >= 32) x += __shfl_xor(x, 16);
  if constexpr (N >= 64) x += __shfl_xor(x, 32);
  return x;
}

// ---- output rounding ---------------------------------------------------------
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu)) return (uint16_t)((u >> 16) | 0x40);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ void store_out(void* out, int64_t idx, float val, pa_dtype t) {
  if (t == PA_F32) {
    ((float*)out)[idx] = val;
  } else if (t == PA_F16) {
    ((_Float16*)out)[idx] = (_Float16)val;
  } else {
    ((uint16_t*)out)[idx] = f32_to_bf16_rne(val);
  }
}

}  // namespace pa
