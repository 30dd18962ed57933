// Device helpers shared by the gfx950 kernels: bf16 / fp8 widening, rounding, MFMA
// operand types and wave-level shuffles. CDNA4 wavefronts are 64 lanes wide.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace csl {

constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;   // MFMA A/B operand, 8 x bf16
typedef __attribute__((ext_vector_type(4))) float f32x4;      // 16x16 MFMA accumulator
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;

// bf16 bit patterns held in 32-bit words: low half = element 2i, high half = element 2i+1.
__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> bf16 bits, round to nearest even; NaN stays a quiet NaN, overflow goes to inf.
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}
// Two fp32 -> packed bf16 pair (lo in bits 0..15) with gfx950's conversion instruction,
// which rounds to nearest even like f32_to_bf16_bits.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __attribute__((ext_vector_type(2))) float f32x2_t;
  typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t{lo, hi}), bf16x2_t));
}

// Four OCP E4M3FN codes packed in a 32-bit word -> two words of bf16 pairs. gfx950's packed
// conversion decodes OCP E4M3FN (bias 7, no infinities, S.1111.111 = NaN) to fp32 exactly;
// every e4m3 value has at most 4 significant bits and an exponent inside bf16's range, so
// keeping the upper half of each fp32 is the exact bf16.
__device__ __forceinline__ u32x2 e4m3x4_to_bf16x4(uint32_t w) {
  const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);  // bytes 0 and 1
  const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);   // bytes 2 and 3
  u32x2 r;
  r.x = (__float_as_uint(lo[0]) >> 16) | (__float_as_uint(lo[1]) & 0xffff0000u);
  r.y = (__float_as_uint(hi[0]) >> 16) | (__float_as_uint(hi[1]) & 0xffff0000u);
  return r;
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// D = A * B + C for a 16x16 tile with K = 32 (gfx950). Per lane l (g = l / 16):
//   A: row l % 16, 8 consecutive k-slots 8g..8g+7; B: column l % 16, same k-slots;
//   C/D: column l % 16, rows 4g..4g+3 (element i of the f32x4 is row 4g+i).
// The k-slot order only has to agree between A and B.
__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float shfl_xor_f(float v, int mask) { return __shfl_xor(v, mask, kWave); }

// The pair (v, value of lane ^ MASK) in some order, MASK = 8, 16 or 32, without a trip through
// LDS: row_ror:8 (DPP) is xor 8 inside a 16-lane row; gfx950's permlane16_swap returns the
// (even row, odd row) pair of each two 16-lane rows and permlane32_swap the (lower, upper)
// half pair. Combined by a commutative operation, the two lanes of a pair get equal bits.
template <int MASK>
__device__ __forceinline__ float2 xor_pair(float v) {
  static_assert(MASK == 8 || MASK == 16 || MASK == 32, "lane distances served by DPP and row swaps");
  if constexpr (MASK == 32) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return make_float2(__uint_as_float(r[0]), __uint_as_float(r[1]));
  } else if constexpr (MASK == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return make_float2(__uint_as_float(r[0]), __uint_as_float(r[1]));
  } else {
    return make_float2(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x128, 0xf, 0xf, false)));
  }
}
template <int MASK>
__device__ __forceinline__ float xor_sum(float v) {
  const float2 p = xor_pair<MASK>(v);
  return p.x + p.y;
}
template <int MASK>
__device__ __forceinline__ float xor_max(float v) {
  const float2 p = xor_pair<MASK>(v);
  return fmaxf(p.x, p.y);
}

// Immediate of s_waitcnt in the gfx9 family's encoding (gfx950 included): vmcnt in bits 3:0
// and 15:14, expcnt in bits 6:4, lgkmcnt in bits 11:8; a field at its maximum does not wait.
// waitcnt_vm(n): wait until at most n vector memory operations of this wave are outstanding.
constexpr int waitcnt_vm(int n) { return (n & 0xf) | (((n >> 4) & 0x3) << 14) | (0x7 << 4) | (0xf << 8); }
static_assert(waitcnt_vm(0) == 0x0f70 && waitcnt_vm(63) == 0xcf7f, "gfx9 s_waitcnt field layout");

// Order-preserving map of an fp32 score to an unsigned key (larger score -> larger key);
// -0.0 is folded onto +0.0 first so that the two compare equal.
__device__ __forceinline__ uint32_t score_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

}  // namespace csl
