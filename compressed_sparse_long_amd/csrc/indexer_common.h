// The decode indexer's per-key arithmetic, shared by the indexer kernels and by the top-k
// finishing step, which recomputes a row's scores when that row's candidate lists cannot prove
// its selection and the indexer left no scores behind: key formats, their widening to the
// MFMA operand, and one 16-key tile's scores. Every caller runs the same instructions in the
// same order, so the scores agree bit for bit.
#pragma once

#include "device_common.h"
#include "launch.h"

namespace csl {

namespace {

enum { kKeyBF16 = 0, kKeyFP8 = 1, kKeyFP4 = 2 };

// Row of entry s of sequence b in the key array: e_base + s, or in the paged layout its pool
// row (table entries past the table are clamped: such entries are never loaded)
template <bool PAGED>
__device__ __forceinline__ int64_t key_row(const PagedView& pg, int b, int64_t e_base, int64_t s) {
  if (!PAGED) return e_base + s;
  int64_t j = s >> pg.eb_shift;
  j = j < pg.max_blocks ? j : pg.max_blocks - 1;
  return ((int64_t)pg.table[(int64_t)b * pg.max_blocks + j] << pg.eb_shift) | (s & ((1 << pg.eb_shift) - 1));
}

// Slot of the fp8 group scale of entry s of sequence b: scale_off[b] + s / scale_group, or in the
// paged layout the pool scale of its key row kr, kr >> scale_shift (the pool keeps its scales
// per block: one per power-of-two group inside a block, or one per block when a group spans
// several blocks)
template <bool PAGED>
__device__ __forceinline__ int64_t fp8_scale_index(const PagedView& pg, int64_t kr, const int64_t* scale_off, int b,
                                                   int64_t s, int scale_group) {
  if (PAGED) return kr >> pg.scale_shift;
  return scale_off[b] + s / scale_group;
}

// first dim of the 8 k-slots that lane group g supplies for MFMA kk (the key and query
// operands share this order)
template <int KT>
__device__ __forceinline__ int kslot_dim(int kk, int g) {
  return KT == kKeyFP4 ? g * 16 + kk * 8 : kk * 32 + g * 8;
}

// One lane's share of a key row for both MFMAs (raw codes; key_operand widens them).
// MXFP4: 8 bytes = dims 16g..16g+15 (block g / 2) plus that block's E8M0 scale byte.
template <int KT>
__device__ __forceinline__ void load_key_tile(const void* __restrict__ kI, const uint8_t* __restrict__ k_mx,
                                              int64_t row, bool ok, int g, u32x4& k0, u32x4& k1) {
  if (!ok) {
    k0 = u32x4{0, 0, 0, 0};
    k1 = u32x4{0, 0, 0, 0};
    return;
  }
  if (KT == kKeyBF16) {
    const uint16_t* p = static_cast<const uint16_t*>(kI) + row * 64 + g * 8;
    k0 = *reinterpret_cast<const u32x4*>(p);
    k1 = *reinterpret_cast<const u32x4*>(p + 32);
  } else if (KT == kKeyFP8) {
    const uint8_t* p = static_cast<const uint8_t*>(kI) + row * 64 + g * 8;
    const u32x2 c0 = *reinterpret_cast<const u32x2*>(p);
    const u32x2 c1 = *reinterpret_cast<const u32x2*>(p + 32);
    // keep the raw codes; they are widened to bf16 just before the MFMA
    k0 = u32x4{c0.x, c0.y, 0, 0};
    k1 = u32x4{c1.x, c1.y, 0, 0};
  } else {
    const u32x2 c = *reinterpret_cast<const u32x2*>(static_cast<const uint8_t*>(kI) + row * 32 + g * 8);
    const uint32_t e = k_mx[row * 2 + (g >> 1)];
    k0 = u32x4{c.x, e, 0, 0};
    k1 = u32x4{c.y, e, 0, 0};
  }
}

template <int KT>
__device__ __forceinline__ bf16x8 key_operand(const u32x4& k) {
  if (KT == kKeyBF16) return as_bf16x8(k);
  if (KT == kKeyFP8) {
    const u32x2 lo = e4m3x4_to_bf16x4(k.x);
    const u32x2 hi = e4m3x4_to_bf16x4(k.y);
    return as_bf16x8(u32x4{lo.x, lo.y, hi.x, hi.y});
  }
  // 8 E2M1 codes (byte j: dims 2j, 2j + 1 in its low and high nibble) times 2^(e - 127),
  // exact in bf16; a zero exponent byte gives the float 2^-127 (subnormal)
  const float sc = k.y ? __uint_as_float(k.y << 23) : __uint_as_float(0x00400000u);
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t r0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(k.x, sc, 0);
  const bf16x2_t r1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(k.x, sc, 1);
  const bf16x2_t r2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(k.x, sc, 2);
  const bf16x2_t r3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(k.x, sc, 3);
  return as_bf16x8(u32x4{__builtin_bit_cast(uint32_t, r0), __builtin_bit_cast(uint32_t, r1),
                         __builtin_bit_cast(uint32_t, r2), __builtin_bit_cast(uint32_t, r3)});
}

// Sum over the HI consecutive lanes that hold one query row's heads (HI a power of two up to
// 16, groups aligned inside a row of 16 lanes): xor-1 and xor-2 quad permutes, then the
// half-row and row mirrors, all DPP, so every lane of the group ends with the group sum.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}
template <int HI>
__device__ __forceinline__ float head_sum(float v) {
  if (HI >= 2) v += dpp_f<0xb1>(v);   // quad_perm [1,0,3,2]
  if (HI >= 4) v += dpp_f<0x4e>(v);   // quad_perm [2,3,0,1]
  if (HI >= 8) v += dpp_f<0x141>(v);  // row_half_mirror
  if (HI >= 16) v += dpp_f<0x140>(v); // row_mirror
  return v;
}

// Decode tiling, one tile: keys (the A operand, lane (g, c) holding k-slots of key c of the
// tile) against the query rows x heads of the B operand; lane (g, c) gets the head-weighted
// ReLU sum over the HI heads of its query row for keys 4g .. 4g + 3 of the tile.
template <int HI, int KT>
__device__ __forceinline__ void decode_score_tile(const u32x4& k0, const u32x4& k1, const bf16x8 (&qb)[2], float wc,
                                                  float (&v)[4]) {
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  acc = mfma16x16x32(key_operand<KT>(k0), qb[0], acc);
  acc = mfma16x16x32(key_operand<KT>(k1), qb[1], acc);
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = head_sum<HI>(wc * fmaxf(acc[i], 0.f));
}

}  // namespace

}  // namespace csl
