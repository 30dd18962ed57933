// indexer_scores: Lightning-indexer scores I(t,s) = sum_j w_j * ReLU(q_j . k_s).
//
// The score of every visible compressed indexer key is a dense contraction
// ([P5] indexer score formula; [P2] "Deep Dive", CSA Lightning Indexer): per query row,
// [HI heads x CI] x [CI x n keys], followed by ReLU, the head weights and a sum over heads.
// It runs on the gfx950 matrix cores as 16x16x32 bf16 MFMA tiles of 16/HI query rows x HI
// heads against 16 consecutive keys of one sequence (streamed from HBM), dot products in fp32.
// ReLU, the head weights, the optional fp8 group scale and the head sum run on the
// accumulator registers, so each key costs 128 bytes of reads (64 for fp8, 34 for MXFP4)
// and 4 bytes of score write per query row.
//
// Key formats: bf16; fp8 e4m3 codes with an fp32 scale per group of entries (widened to
// bf16 in registers, the scale applied to the score); MXFP4 ([P1] section 4.2 and [P2]
// "Where It Breaks": an FP4 indexer), E2M1 codes with an E8M0 scale per 32 dims, widened
// and scaled to bf16 exactly by gfx950's scaled fp4 conversion. For MXFP4 a lane holds 16
// consecutive dims of a key (one scale block) and the query operand takes the same
// k-slot order, which only has to agree between the two operands.
//
// Two tilings:
//   decode  (indexer_decode_kernel): 8 waves per workgroup, each with one pass over its own
//           64 consecutive keys (a single pass per wave keeps the memory pipeline full). The
//           keys are the MFMA A operand and the query rows x heads the B operand, so the head
//           sum is a DPP reduction inside a row of 16 lanes and the scores leave through LDS as
//           coalesced 256-byte stores. With a top-k workspace (single query row per sequence,
//           long rows) each workgroup also leaves its 512-entry slice's top-k candidate list
//           (topk_common.h), so the selection never re-reads the scores.
//   prefill (indexer_kernel, many query rows): each wave holds 8 A tiles of queries
//           (16/HI * 8 query rows) and the 4 waves walk the same key range, so a key tile
//           fetched once is reused for 64/HI * 8 query rows through L1/L2.
#include "compress_common.h"
#include "device_common.h"
#include "launch.h"
#include "topk_common.h"

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

template <int HI, int NB, int NWAVES, int WQ, int U, int KT, bool PAGED>
__global__ __launch_bounds__(NWAVES * 64) void indexer_kernel(
    const uint16_t* __restrict__ qI, const float* __restrict__ w, const void* __restrict__ kI,
    const void* __restrict__ k_scale_v, const int64_t* __restrict__ scale_off, int scale_group,
    const int64_t* __restrict__ ent_off, const int64_t* __restrict__ q_pos, int m, int T,
    int64_t max_entries, float* __restrict__ scores, int64_t ld, int epw, PagedView pg) {
  constexpr int QPB = 16 / HI;       // query rows per A tile
  constexpr int QPW = NB * QPB;      // query rows per wave
  constexpr int WE = NWAVES / WQ;    // key sub-ranges per block
  constexpr int ROWS_PER_GROUP = (HI >= 4) ? 1 : 4 / HI;  // query rows in one lane group's 4 C rows

  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  const int g = lane / 16;
  const int c = lane % 16;
  const int wq = wave % WQ;
  const int we = wave / WQ;
  const int b = blockIdx.z;

  const int t0 = (blockIdx.y * WQ + wq) * QPW;
  if (t0 >= T) return;
  constexpr bool FP8 = KT == kKeyFP8;
  const float* k_scale = static_cast<const float*>(k_scale_v);          // fp8: per entry group
  const uint8_t* k_mx = static_cast<const uint8_t*>(k_scale_v);         // MXFP4: E8M0 per block

  const int64_t e_base = ent_off[b];
  const int64_t n_ent = ent_off[b + 1] - e_base;
  const int64_t p0 = q_pos[b];
  // visible entries of query row t (masks the score writes only: the key loads below depend
  // on nothing but the sequence's entry range, so they leave without waiting for this)
  auto n_vis = [&](int t) -> int64_t {
    const int64_t p = p0 + t;
    int64_t nv = (p >= 0 && p < ((int64_t)1 << 32)) ? (int64_t)((uint32_t)p / (uint32_t)m) : p / m;
    nv = nv < n_ent ? nv : n_ent;
    nv = nv < max_entries ? nv : max_entries;
    return nv < 0 ? 0 : nv;
  };
  const int64_t wg_e0 = (int64_t)blockIdx.x * epw * WE;
  const int64_t e0 = wg_e0 + (int64_t)we * epw;
  const int64_t n_load = n_ent < max_entries ? n_ent : max_entries;
  const int64_t e_end = min(e0 + epw, n_load);
  if (e0 >= e_end) return;

  // A operands (queries) and the head weights this lane needs in the epilogue
  bf16x8 a[NB][2];
  float wv[NB][4];
  int64_t nv_row[NB][ROWS_PER_GROUP];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int tq = nb * QPB + c / HI;
    const int t = t0 + tq;
    const int j = c % HI;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      u32x4 v = u32x4{0, 0, 0, 0};
      if (t < T) v = *reinterpret_cast<const u32x4*>(qI + (((int64_t)b * T + t) * HI + j) * 64 + kslot_dim<KT>(kk, g));
      a[nb][kk] = as_bf16x8(v);
    }
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int r = 4 * g + it;
      const int tt = t0 + nb * QPB + r / HI;
      wv[nb][it] = (tt < T) ? w[((int64_t)b * T + tt) * HI + (r % HI)] : 0.f;
    }
#pragma unroll
    for (int q = 0; q < ROWS_PER_GROUP; ++q) {
      // query row written by this lane group (row index inside the A tile)
      const int rq = (HI >= 8) ? (4 * g) / HI : (4 * g) / HI + q;
      const int tt = t0 + nb * QPB + rq;
      nv_row[nb][q] = (tt < T) ? n_vis(tt) : 0;
    }
  }

  for (int64_t s0 = e0; s0 < e_end; s0 += 16 * U) {  // empty when this wave has no keys
    u32x4 kb[U][2];
    float sc[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t s = s0 + u * 16 + c;
      const bool ok = s < e_end;
      load_key_tile<KT>(kI, k_mx, key_row<PAGED>(pg, b, e_base, s), ok, g, kb[u][0], kb[u][1]);
      if (FP8) sc[u] = ok ? k_scale[scale_off[b] + s / scale_group] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t s = s0 + u * 16 + c;
      if (s0 + u * 16 >= e_end) break;
      const bf16x8 b0 = key_operand<KT>(kb[u][0]);
      const bf16x8 b1 = key_operand<KT>(kb[u][1]);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        acc = mfma16x16x32(a[nb][0], b0, acc);
        acc = mfma16x16x32(a[nb][1], b1, acc);
        float part[ROWS_PER_GROUP];
#pragma unroll
        for (int q = 0; q < ROWS_PER_GROUP; ++q) part[q] = 0.f;
#pragma unroll
        for (int it = 0; it < 4; ++it) {
          const int q = (HI >= 4) ? 0 : it / HI;
          part[q] = fmaf(wv[nb][it], fmaxf(acc[it], 0.f), part[q]);
        }
        if (HI == 16) {
          part[0] += shfl_xor_f(part[0], 16);
          part[0] += shfl_xor_f(part[0], 32);
        } else if (HI == 8) {
          part[0] += shfl_xor_f(part[0], 16);
        }
        const bool writer = (HI == 16) ? (g == 0) : (HI == 8) ? ((g & 1) == 0) : true;
        if (writer) {
#pragma unroll
          for (int q = 0; q < ROWS_PER_GROUP; ++q) {
            const int rq = (HI >= 8) ? (4 * g) / HI : (4 * g) / HI + q;
            const int tt = t0 + nb * QPB + rq;
            if (tt < T && s < nv_row[nb][q]) {
              float v = part[q];
              if (FP8) v *= sc[u];
              scores[((int64_t)b * T + tt) * ld + s] = v;
            }
          }
        }
      }
    }
  }
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

// Decode tiling: 8 waves, each with one pass over its own 64 consecutive keys (4 tiles of 16).
// The keys are the MFMA A operand and the 16/HI query rows x HI heads the B operand, so the
// accumulator holds 4 keys x 1 (row, head) per lane and the head sum stays inside a row of 16
// lanes (DPP). The scores go through LDS and leave as one coalesced 256-byte store per wave
// and query row; with a top-k workspace (T == 1) every thread then holds the key of one entry
// of the block's 512-entry slice for the candidate lists. Workgroups past the key range
// (blockIdx.x >= key_blocks, first query tile) run a CompressJob instead: 4 row-splits x 16
// lanes per entry, one row per thread (two for the overlapped pair), so the job adds no
// registers to the streaming path.
constexpr int kJobRS = 4;
constexpr int kJobEntriesPerBlock = kSlice / (16 * kJobRS);

template <int HI, int KT, bool PREP, bool PAGED>
__global__ __launch_bounds__(kSlice) void indexer_decode_kernel(
    const uint16_t* __restrict__ qI, const float* __restrict__ w, const void* __restrict__ kI,
    const void* __restrict__ k_scale_v, const int64_t* __restrict__ scale_off, int scale_group,
    const int64_t* __restrict__ ent_off, const int64_t* __restrict__ q_pos, int m, int T,
    int64_t max_entries, float* __restrict__ scores, int64_t ld, void* topk_ws, int topk_k, int slot_budget,
    int key_blocks, CompressJob job, PagedView pg) {
  constexpr int NW = kSlice / kWave;
  constexpr int QPB = 16 / HI;  // query rows per tile
  constexpr int U = 4;
  constexpr int EPW = 16 * U;   // keys per wave: one per lane on the way out
  constexpr int EPB = EPW * NW; // keys per block
  static_assert(EPW == kWave && EPB == kSlice, "one key per thread, one slice per block");
  __shared__ __align__(16) float sval[QPB][EPB];
  __shared__ SliceScratch sc;

  // paged: workgroups walk the sequences fastest, so consecutive workgroups take the same slice
  // of every sequence and the key reads in flight together spread over all sequences' blocks
  // (blocks handed out round-robin would otherwise be read at a stride of B blocks); the
  // packed layout keeps the launch order, one sequence's contiguous range at a time
  const uint32_t lin = blockIdx.x + gridDim.x * blockIdx.z;
  const int bx = PAGED ? (int)(lin / gridDim.z) : (int)blockIdx.x;
  const int bz = PAGED ? (int)(lin % gridDim.z) : (int)blockIdx.z;
  if ((int)bx >= key_blocks) {
    if (blockIdx.y == 0) {
      const uint16_t* k16 = static_cast<const uint16_t*>(job.kv);
      const uint16_t* z16 = static_cast<const uint16_t*>(job.z);
      const int64_t blk = (int64_t)bx - key_blocks;
      if (job.kv_b) {
        // overlapped pair: up to 2m <= 16 rows per entry, one row in flight per thread (the
        // job hides under the key stream; two would raise the whole kernel's register count)
        const uint16_t* kb16 = static_cast<const uint16_t*>(job.kv_b);
        const uint16_t* zb16 = static_cast<const uint16_t*>(job.z_b);
        if (z16)
          compress_block<kSlice, 16, kJobRS, true, true, 1, 1, true>(k16, z16, job.kv_off, ent_off, job.first_entry,
                                                                     128, job.m, job.max_new, job.out, bz,
                                                                     blk, kb16, zb16, pg);
        else
          compress_block<kSlice, 16, kJobRS, false, true, 1, 1, true>(k16, z16, job.kv_off, ent_off, job.first_entry,
                                                                      128, job.m, job.max_new, job.out, bz,
                                                                      blk, kb16, zb16, pg);
      } else if (z16) {
        compress_block<kSlice, 16, kJobRS, true, true, 1>(k16, z16, job.kv_off, ent_off, job.first_entry, 128, job.m,
                                                       job.max_new, job.out, bz, blk, nullptr, nullptr, pg);
      } else {
        compress_block<kSlice, 16, kJobRS, false, true, 1>(k16, z16, job.kv_off, ent_off, job.first_entry, 128, job.m,
                                                        job.max_new, job.out, bz, blk, nullptr, nullptr, pg);
      }
    }
    return;
  }
  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  const int g = lane / 16;
  const int c = lane % 16;
  const int b = bz;
  const int t0 = blockIdx.y * QPB;
  constexpr bool FP8 = KT == kKeyFP8;
  const float* k_scale = static_cast<const float*>(k_scale_v);   // fp8: per entry group
  const uint8_t* k_mx = static_cast<const uint8_t*>(k_scale_v);  // MXFP4: E8M0 per block

  const int64_t wg_e0 = (int64_t)bx * EPB;
  const int64_t e0 = wg_e0 + (int64_t)wave * EPW;
  const int64_t e_base = ent_off[b];
  const int64_t n_ent = ent_off[b + 1] - e_base;
  // paged layout: the pool rows of this lane's keys depend only on the block's position, so
  // their table entries load together with the entry offsets and the keys wait for one
  // round trip, not two
  int64_t prow[U];
  if (PAGED) {
    if (pg.eb_shift >= 4) {
      // blocks of 16 or more entries: each 16-key tile lies in one block, so its table entry
      // is the same for the whole wave; the table is read-only for the kernel's lifetime and
      // a constant-space read issues as a scalar load, all four before any is used
      const __attribute__((address_space(4))) int32_t* tbl =
          (const __attribute__((address_space(4))) int32_t*)(pg.table + (int64_t)b * pg.max_blocks);
      const uint32_t we0 = (uint32_t)wg_e0 + (uint32_t)__builtin_amdgcn_readfirstlane(threadIdx.x / kWave) * EPW;
      const uint32_t sh = (uint32_t)pg.eb_shift, jmax = (uint32_t)pg.max_blocks - 1u;
      uint32_t blk[U];
#pragma unroll
      for (int u = 0; u < U; ++u) blk[u] = (uint32_t)tbl[min((we0 + u * 16) >> sh, jmax)];
#pragma unroll
      for (int u = 0; u < U; ++u)
        prow[u] = ((int64_t)blk[u] << sh) | (int64_t)((we0 + u * 16 + c) & ((1u << sh) - 1u));
    } else {
#pragma unroll
      for (int u = 0; u < U; ++u) prow[u] = key_row<true>(pg, b, 0, e0 + u * 16 + c);
    }
  }

  const int64_t n_load = n_ent < max_entries ? n_ent : max_entries;
  if (wg_e0 >= n_load) return;  // the whole slice lies past this sequence: nothing to score or list
  const int64_t e_end = min(e0 + EPW, n_load);

  // key tiles first: they depend on nothing but the sequence's entry range
  u32x4 kb[U][2];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t s = e0 + u * 16 + c;
    load_key_tile<KT>(kI, k_mx, PAGED ? prow[u] : e_base + s, s < e_end, g, kb[u][0], kb[u][1]);
  }
  float my_scale = 1.f;  // fp8 group scale of this lane's entry on the way out
  if (FP8 && e0 + lane < e_end) my_scale = k_scale[scale_off[b] + (e0 + lane) / scale_group];

  // B operand: column c is head c % HI of query row t0 + c / HI
  const int tq = t0 + c / HI;
  bf16x8 qb[2];
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) {
    u32x4 v = u32x4{0, 0, 0, 0};
    if (tq < T) v = *reinterpret_cast<const u32x4*>(qI + (((int64_t)b * T + tq) * HI + c % HI) * 64 + kslot_dim<KT>(kk, g));
    qb[kk] = as_bf16x8(v);
  }
  const float wc = (tq < T) ? w[((int64_t)b * T + tq) * HI + c % HI] : 0.f;
  const int64_t p0 = q_pos[b];
  auto n_vis = [&](int t) -> int64_t {
    const int64_t p = p0 + t;
    int64_t nv = (p >= 0 && p < ((int64_t)1 << 32)) ? (int64_t)((uint32_t)p / (uint32_t)m) : p / m;
    nv = nv < n_load ? nv : n_load;
    return nv < 0 ? 0 : nv;
  };

  const bool writer = (c % HI) == 0 && tq < T;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    acc = mfma16x16x32(key_operand<KT>(kb[u][0]), qb[0], acc);
    acc = mfma16x16x32(key_operand<KT>(kb[u][1]), qb[1], acc);
    float v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = head_sum<HI>(wc * fmaxf(acc[i], 0.f));
    if (writer)
      *reinterpret_cast<float4*>(&sval[c / HI][wave * EPW + u * 16 + 4 * g]) = make_float4(v[0], v[1], v[2], v[3]);
  }
  // each wave reads back only what it wrote: LDS operations of one wave complete in order
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

  const int64_t s = e0 + lane;
  float mine = 0.f;
#pragma unroll
  for (int q = 0; q < QPB; ++q) {
    const int tt = t0 + q;
    if (tt >= T) break;
    const float val = sval[q][wave * EPW + lane] * my_scale;
    if (q == 0) mine = val;
    if (s < n_vis(tt)) scores[((int64_t)b * T + tt) * ld + s] = val;
  }
  if (PREP) {
    const int64_t n = n_vis(0);
    if (n > topk_k && wg_e0 < n && !topk_row_dense(n, topk_k)) {
      const uint32_t x = (s < n) ? score_key(mine) : 0u;
      const TopkRowWs rw = topk_row_ws(topk_ws, (int64_t)b * T, max_entries, slot_budget);
      const int R = topk_row_slots(n, max_entries, slot_budget);
      slice_candidates(x, slice_quota(n, topk_k, R), topk_wave_list(n, topk_k), R, sc, wg_e0, &rw.cuts[bx],
                       rw.slots + (int64_t)bx * R);
    }
  }
}

template <int HI, int KT>
hipError_t launch_hi(const void* qI, const float* w, const void* kI, const void* k_scale,
                     const int64_t* scale_off, int scale_group, const int64_t* ent_off,
                     const int64_t* q_pos, int m, int B, int T, int64_t max_entries, float* scores,
                     int64_t ld, void* topk_ws, int topk_k, hipStream_t st, const CompressJob* job,
                     const PagedView& pg) {
  const uint16_t* q16 = static_cast<const uint16_t*>(qI);
  const int rows = B * T;
  const bool prep = indexer_prepares_topk(topk_ws, T, max_entries);
  if (!prep && rows >= 64 && T >= 16) {  // prefill tiling (never carries a compress job)
    // prefill tiling: 8 A tiles per wave, 4 waves over the same keys
    constexpr int NB = 8, NW = 4, WQ = 4, U = 2;
    constexpr int QPW = NB * (16 / HI);
    const int epw = 256;
    const int64_t gx = (max_entries + epw - 1) / epw;
    const int gy = (T + QPW * WQ - 1) / (QPW * WQ);
    dim3 grid((unsigned)(gx > 0 ? gx : 1), (unsigned)gy, (unsigned)B);
    if (pg.table)
      indexer_kernel<HI, NB, NW, WQ, U, KT, true><<<grid, NW * 64, 0, st>>>(
          q16, w, kI, k_scale, scale_off, scale_group, ent_off, q_pos, m, T, max_entries, scores, ld, epw, pg);
    else
      indexer_kernel<HI, NB, NW, WQ, U, KT, false><<<grid, NW * 64, 0, st>>>(
          q16, w, kI, k_scale, scale_off, scale_group, ent_off, q_pos, m, T, max_entries, scores, ld, epw, pg);
  } else {
    // decode tiling: 8 waves per block, each with one pass over 64 keys (plus the job's blocks)
    constexpr int QPB = 16 / HI;
    const int64_t kb = (max_entries + kSlice - 1) / kSlice;
    const int64_t jb = job ? (job->max_new + kJobEntriesPerBlock - 1) / kJobEntriesPerBlock : 0;
    const int gy = (T + QPB - 1) / QPB;
    if ((kb + jb) * B >= ((int64_t)1 << 32)) return hipErrorInvalidValue;  // the kernel's linear block id
    dim3 grid((unsigned)(kb + jb), (unsigned)gy, (unsigned)B);
    const CompressJob none{};
    const CompressJob& cj = job ? *job : none;
#define CSL_IDX_DECODE(PREP, PG)                                                                                    \
  indexer_decode_kernel<HI, KT, PREP, PG><<<grid, kSlice, 0, st>>>(                                                 \
      q16, w, kI, k_scale, scale_off, scale_group, ent_off, q_pos, m, T, max_entries, scores, ld,                  \
      PREP ? topk_ws : nullptr, PREP ? topk_k : 0, PREP ? topk_slot_budget(max_entries, topk_k) : 0, (int)kb, cj, pg)
    if (prep) {
      if (pg.table) CSL_IDX_DECODE(true, true);
      else CSL_IDX_DECODE(true, false);
    } else {
      if (pg.table) CSL_IDX_DECODE(false, true);
      else CSL_IDX_DECODE(false, false);
    }
#undef CSL_IDX_DECODE
  }
  return hipGetLastError();
}

template <int KT>
hipError_t launch_kt(int HI, const void* qI, const float* w, const void* kI, const void* k_scale,
                      const int64_t* scale_off, int scale_group, const int64_t* ent_off,
                      const int64_t* q_pos, int m, int B, int T, int64_t max_entries, float* scores,
                      int64_t ld, void* topk_ws, int topk_k, hipStream_t st, const CompressJob* job,
                      const PagedView& pg) {
#define CSL_IDX_CASE(H)                                                                                          \
  case H:                                                                                                        \
    return launch_hi<H, KT>(qI, w, kI, k_scale, scale_off, scale_group, ent_off, q_pos, m, B, T, max_entries, \
                             scores, ld, topk_ws, topk_k, st, job, pg);
  switch (HI) {
    CSL_IDX_CASE(1)
    CSL_IDX_CASE(2)
    CSL_IDX_CASE(4)
    CSL_IDX_CASE(8)
    CSL_IDX_CASE(16)
    default: return hipErrorInvalidValue;
  }
#undef CSL_IDX_CASE
}

}  // namespace

bool indexer_prepares_topk(const void* topk_ws, int T, int64_t max_entries) {
  return topk_ws != nullptr && T == 1 && !topk_uses_row_kernel(max_entries) && max_entries <= kMultiMaxEntries;
}

static bool uses_prefill_tiling(const void* topk_ws, int B, int T, int64_t max_entries) {
  return !indexer_prepares_topk(topk_ws, T, max_entries) && (int64_t)B * T >= 64 && T >= 16;
}

bool indexer_carries_compress(const void* topk_ws, int B, int T, int64_t max_entries, int D, int m) {
  return D == 128 && m >= 1 && m <= 8 && max_entries > 0 && !uses_prefill_tiling(topk_ws, B, T, max_entries);
}

hipError_t launch_indexer(const void* qI, const float* w, const void* kI, int key_type, const void* k_scale,
                          const int64_t* scale_off, int scale_group, const int64_t* ent_off,
                          const int64_t* q_pos, int m, int B, int T, int HI, int64_t max_entries,
                          float* scores, int64_t ld, void* topk_ws, int topk_k, hipStream_t stream,
                          const CompressJob* job, const PagedView* paged) {
  const PagedView pg = paged ? *paged : PagedView{};
#define CSL_IDX_KT(KT)                                                                                     \
  launch_kt<KT>(HI, qI, w, kI, k_scale, scale_off, scale_group, ent_off, q_pos, m, B, T, max_entries, scores, \
                ld, topk_ws, topk_k, stream, job, pg)
  switch (key_type) {
    case kKeyFP8: return CSL_IDX_KT(kKeyFP8);
    case kKeyFP4: return CSL_IDX_KT(kKeyFP4);
    default: return CSL_IDX_KT(kKeyBF16);
  }
#undef CSL_IDX_KT
}

}  // namespace csl
