// indexer_scores: Lightning-indexer scores I(t,s) = sum_j w_j * ReLU(q_j . k_s).
//
// The score of every visible compressed indexer key is a dense contraction
// ([P5] indexer score formula; [P2] "Deep Dive", CSA Lightning Indexer): per query row,
// [HI heads x CI] x [CI x n keys], followed by ReLU, the head weights and a sum over heads.
// It runs on the gfx950 matrix cores as 16x16x32 bf16 MFMA tiles:
//   A (16 rows)   = 16/HI query rows x HI heads, held in registers for the whole kernel,
//   B (16 cols)   = 16 consecutive keys of one sequence, streamed from HBM,
//   D (16 x 16)   = per (query row, head) x key dot products in fp32.
// ReLU, the head weights, the optional fp8 group scale and the head sum run on the
// accumulator registers, so each key costs 128 bytes of reads (64 for fp8) and 4 bytes
// of score write per query row.
//
// Two tilings share the kernel:
//   decode  (NB=1, WQ=1): one A tile per wave; the 8 waves of a block split a contiguous
//           range of 512 keys, each wave issuing all its U=4 key tiles (8 KiB) in one pass
//           (a single pass per wave keeps the memory pipeline full; looping waves do not).
//   prefill (NB=8, WQ=4): each wave holds 8 A tiles (16/HI * 8 query rows) and the 4
//           waves walk the same key range, so a key tile fetched once is reused for
//           64/HI * 8 query rows through L1/L2.
// With a top-k workspace (single query row per sequence, long rows), each decode
// workgroup also keeps its 512 scores' keys in LDS and leaves that slice's top-k
// candidate list in the workspace (topk_common.h), so the selection never re-reads the
// scores.
#include "device_common.h"
#include "launch.h"
#include "topk_common.h"

namespace csl {

namespace {

template <bool FP8>
__device__ __forceinline__ void load_key_tile(const void* __restrict__ kI, int64_t row, bool ok, int g,
                                              u32x4& k0, u32x4& k1) {
  if (!ok) {
    k0 = u32x4{0, 0, 0, 0};
    k1 = u32x4{0, 0, 0, 0};
    return;
  }
  if (!FP8) {
    const uint16_t* p = static_cast<const uint16_t*>(kI) + row * 64 + g * 8;
    k0 = *reinterpret_cast<const u32x4*>(p);
    k1 = *reinterpret_cast<const u32x4*>(p + 32);
  } else {
    const uint8_t* p = static_cast<const uint8_t*>(kI) + row * 64 + g * 8;
    const u32x2 c0 = *reinterpret_cast<const u32x2*>(p);
    const u32x2 c1 = *reinterpret_cast<const u32x2*>(p + 32);
    // keep the raw codes; they are widened to bf16 just before the MFMA
    k0 = u32x4{c0.x, c0.y, 0, 0};
    k1 = u32x4{c1.x, c1.y, 0, 0};
  }
}

template <bool FP8>
__device__ __forceinline__ bf16x8 key_operand(const u32x4& k) {
  if (!FP8) return as_bf16x8(k);
  const u32x2 lo = e4m3x4_to_bf16x4(k.x);
  const u32x2 hi = e4m3x4_to_bf16x4(k.y);
  return as_bf16x8(u32x4{lo.x, lo.y, hi.x, hi.y});
}

template <int HI, int NB, int NWAVES, int WQ, int U, bool FP8, bool PREP>
__global__ __launch_bounds__(NWAVES * 64) void indexer_kernel(
    const uint16_t* __restrict__ qI, const float* __restrict__ w, const void* __restrict__ kI,
    const float* __restrict__ k_scale, const int64_t* __restrict__ scale_off, int scale_group,
    const int64_t* __restrict__ ent_off, const int64_t* __restrict__ q_pos, int m, int T,
    int64_t max_entries, float* __restrict__ scores, int64_t ld, int epw, void* topk_ws, int topk_k) {
  constexpr int QPB = 16 / HI;       // query rows per A tile
  constexpr int QPW = NB * QPB;      // query rows per wave
  constexpr int WE = NWAVES / WQ;    // key sub-ranges per block
  constexpr int NT = NWAVES * 64;
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
  if (!PREP && e0 >= e_end) return;  // with PREP every wave must reach the slice barrier
  constexpr int S = PREP ? WE * 16 * U : 1;  // a block's keys form one top-k slice
  static_assert(!PREP || (S == kSlice && NT == kSlice), "a prepared slice is one decode block, one key per thread");
  __shared__ uint32_t skeys[S];

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
      if (t < T) v = *reinterpret_cast<const u32x4*>(qI + (((int64_t)b * T + t) * HI + j) * 64 + kk * 32 + g * 8);
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
      load_key_tile<FP8>(kI, e_base + s, ok, g, kb[u][0], kb[u][1]);
      if (FP8) sc[u] = ok ? k_scale[scale_off[b] + s / scale_group] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t s = s0 + u * 16 + c;
      if (s0 + u * 16 >= e_end) break;
      const bf16x8 b0 = key_operand<FP8>(kb[u][0]);
      const bf16x8 b1 = key_operand<FP8>(kb[u][1]);
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
              if (PREP) skeys[s - wg_e0] = score_key(v);
            }
          }
        }
      }
    }
  }
  if (PREP) {
    __shared__ SliceScratch sc;
    __syncthreads();  // every wave's keys are in skeys
    const int64_t n = n_vis(0);
    if (n > topk_k && wg_e0 < n) {
      const uint32_t x = (wg_e0 + threadIdx.x < n) ? skeys[threadIdx.x] : 0u;
      const TopkRowWs rw = topk_row_ws(topk_ws, (int64_t)b * T, max_entries);
      slice_candidates(x, slice_quota(n, topk_k), sc, wg_e0, &rw.cuts[blockIdx.x],
                       rw.slots + (int64_t)blockIdx.x * kSliceSlots);
    }
  }
}

template <int HI, bool FP8>
hipError_t launch_hi(const void* qI, const float* w, const void* kI, const float* k_scale,
                     const int64_t* scale_off, int scale_group, const int64_t* ent_off,
                     const int64_t* q_pos, int m, int B, int T, int64_t max_entries, float* scores,
                     int64_t ld, void* topk_ws, int topk_k, hipStream_t st) {
  const uint16_t* q16 = static_cast<const uint16_t*>(qI);
  const int rows = B * T;
  const bool prep = indexer_prepares_topk(topk_ws, T, max_entries);
  if (!prep && rows >= 64 && T >= 16) {
    // prefill tiling: 8 A tiles per wave, 4 waves over the same keys
    constexpr int NB = 8, NW = 4, WQ = 4, U = 2;
    constexpr int QPW = NB * (16 / HI);
    const int epw = 256;
    const int64_t gx = (max_entries + epw - 1) / epw;
    const int gy = (T + QPW * WQ - 1) / (QPW * WQ);
    dim3 grid((unsigned)(gx > 0 ? gx : 1), (unsigned)gy, (unsigned)B);
    indexer_kernel<HI, NB, NW, WQ, U, FP8, false><<<grid, NW * 64, 0, st>>>(
        q16, w, kI, k_scale, scale_off, scale_group, ent_off, q_pos, m, T, max_entries, scores, ld, epw, nullptr, 0);
  } else {
    // decode tiling: every wave streams one pass of U key tiles (64 keys), 8 waves per block
    constexpr int NB = 1, NW = 8, WQ = 1, U = 4;
    constexpr int QPW = 16 / HI;
    const int epw = 16 * U;
    const int64_t per_block = (int64_t)epw * NW;
    const int64_t gx = (max_entries + per_block - 1) / per_block;
    const int gy = (T + QPW - 1) / QPW;
    dim3 grid((unsigned)(gx > 0 ? gx : 1), (unsigned)gy, (unsigned)B);
    if (prep)
      indexer_kernel<HI, NB, NW, WQ, U, FP8, true><<<grid, NW * 64, 0, st>>>(
          q16, w, kI, k_scale, scale_off, scale_group, ent_off, q_pos, m, T, max_entries, scores, ld, epw, topk_ws,
          topk_k);
    else
      indexer_kernel<HI, NB, NW, WQ, U, FP8, false><<<grid, NW * 64, 0, st>>>(
          q16, w, kI, k_scale, scale_off, scale_group, ent_off, q_pos, m, T, max_entries, scores, ld, epw, nullptr, 0);
  }
  return hipGetLastError();
}

template <bool FP8>
hipError_t launch_fp8(int HI, const void* qI, const float* w, const void* kI, const float* k_scale,
                      const int64_t* scale_off, int scale_group, const int64_t* ent_off,
                      const int64_t* q_pos, int m, int B, int T, int64_t max_entries, float* scores,
                      int64_t ld, void* topk_ws, int topk_k, hipStream_t st) {
#define CSL_IDX_CASE(H)                                                                                          \
  case H:                                                                                                        \
    return launch_hi<H, FP8>(qI, w, kI, k_scale, scale_off, scale_group, ent_off, q_pos, m, B, T, max_entries, \
                             scores, ld, topk_ws, topk_k, st);
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

hipError_t launch_indexer(const void* qI, const float* w, const void* kI, bool fp8, const float* k_scale,
                          const int64_t* scale_off, int scale_group, const int64_t* ent_off,
                          const int64_t* q_pos, int m, int B, int T, int HI, int64_t max_entries,
                          float* scores, int64_t ld, void* topk_ws, int topk_k, hipStream_t stream) {
  if (fp8)
    return launch_fp8<true>(HI, qI, w, kI, k_scale, scale_off, scale_group, ent_off, q_pos, m, B, T, max_entries,
                            scores, ld, topk_ws, topk_k, stream);
  return launch_fp8<false>(HI, qI, w, kI, k_scale, scale_off, scale_group, ent_off, q_pos, m, B, T, max_entries,
                           scores, ld, topk_ws, topk_k, stream);
}

}  // namespace csl
