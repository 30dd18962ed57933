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
#include "indexer_common.h"

namespace csl {

namespace {

// Prefill tiling: queries are the MFMA A operand (16/HI query rows x HI heads per tile) and
// keys the B operand, so lane (g, c) holds products 4g..4g+3 (query row, head) of key c. The
// head-weighted ReLU sum of one query row gathers in part[q]; it is complete in the writer
// lanes, and prefill_row names its row inside the A tile. The indexer and the fused
// indexer/top-k kernel share this arithmetic, so their scores agree bit for bit.
template <int HI>
constexpr int prefill_rows_per_group() { return HI >= 4 ? 1 : 4 / HI; }

// max(0, x) as one integer max on the bits: a negative float (and -0) is a negative integer,
// so it becomes +0; the same as the float maximum for every value but NaN, which products of
// finite bf16 values do not produce
__device__ __forceinline__ float relu_bits(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

template <int HI>
__device__ __forceinline__ void prefill_head_sum(const f32x4& acc, const float (&wv)[4],
                                                 float (&part)[prefill_rows_per_group<HI>()]) {
  constexpr int RPG = prefill_rows_per_group<HI>();
#pragma unroll
  for (int q = 0; q < RPG; ++q) part[q] = 0.f;
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int q = (HI >= 4) ? 0 : it / HI;
    part[q] = fmaf(wv[it], relu_bits(acc[it]), part[q]);
  }
  // the partner row's value comes from gfx950's row swaps, not through LDS: permlane16_swap
  // returns (even row, odd row) of each pair of 16-lane rows in every lane, permlane32_swap
  // (lower half, upper half), so their sum is the lane's value plus its partner's
  if (HI >= 8) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(part[0]), __float_as_uint(part[0]), false, false);
    part[0] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
  if (HI == 16) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(part[0]), __float_as_uint(part[0]), false, false);
    part[0] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
}

template <int HI>
__device__ __forceinline__ bool prefill_writer(int g) {
  return (HI == 16) ? (g == 0) : (HI == 8) ? ((g & 1) == 0) : true;
}

template <int HI>
__device__ __forceinline__ int prefill_row(int g, int q) {
  return (HI >= 8) ? (4 * g) / HI : (4 * g) / HI + q;
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
  constexpr int ROWS_PER_GROUP = prefill_rows_per_group<HI>();  // query rows in one lane group's 4 C rows

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
      const int rq = prefill_row<HI>(g, q);
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
      const int64_t kr = key_row<PAGED>(pg, b, e_base, s);
      load_key_tile<KT>(kI, k_mx, kr, ok, g, kb[u][0], kb[u][1]);
      if (FP8) sc[u] = ok ? k_scale[fp8_scale_index<PAGED>(pg, kr, scale_off, b, s, scale_group)] : 0.f;
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
        prefill_head_sum<HI>(acc, wv[nb], part);
        if (prefill_writer<HI>(g)) {
#pragma unroll
          for (int q = 0; q < ROWS_PER_GROUP; ++q) {
            const int rq = prefill_row<HI>(g, q);
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

// ---------------------------------------------------------------------------------------------
// Indexer fused with top-k: the scores never leave the chip. A workgroup takes QR query rows
// (8; 16 at HI = 1) over the whole key range, in chunks of 256 keys: its 8 waves score the
// chunk with the prefill tiling's MFMAs and arithmetic into one of two LDS staging buffers,
// then each wave files the scores of its own rows into that row's candidate buffer in LDS
// (the LDS left to the workgroup: 960 slots per row, 2240 at HI = 16),
// admitting only keys above the row's bar. The keys of the next chunk are in flight while a
// chunk is filed, and with two staging buffers one barrier per chunk suffices: a
// wave that passes the barrier of chunk j has filed chunk j - 1, whose buffer chunk j + 1
// then reuses. The buffer holds (key << 32 | id) in ascending id order. When it could
// overflow, the wave cuts it to exactly the k best by (score descending, id ascending) and
// raises the bar to the k-th key: a later entry at or below the bar can never enter the top-k
// (its key is lower, or equal with a higher id), and an entry cut is below k better ones. At
// the end the buffer is cut to k once more and written out in id order, -1 padded.

constexpr int kFusedWaves = 8;
constexpr int kFusedU = 2;                               // key tiles of 16 per wave and chunk
constexpr int kFusedChunk = kFusedWaves * kFusedU * 16;  // keys per chunk
constexpr int kFusedCuLds = 160 * 1024;                  // LDS of one gfx950 compute unit

template <int HI, bool WIDE = false>
struct FusedShape {
  static constexpr int QPB = 16 / HI;
  static constexpr int QR = QPB > 8 ? QPB : 8;  // query rows per workgroup: 8 (16 at HI = 1)
  static constexpr int NB = QR / QPB;           // A tiles (all waves hold all of them)
  // two workgroups per compute unit, so each wave has three others on its SIMD to hide
  // latency behind (one at HI = 1, whose A tile alone spans 16 rows, and at HI = 16, whose
  // 8 A tiles need more registers than 4 waves per SIMD leave). WIDE: one workgroup per CU
  // and so twice the candidate slots, for k beyond what two workgroups' buffers hold
  static constexpr int WG_PER_CU = (!WIDE && QR == 8 && NB <= 4) ? 2 : 1;
  static constexpr int WAVES_PER_SIMD = WG_PER_CU * kFusedWaves / 4;
  // candidate slots per row: the workgroup's LDS share left beside the two staging buffers
  static constexpr int CAP = (kFusedCuLds / WG_PER_CU - 2 * QR * kFusedChunk * 4 - 256) / (8 * QR) / 64 * 64;
  static_assert(CAP % 64 == 0 && CAP >= 512, "whole waves of slots");
};

// Cut a row's candidate buffer (n > k entries, ascending ids) in place, keeping id order, and
// return the new bar. EXACT: exactly its k best remain and the bar is the k-th best key.
// Otherwise the search may stop at a key prefix P that at least k and at most k + 32 keys
// reach (fewer when k is close to CAP - 64), which takes fewer steps: those all remain. The bar is the smallest key kept: at
// least k kept keys reach it, so a later key at or below it has k better ones before it.
// One wave, wave-uniform result.
template <int CAP, bool EXACT>
__device__ __forceinline__ uint32_t cut_to_k(uint64_t* row, uint32_t& n, int k) {
  constexpr int J = CAP / kWave;
  const int lane = (int)lane_id();
  uint32_t xs[J];
  uint32_t hi = 0u, lo = 0xffffffffu;
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const uint32_t i = (uint32_t)(j * kWave + lane);
    xs[j] = i < n ? (uint32_t)(row[i] >> 32) : 0u;
    if (i < n) {
      hi = max(hi, xs[j]);
      lo = min(lo, xs[j]);
    }
  }
  hi = wave_max_u32(hi);
  lo = wave_min_u32(lo);
  // the k-th largest key, bit by bit below the prefix all keys share; a prefix that already
  // has exactly k keys at or above it ends the search (those k are the k best). The bits
  // below the prefix come from smearing hi ^ lo rightwards: plain arithmetic, which also
  // covers hi == lo (a select on the leading-zero count of hi ^ lo was built wrongly here:
  // the select read a condition flag that the shift before it had overwritten)
  uint32_t below = hi ^ lo;
  below |= below >> 1;
  below |= below >> 2;
  below |= below >> 4;
  below |= below >> 8;
  below |= below >> 16;
  uint32_t t = hi & ~below;
  bool exact = false;  // every key at or above t remains: no ties to resolve
  uint32_t reach = n;  // keys at or above t
  // a coarse cut keeps at most k + 32 keys, and always room for a 64-key step after it
  const uint32_t loose = (uint32_t)k + min(32u, (uint32_t)(CAP - kWave - k));
  {
    for (int bit = __popc(below) - 1; bit >= 0; --bit) {
      if (!EXACT && reach <= loose) {
        exact = true;
        break;
      }
      const uint32_t c = t | (1u << bit);
      uint32_t cnt = 0;
#pragma unroll
      for (int j = 0; j < J; ++j) cnt += (uint32_t)__popcll(__ballot(xs[j] >= c));
      if (cnt >= (uint32_t)k) {
        t = c;
        reach = cnt;
        if (cnt == (uint32_t)k) {
          exact = true;
          break;
        }
      }
    }
  }
  // otherwise t is the k-th key itself: keep every key above it and the lowest-id ties
  uint32_t need = (uint32_t)k;
  if (!exact) {
    uint32_t gt = 0;
#pragma unroll
    for (int j = 0; j < J; ++j) gt += (uint32_t)__popcll(__ballot(xs[j] > t));
    need = (uint32_t)k - gt;
  }
  uint32_t out = 0, ties = 0, bar = 0xffffffffu;
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const uint32_t i = (uint32_t)(j * kWave + lane);
    const bool valid = i < n;
    const uint32_t x = xs[j];
    const uint64_t v = valid ? row[i] : 0ull;  // slots at or after j * 64 are not yet rewritten
    bool keep;
    if (exact) {
      keep = valid && x >= t;
    } else {
      const bool tie = valid && x == t;
      const uint64_t tm = __ballot(tie);
      const uint32_t tr = ties + rank_in_wave(tm);
      ties += (uint32_t)__popcll(tm);
      keep = valid && (x > t || (tie && tr < need));
    }
    const uint64_t km = __ballot(keep);
    if (keep) {
      row[out + rank_in_wave(km)] = v;
      bar = min(bar, x);
    }
    out += (uint32_t)__popcll(km);
  }
  n = out;
  return wave_min_u32(bar);  // the smallest key kept: at least k keys reach it
}

template <int HI, int KT, bool PAGED, bool WIDE>
__global__ __launch_bounds__(kFusedWaves * kWave, (FusedShape<HI, WIDE>::WAVES_PER_SIMD)) void indexer_topk_kernel(
    const uint16_t* __restrict__ qI, const float* __restrict__ w, const void* __restrict__ kI,
    const void* __restrict__ k_scale_v, const int64_t* __restrict__ scale_off, int scale_group,
    const int64_t* __restrict__ ent_off, const int64_t* __restrict__ q_pos, int m, int T,
    int64_t max_entries, int k, int32_t* __restrict__ idx, PagedView pg) {
  using FS = FusedShape<HI, WIDE>;
  constexpr int QPB = FS::QPB, NB = FS::NB, QR = FS::QR, CAP = FS::CAP;
  constexpr int U = kFusedU, CH = kFusedChunk;
  constexpr int RPW = QR / kFusedWaves;  // rows each wave files (1, or 2 at HI = 1)
  constexpr int RPG = prefill_rows_per_group<HI>();
  static_assert(RPW >= 1 && QR % kFusedWaves == 0, "whole rows per wave");
  __shared__ __align__(16) float sval[2][QR][CH];
  __shared__ uint64_t cand[QR][CAP];
  __shared__ uint32_t cut_req;  // last chunk index by which some row asked all rows to cut

  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  const int g = lane / 16;
  const int c = lane % 16;
  const int b = blockIdx.z;
  const int t0 = blockIdx.x * QR;
  constexpr bool FP8 = KT == kKeyFP8;
  const float* k_scale = static_cast<const float*>(k_scale_v);
  const uint8_t* k_mx = static_cast<const uint8_t*>(k_scale_v);

  const int64_t e_base = ent_off[b];
  const int64_t n_ent = ent_off[b + 1] - e_base;
  const int64_t n_load = n_ent < max_entries ? n_ent : max_entries;
  const int64_t p0 = q_pos[b];
  auto n_vis = [&](int t) -> int64_t {
    const int64_t p = p0 + t;
    int64_t nv = (p >= 0 && p < ((int64_t)1 << 32)) ? (int64_t)((uint32_t)p / (uint32_t)m) : p / m;
    nv = nv < n_load ? nv : n_load;
    return nv < 0 ? 0 : nv;
  };

  // queries and head weights of all QR rows (every wave scores every row)
  bf16x8 a[NB][2];
  float wv[NB][4];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int t = t0 + nb * QPB + c / HI;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      u32x4 v = u32x4{0, 0, 0, 0};
      if (t < T) v = *reinterpret_cast<const u32x4*>(qI + (((int64_t)b * T + t) * HI + c % HI) * 64 + kslot_dim<KT>(kk, g));
      a[nb][kk] = as_bf16x8(v);
    }
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int r = 4 * g + it;
      const int tt = t0 + nb * QPB + r / HI;
      wv[nb][it] = (tt < T) ? w[((int64_t)b * T + tt) * HI + (r % HI)] : 0.f;
    }
  }
  // the rows this wave files: visible entries, buffer fill and bar (wave-uniform)
  int64_t nv_mine[RPW];
  uint32_t cnt[RPW], bar[RPW];
#pragma unroll
  for (int i = 0; i < RPW; ++i) {
    const int t = t0 + wave * RPW + i;
    nv_mine[i] = t < T ? n_vis(t) : 0;
    cnt[i] = 0;
    bar[i] = 0;  // every real key is above 0
  }
  const int t_last = min(t0 + QR, T) - 1;
  const int64_t n_max = t_last >= t0 ? n_vis(t_last) : 0;  // visibility grows with t

  // key tiles of one chunk for this wave: keys s0 + (wave * U + u) * 16 + c. The narrow shape
  // holds one chunk ahead; the wide one, with registers to spare, two (KD key buffers in turn).
  // Past the row's end the loads take key 0 of the sequence and the values are masked, so the
  // loads never branch and the wait before each chunk's products counts exactly the newer
  // chunk's loads.
  constexpr int KD = WIDE ? 2 : 1;
  struct Keys {
    u32x4 k[U][2];
    float sc[U];
  };
  Keys kbuf[KD];
  auto load_chunk = [&](int64_t s0, Keys& kk) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t s = s0 + (wave * U + u) * 16 + c;
      const bool ok = s < n_max;
      const int64_t kr = key_row<PAGED>(pg, b, e_base, (WIDE && !ok) ? 0 : s);
      if (WIDE) {
        load_key_tile<KT>(kI, k_mx, kr, true, g, kk.k[u][0], kk.k[u][1]);
        if (FP8) kk.sc[u] = k_scale[fp8_scale_index<PAGED>(pg, kr, scale_off, b, ok ? s : 0, scale_group)];
      } else {
        load_key_tile<KT>(kI, k_mx, kr, ok, g, kk.k[u][0], kk.k[u][1]);
        if (FP8) kk.sc[u] = ok ? k_scale[fp8_scale_index<PAGED>(pg, kr, scale_off, b, s, scale_group)] : 0.f;
      }
    }
  };
  if (threadIdx.x == 0) cut_req = 0;  // read only after the first chunk's barrier
  if (n_max > 0) {
    load_chunk(0, kbuf[0]);
    if (KD > 1) load_chunk(CH, kbuf[KD - 1]);
  }
  int buf = 0;
  uint32_t jc = 0;  // chunk index
  // one chunk (keys s0 .., its key buffer kk, which then takes the keys KD chunks ahead): the
  // narrow shape walks it in a plain loop, the wide one twice per trip so that each copy names
  // its key buffer at compile time (written out, not as a lambda: a lambda capturing the
  // kernel's arrays costs the narrow shape registers)
#define CSL_FUSED_CHUNK(S0_, kk)                                                                                   \
  do {                                                                                                            \
    const int64_t s0 = (S0_);                                                                                     \
    bf16x8 b0[U], b1[U];                                                                                          \
    float scu[U];                                                                                                 \
_Pragma("unroll")                                                                                                 \
    for (int u = 0; u < U; ++u) {                                                                                 \
      b0[u] = key_operand<KT>(kk.k[u][0]);                                                                        \
      b1[u] = key_operand<KT>(kk.k[u][1]);                                                                        \
      scu[u] = kk.sc[u];                                                                                          \
    }                                                                                                             \
_Pragma("unroll")                                                                                                 \
    for (int u = 0; u < U; ++u) {                                                                                 \
      /* the NB products of a key tile are independent: issue them back to back */                                \
      f32x4 acc[NB];                                                                                              \
_Pragma("unroll")                                                                                                 \
      for (int nb = 0; nb < NB; ++nb) acc[nb] = mfma16x16x32(a[nb][0], b0[u], f32x4{0.f, 0.f, 0.f, 0.f});         \
_Pragma("unroll")                                                                                                 \
      for (int nb = 0; nb < NB; ++nb) acc[nb] = mfma16x16x32(a[nb][1], b1[u], acc[nb]);                           \
_Pragma("unroll")                                                                                                 \
      for (int nb = 0; nb < NB; ++nb) {                                                                           \
        float part[RPG];                                                                                          \
        prefill_head_sum<HI>(acc[nb], wv[nb], part);                                                              \
        /* every lane writes: lanes that share a (row, key) hold the same sum bit for bit */                      \
_Pragma("unroll")                                                                                                 \
        for (int q = 0; q < RPG; ++q) {                                                                           \
          float v = part[q];                                                                                      \
          if (FP8) v *= scu[u];                                                                                   \
          sval[buf][nb * QPB + prefill_row<HI>(g, q)][(wave * U + u) * 16 + c] = v;                               \
        }                                                                                                         \
      }                                                                                                           \
    }                                                                                                             \
    /* the next chunk's keys fly during the barrier and the filing (issued after the MFMAs, so */                 \
    /* they do not hold registers beside this chunk's operands); with two buffers, the chunk */                   \
    /* after it goes into this chunk's buffer */                                                                  \
    if (KD == 1) {                                                                                                \
      if (s0 + CH < n_max) load_chunk(s0 + CH, kk);                                                               \
    } else {                                                                                                      \
      load_chunk(s0 + KD * CH, kk);                                                                               \
    }                                                                                                             \
    __syncthreads();                                                                                              \
    /* Rows fill at similar rates, so cuts are taken together: a row that the next chunk might */                 \
    /* overflow asks for a cut by chunk jc + 1, and at that chunk every wave cuts its rows that */                \
    /* hold more than k + 64 entries. Cuts taken apart would each hold up the others at the */                    \
    /* next barrier. (A wave that reads a later request cuts early: harmless.) */                                 \
    const bool cut_now = jc > 0 && *(volatile uint32_t*)&cut_req >= jc;                                           \
    bool ask = false;                                                                                             \
_Pragma("unroll")                                                                                                 \
    for (int i = 0; i < RPW; ++i) {                                                                               \
      const int r = wave * RPW + i;                                                                               \
      if (cut_now && cnt[i] > (uint32_t)k + 64u) bar[i] = cut_to_k<CAP, false>(cand[r], cnt[i], k);               \
      /* a coarse cut leaves at most k + 32 entries; when a whole chunk fits after that, one */                   \
      /* check per chunk suffices, against the keys the chunk actually admits */                                  \
      const bool chunk_check = (uint32_t)k + 32u + CH <= (uint32_t)CAP;                                           \
      if (chunk_check || cnt[i] + CH <= (uint32_t)CAP) {                                                          \
        /* the chunk's score reads go out together, then the ballots */                                           \
        uint32_t x[CH / kWave];                                                                                   \
        float v[CH / kWave];                                                                                      \
_Pragma("unroll")                                                                                                 \
        for (int j = 0; j < CH / kWave; ++j) v[j] = sval[buf][r][j * kWave + lane]; /* in range: read unmasked */ \
_Pragma("unroll")                                                                                                 \
        for (int j = 0; j < CH / kWave; ++j) {                                                                    \
          const int64_t s = s0 + j * kWave + lane;                                                                \
          x[j] = s < nv_mine[i] ? score_key(v[j]) : 0u;                                                           \
        }                                                                                                         \
        uint64_t mk[CH / kWave];                                                                                  \
        uint32_t adm = 0;                                                                                         \
_Pragma("unroll")                                                                                                 \
        for (int j = 0; j < CH / kWave; ++j) {                                                                    \
          mk[j] = __ballot(x[j] > bar[i]);                                                                        \
          adm += (uint32_t)__popcll(mk[j]);                                                                       \
        }                                                                                                         \
        if (cnt[i] + adm > (uint32_t)CAP) { /* only with chunk_check: cut, then admit above the new bar */        \
          bar[i] = cut_to_k<CAP, false>(cand[r], cnt[i], k);                                                      \
_Pragma("unroll")                                                                                                 \
          for (int j = 0; j < CH / kWave; ++j) mk[j] = __ballot(x[j] > bar[i]);                                   \
          adm = 0;                                                                                                \
        }                                                                                                         \
_Pragma("unroll")                                                                                                 \
        for (int j = 0; j < CH / kWave; ++j) {                                                                    \
          if ((mk[j] >> lane) & 1ull)                                                                             \
            cand[r][cnt[i] + rank_in_wave(mk[j])] = ((uint64_t)x[j] << 32) | (uint32_t)(s0 + j * kWave + lane);   \
          cnt[i] += (uint32_t)__popcll(mk[j]);                                                                    \
        }                                                                                                         \
        /* ask for a shared cut when the next chunks are likely to overflow this row */                           \
        ask = ask || cnt[i] + (chunk_check ? 2u * max(adm, 32u) : (uint32_t)CH) > (uint32_t)CAP;                  \
      } else {                                                                                                    \
_Pragma("unroll 1")                                                                                               \
        for (int j = 0; j < CH / kWave; ++j) { /* not unrolled: one copy of the cut per row */                    \
          if (cnt[i] + kWave > (uint32_t)CAP) bar[i] = cut_to_k<CAP, false>(cand[r], cnt[i], k);                  \
          const int64_t s = s0 + j * kWave + lane;                                                                \
          const float v = sval[buf][r][j * kWave + lane];                                                         \
          const uint32_t x = s < nv_mine[i] ? score_key(v) : 0u;                                                  \
          const bool admit = x > bar[i];                                                                          \
          const uint64_t mk = __ballot(admit);                                                                    \
          if (admit) cand[r][cnt[i] + rank_in_wave(mk)] = ((uint64_t)x << 32) | (uint32_t)s;                      \
          cnt[i] += (uint32_t)__popcll(mk);                                                                       \
        }                                                                                                         \
        ask = ask || cnt[i] + CH > (uint32_t)CAP;                                                                 \
      }                                                                                                           \
    }                                                                                                             \
    if (ask && lane == 0) atomicMax(&cut_req, jc + 1);                                                            \
  } while (0)
  if constexpr (KD == 1) {
    for (int64_t c0 = 0; c0 < n_max; c0 += CH, buf ^= 1, ++jc) CSL_FUSED_CHUNK(c0, kbuf[0]);
  } else {
    for (int64_t c0 = 0; c0 < n_max; c0 += 2 * CH) {
      CSL_FUSED_CHUNK(c0, kbuf[0]);
      buf ^= 1;
      ++jc;
      if (c0 + CH >= n_max) break;
      CSL_FUSED_CHUNK(c0 + CH, kbuf[KD - 1]);
      buf ^= 1;
      ++jc;
    }
  }
#undef CSL_FUSED_CHUNK
#pragma unroll
  for (int i = 0; i < RPW; ++i) {
    const int r = wave * RPW + i;
    const int t = t0 + r;
    if (t >= T) continue;
    if (cnt[i] > (uint32_t)k) cut_to_k<CAP, true>(cand[r], cnt[i], k);
    int32_t* out = idx + ((int64_t)b * T + t) * k;
    for (int j = lane; j < k; j += kWave) out[j] = (uint32_t)j < cnt[i] ? (int32_t)(uint32_t)cand[r][j] : -1;
  }
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
    int key_blocks, CompressJob job, PagedView pg, int on_demand) {
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
  if (FP8 && e0 + lane < e_end) {
    int64_t kr = e0 + lane;
    if (PAGED) {  // entry e0 + lane is key u = lane / 16 of this lane's column c: pool row prow[u]
      kr = prow[0];
#pragma unroll
      for (int u = 1; u < U; ++u)
        if (lane / 16 == u) kr = prow[u];
    }
    my_scale = k_scale[fp8_scale_index<PAGED>(pg, kr, scale_off, b, e0 + lane, scale_group)];
  }

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
    float v[4];
    decode_score_tile<HI, KT>(kb[u][0], kb[u][1], qb, wc, v);
    if (writer)
      *reinterpret_cast<float4*>(&sval[c / HI][wave * EPW + u * 16 + 4 * g]) = make_float4(v[0], v[1], v[2], v[3]);
  }
  // each wave reads back only what it wrote: LDS operations of one wave complete in order
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

  const int64_t s = e0 + lane;
  float mine = 0.f;
  // scores on demand: a row whose selection runs on candidate lists keeps no scores (the
  // finishing step recomputes a row's scores if its lists cannot prove the selection); rows
  // too dense for lists are selected from their scores
  const bool keep_scores = !(PREP && on_demand) || topk_row_dense(n_vis(0), topk_k);
#pragma unroll
  for (int q = 0; q < QPB; ++q) {
    const int tt = t0 + q;
    if (tt >= T) break;
    const float val = sval[q][wave * EPW + lane] * my_scale;
    if (q == 0) mine = val;
    if (keep_scores && s < n_vis(tt)) scores[((int64_t)b * T + tt) * ld + s] = val;
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
                     const PagedView& pg, bool on_demand) {
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
      PREP ? topk_ws : nullptr, PREP ? topk_k : 0, PREP ? topk_slot_budget(max_entries, topk_k) : 0, (int)kb, cj, pg, \
      (PREP && on_demand) ? 1 : 0)
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

template <int HI, int KT>
hipError_t launch_topk_hi(const void* qI, const float* w, const void* kI, const void* k_scale,
                          const int64_t* scale_off, int scale_group, const int64_t* ent_off, const int64_t* q_pos,
                          int m, int B, int T, int64_t max_entries, int k, int32_t* idx, hipStream_t st,
                          const PagedView& pg) {
  constexpr int QR = FusedShape<HI>::QR;
  dim3 grid((unsigned)((T + QR - 1) / QR), 1u, (unsigned)B);
  const uint16_t* q16 = static_cast<const uint16_t*>(qI);
  // the wide shape (one workgroup per CU, twice the candidate slots) once k leaves the narrow
  // buffer less than a chunk of room after a cut: a buffer that tight is cut almost every chunk
  constexpr bool kHasWide = FusedShape<HI, true>::CAP > FusedShape<HI, false>::CAP;
  const bool wide = kHasWide && k + kFusedChunk + 32 > FusedShape<HI, false>::CAP;
#define CSL_TOPK_LAUNCH(PG, WD)                                                                   \
  indexer_topk_kernel<HI, KT, PG, WD><<<grid, kFusedWaves * kWave, 0, st>>>(                    \
      q16, w, kI, k_scale, scale_off, scale_group, ent_off, q_pos, m, T, max_entries, k, idx, pg)
  if (wide) {
    if constexpr (kHasWide) {
      if (pg.table) CSL_TOPK_LAUNCH(true, true);
      else CSL_TOPK_LAUNCH(false, true);
    }
  } else {
    if (pg.table) CSL_TOPK_LAUNCH(true, false);
    else CSL_TOPK_LAUNCH(false, false);
  }
#undef CSL_TOPK_LAUNCH
  return hipGetLastError();
}

template <int KT>
hipError_t launch_topk_kt(int HI, const void* qI, const float* w, const void* kI, const void* k_scale,
                          const int64_t* scale_off, int scale_group, const int64_t* ent_off, const int64_t* q_pos,
                          int m, int B, int T, int64_t max_entries, int k, int32_t* idx, hipStream_t st,
                          const PagedView& pg) {
#define CSL_FUSED_CASE(H)                                                                                       \
  case H:                                                                                                       \
    return launch_topk_hi<H, KT>(qI, w, kI, k_scale, scale_off, scale_group, ent_off, q_pos, m, B, T,           \
                                 max_entries, k, idx, st, pg);
  switch (HI) {
    CSL_FUSED_CASE(1)
    CSL_FUSED_CASE(2)
    CSL_FUSED_CASE(4)
    CSL_FUSED_CASE(8)
    CSL_FUSED_CASE(16)
    default: return hipErrorInvalidValue;
  }
#undef CSL_FUSED_CASE
}

template <int KT>
hipError_t launch_kt(int HI, const void* qI, const float* w, const void* kI, const void* k_scale,
                      const int64_t* scale_off, int scale_group, const int64_t* ent_off,
                      const int64_t* q_pos, int m, int B, int T, int64_t max_entries, float* scores,
                      int64_t ld, void* topk_ws, int topk_k, hipStream_t st, const CompressJob* job,
                      const PagedView& pg, bool on_demand) {
#define CSL_IDX_CASE(H)                                                                                          \
  case H:                                                                                                        \
    return launch_hi<H, KT>(qI, w, kI, k_scale, scale_off, scale_group, ent_off, q_pos, m, B, T, max_entries, \
                             scores, ld, topk_ws, topk_k, st, job, pg, on_demand);
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

int indexer_topk_max_k(int HI) {
  // the larger of the two shapes' buffers (HI = 2, 4 and 8 share theirs), less a chunk and the
  // 32 a coarse cut may keep: a cut always leaves room for a whole chunk (a buffer cut more
  // often than that spends most of its time cutting)
  const int cap = HI == 1 ? FusedShape<1, true>::CAP : HI == 16 ? FusedShape<16, true>::CAP : FusedShape<8, true>::CAP;
  return cap - kFusedChunk - 32;
}

hipError_t launch_indexer_topk(const void* qI, const float* w, const void* kI, int key_type, const void* k_scale,
                               const int64_t* scale_off, int scale_group, const int64_t* ent_off,
                               const int64_t* q_pos, int m, int B, int T, int HI, int64_t max_entries, int k,
                               int32_t* idx, hipStream_t st, const PagedView* paged) {
  const PagedView pg = paged ? *paged : PagedView{};
  switch (key_type) {
    case kKeyBF16:
      return launch_topk_kt<kKeyBF16>(HI, qI, w, kI, k_scale, scale_off, scale_group, ent_off, q_pos, m, B, T,
                                      max_entries, k, idx, st, pg);
    case kKeyFP8:
      return launch_topk_kt<kKeyFP8>(HI, qI, w, kI, k_scale, scale_off, scale_group, ent_off, q_pos, m, B, T,
                                     max_entries, k, idx, st, pg);
    case kKeyFP4:
      return launch_topk_kt<kKeyFP4>(HI, qI, w, kI, k_scale, scale_off, scale_group, ent_off, q_pos, m, B, T,
                                     max_entries, k, idx, st, pg);
    default: return hipErrorInvalidValue;
  }
}

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
                          const CompressJob* job, const PagedView* paged, bool scores_on_demand) {
  const PagedView pg = paged ? *paged : PagedView{};
  // scores on demand only where the finishing step can recompute a row: packed layout
  const bool on_demand = scores_on_demand && !paged;
#define CSL_IDX_KT(KT)                                                                                     \
  launch_kt<KT>(HI, qI, w, kI, k_scale, scale_off, scale_group, ent_off, q_pos, m, B, T, max_entries, scores, \
                ld, topk_ws, topk_k, stream, job, pg, on_demand)
  switch (key_type) {
    case kKeyFP8: return CSL_IDX_KT(kKeyFP8);
    case kKeyFP4: return CSL_IDX_KT(kKeyFP4);
    default: return CSL_IDX_KT(kKeyBF16);
  }
#undef CSL_IDX_KT
}

}  // namespace csl
