// topk_select: the k highest indexer scores of every query row, lower id first on ties,
// written as ascending ids padded with -1 ([P2] "Deep Dive", CSA top-k selection).
//
// Scores are compared through an order-preserving 32-bit key; a tie on the key is broken
// by the lower id, so (key descending, id ascending) is a strict total order and the top-k
// set is unique. Two paths:
//
//   * short rows (n <= 34816, e.g. a 4K-context decode or a prefill chunk over a 131K
//     prefix): one 1024-thread workgroup per row holds the row's keys in registers
//     (element i = j*1024 + tid), radix-selects the k-th best key on the bits below the keys'
//     common prefix, and writes the selection with a block-wide ordered compaction (lower
//     ids first among keys tied at the threshold), so the output is ascending by construction;
//
//   * long rows (decode at 1M context: 262144 scores per row): every 512-entry slice of the
//     row lists its own candidates above an honest slice cut (topk_common.h) -- either
//     inside indexer_scores, which already holds the scores, or in a prepare kernel here --
//     and one workgroup per row finishes: it radix-selects the k best listed entries on
//     their 32-bit keys (lower id first within the last tied key), checks that the k-th
//     best listed key reaches every slice's cut (then the selection is the row's), and
//     writes the winners in ascending id order straight from the slot order with one
//     block-wide scan. If the check fails it runs an exact pass over the whole row instead.
#include "device_common.h"
#include "indexer_common.h"
#include "launch.h"
#include "topk_common.h"
#include "topk_finish.h"
#include "topk_short.h"

namespace csl {

namespace {

// ---------------------------------------------------------------------------------------
// Long rows: slice candidates, then one finishing workgroup per row.
// ---------------------------------------------------------------------------------------
__global__ __launch_bounds__(kSlice) void topk_prepare_kernel(const float* __restrict__ scores, int64_t ld,
                                                               const int64_t* __restrict__ ent_off,
                                                               const int64_t* __restrict__ q_pos, int m, int T, int k,
                                                               int64_t max_entries, void* ws, int budget) {
  __shared__ SliceScratch sc;
  const int row = blockIdx.y;
  const int b = row / T, t = row % T;
  const int64_t n = visible_entries(ent_off, q_pos, b, t, m, max_entries);
  if (n <= k || topk_row_dense(n, k)) return;  // the finishing kernel selects everything / searches the row
  const int64_t lo = (int64_t)blockIdx.x * kSlice;
  if (lo >= n) return;
  const int64_t i = lo + threadIdx.x;
  const uint32_t x = (i < n) ? score_key(scores[(int64_t)row * ld + i]) : 0u;
  const TopkRowWs rw = topk_row_ws(ws, row, max_entries, budget);
  const int R = topk_row_slots(n, max_entries, budget);
  slice_candidates(x, slice_quota(n, k, R), topk_wave_list(n, k), R, sc, lo, &rw.cuts[blockIdx.x],
                   rw.slots + (int64_t)blockIdx.x * R);
}

constexpr int kFinNT = 1024;
constexpr int kFinWaves = kFinNT / kWave;

// ---------------------------------------------------------------------------------------
// Short rows: one workgroup per row, keys in registers (element i = j * kFinNT + tid).
// Radix select of the keep-th largest 32-bit key, first on the 11 bits just below the keys'
// common prefix, then on the rest; winners are the keys above the threshold bin plus, when
// the bin is not taken whole, the first `need` keys equal to the threshold in id order. The
// winners are written in id order through one packed block scan of per-(item, wave) counts.
// ---------------------------------------------------------------------------------------
// fin_threshold over COPIES interleaved copies of a 2048-bin histogram (hist[bin * COPIES +
// copy]), summed per bin: lanes spread their atomics over the copies, so keys that pile into a
// few bins do not serialise a whole wave on one LDS address.
template <int COPIES>
__device__ __forceinline__ void fin_threshold_copies(const uint32_t* hist, uint32_t need, uint32_t* wsum,
                                                     uint32_t* res) {
  constexpr int BINS = 2048;
  constexpr int PER = BINS / kFinNT;
  const int tid = threadIdx.x;
  uint32_t v[PER];
  uint32_t local = 0;
#pragma unroll
  for (int q = 0; q < PER; ++q) {
    const int bin = BINS - 1 - (tid * PER + q);
    uint32_t x = 0;
#pragma unroll
    for (int c = 0; c < COPIES; ++c) x += hist[bin * COPIES + c];
    v[q] = x;
    local += x;
  }
  const uint32_t incl = wave_incl_scan(local);
  if (lane_id() == kWave - 1) wsum[tid / kWave] = incl;
  __syncthreads();
  uint32_t before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < kFinWaves; ++w) {
    const uint32_t x = wsum[w];
    before += (w < tid / kWave) ? x : 0u;
    all += x;
  }
  uint32_t excl = before + incl - local;
#pragma unroll
  for (int q = 0; q < PER; ++q) {
    if (excl < need && need <= excl + v[q]) {
      res[0] = (uint32_t)(BINS - 1 - (tid * PER + q));
      res[1] = excl;
      res[2] = v[q];
    }
    excl += v[q];
  }
  if (tid == 0) res[3] = all;
  __syncthreads();
}

template <int ITEMS>
__global__ __launch_bounds__(kFinNT) void topk_row_kernel(const float* __restrict__ scores, int64_t ld,
                                                          const int64_t* __restrict__ ent_off,
                                                          const int64_t* __restrict__ q_pos, int m, int T, int k,
                                                          int64_t max_entries, int32_t* __restrict__ idx) {
  constexpr int COPIES = 8;  // first-pass histogram copies (lane % COPIES)
  __shared__ uint32_t hist_a[2048 * COPIES];
  __shared__ uint32_t hist_b[2048];
  __shared__ uint32_t hist_c[1024];
  __shared__ uint32_t wsum[2 * kFinWaves];
  __shared__ uint32_t res[4];
  __shared__ uint32_t cnt[ITEMS * kFinWaves];

  const int row = blockIdx.x;
  const int b = row / T, t = row % T;
  const int tid = threadIdx.x;
  const int wave = tid / kWave;
  const int64_t n = visible_entries(ent_off, q_pos, b, t, m, max_entries);
  const uint32_t keep = (uint32_t)(n < k ? n : k);
  int32_t* out = idx + (int64_t)row * k;
  const float* srow = scores + (int64_t)row * ld;
  if ((int64_t)keep == n) {  // everything visible is selected
    for (int p = tid; p < k; p += kFinNT) out[p] = p < n ? p : -1;
    return;
  }

  // loads from a clamped index (no branch per load, so all of them are in flight together),
  // then the entries past the row are masked to 0 (keys of real scores are never 0)
  uint32_t key[ITEMS];
#pragma unroll
  for (int j = 0; j < ITEMS; ++j) {
    const int i = j * kFinNT + tid;
    key[j] = score_key(srow[i < n ? i : n - 1]);
  }
#pragma unroll
  for (int j = 0; j < ITEMS; ++j)
    if (j * kFinNT + tid >= n) key[j] = 0u;
  for (int q = tid; q < 2048 * COPIES; q += kFinNT) hist_a[q] = 0;
  for (int q = tid; q < 2048; q += kFinNT) hist_b[q] = 0;
  hist_c[tid] = 0;
  uint32_t kmin = 0xffffffffu, kmax = 0u;
#pragma unroll
  for (int j = 0; j < ITEMS; ++j)
    if (key[j]) {
      kmin = min(kmin, key[j]);
      kmax = max(kmax, key[j]);
    }
  kmin = wave_min_u32(kmin);
  kmax = wave_max_u32(kmax);
  if (lane_id() == 0) {
    wsum[wave] = kmin;
    wsum[kFinWaves + wave] = kmax;
  }
  __syncthreads();
#pragma unroll
  for (int w = 0; w < kFinWaves; ++w) {
    kmin = min(kmin, wsum[w]);
    kmax = max(kmax, wsum[kFinWaves + w]);
  }
  const int common = __clz(kmin ^ kmax);
  int shift = common >= 21 ? 0 : 21 - common;
  uint32_t need = keep;
  const uint32_t copy = lane_id() % COPIES;
#pragma unroll
  for (int j = 0; j < ITEMS; ++j)
    if (key[j]) atomicAdd(&hist_a[((key[j] >> shift) & 2047u) * COPIES + copy], 1u);
  __syncthreads();
  fin_threshold_copies<COPIES>(hist_a, need, wsum, res);
  uint32_t prefix = ((shift < 21 ? (kmin >> shift) : 0u) & ~2047u) | res[0];
  need -= res[1];
  bool all_in = res[2] == need;
  if (!all_in && shift > 0) {
    const int wb = shift < 11 ? shift : 11;
    const int sb = shift - wb;
#pragma unroll
    for (int j = 0; j < ITEMS; ++j)
      if (key[j] && (key[j] >> shift) == prefix) atomicAdd(&hist_b[(key[j] >> sb) & ((1u << wb) - 1u)], 1u);
    __syncthreads();
    fin_threshold<kFinNT, 2048>(hist_b, need, wsum, res);
    prefix = (prefix << wb) | res[0];
    shift = sb;
    need -= res[1];
    all_in = res[2] == need;
    if (!all_in && shift > 0) {  // shift <= 10 here
#pragma unroll
      for (int j = 0; j < ITEMS; ++j)
        if (key[j] && (key[j] >> shift) == prefix) atomicAdd(&hist_c[key[j] & ((1u << shift) - 1u)], 1u);
      __syncthreads();
      fin_threshold<kFinNT, 1024>(hist_c, need, wsum, res);
      prefix = (prefix << shift) | res[0];
      shift = 0;
      need -= res[1];
      all_in = res[2] == need;
    }
  }
  const uint32_t need_eq = all_in ? 0u : need;

  // ordered output: per (item, wave) counts of keys above the threshold and tied with it
  // (id order is item, then wave, then lane). Each count is a ballot and a popcount; lane j
  // of the wave collects item j's count branch-free and the wave posts them with one store
  // per lane. Tied keys are rare (the threshold key itself), so their ballots run only in
  // waves that hold one.
  auto above = [&](uint32_t x) {
    const uint32_t h = x >> shift;
    return x != 0u && (h > prefix || (all_in && h == prefix));
  };
  auto tied = [&](uint32_t x) { return x != 0u && !all_in && (x >> shift) == prefix; };
  static_assert(ITEMS <= kWave, "one item count per lane");
  const int lane = (int)lane_id();
  bool my_tied = false;
#pragma unroll
  for (int j = 0; j < ITEMS; ++j) my_tied |= tied(key[j]);
  const bool wave_tied = __ballot(my_tied) != 0ull;  // wave-uniform
  {
    uint32_t mycnt = 0u;  // lane j: (above | tied << 16) count of item j in this wave
#pragma unroll
    for (int j = 0; j < ITEMS; ++j) {
      uint32_t c = (uint32_t)__popcll(__ballot(above(key[j])));
      if (wave_tied) c |= (uint32_t)__popcll(__ballot(tied(key[j]))) << 16;
      mycnt = (lane == j) ? c : mycnt;
    }
    if (lane < ITEMS) cnt[lane * kFinWaves + wave] = mycnt;
  }
  __syncthreads();
  {
    constexpr int NC = ITEMS * kFinWaves;
    static_assert(NC <= kFinNT, "one count per thread");
    const uint32_t v = (tid < NC) ? cnt[tid] : 0u;
    const uint32_t incl = wave_incl_scan(v);
    if (lane_id() == kWave - 1) wsum[wave] = incl;
    __syncthreads();
    uint32_t before = 0;
#pragma unroll
    for (int w = 0; w < kFinWaves; ++w) before += (w < wave) ? wsum[w] : 0u;
    if (tid < NC) cnt[tid] = before + incl - v;  // exclusive prefix of (gt | eq << 16)
    __syncthreads();
  }
  // lane j holds item j's base for this wave; each item reads it with one lane read
  const uint32_t mybase = (lane < ITEMS) ? cnt[lane * kFinWaves + wave] : 0u;
#pragma unroll
  for (int j = 0; j < ITEMS; ++j) {
    const uint32_t base = __builtin_amdgcn_readlane(mybase, j);
    const bool g = above(key[j]);
    const uint64_t gm = __ballot(g);
    const uint32_t gb = (base & 0xffffu) + rank_in_wave(gm);
    const int i = j * kFinNT + tid;
    if (wave_tied) {
      const bool e = tied(key[j]);
      const uint64_t em = __ballot(e);
      const uint32_t eb = (base >> 16) + rank_in_wave(em);
      if (g) out[gb + min(eb, need_eq)] = i;
      else if (e && eb < need_eq) out[gb + eb] = i;
    } else if (g) {
      out[gb + min(base >> 16, need_eq)] = i;  // no tied key in this wave: every earlier tie is before
    }
  }
  for (int p = (int)keep + tid; p < k; p += kFinNT) out[p] = -1;
}

// Scores on demand: the scores of entries [e0, min(e0 + 64, n)) of sequence b's one query row,
// recomputed by one wave with the decode indexer's loads, tile arithmetic (decode_score_tile)
// and LDS staging (64 floats of the wave's own), so each score has the indexer's bits. The
// query operand holds row 0 only: the lists exist only for one query row per sequence.
template <int HI, int KT>
__device__ __forceinline__ void rescore_wave_hk(const RescoreIn& rs, const int64_t* __restrict__ ent_off, int b,
                                                int64_t e0, int64_t n, float* __restrict__ srow, float* stage) {
  const int lane = threadIdx.x % kWave;
  const int g = lane / 16, c = lane % 16;
  const int64_t e_base = ent_off[b];
  const float* k_scale = static_cast<const float*>(rs.k_scale);
  const uint8_t* k_mx = static_cast<const uint8_t*>(rs.k_scale);
  const uint16_t* q16 = static_cast<const uint16_t*>(rs.qI);
  // B operand: column c is head c % HI of query row c / HI, and only row 0 exists
  const bool row0 = c / HI == 0;
  bf16x8 qb[2];
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) {
    u32x4 v = u32x4{0, 0, 0, 0};
    if (row0) v = *reinterpret_cast<const u32x4*>(q16 + ((int64_t)b * HI + c % HI) * 64 + kslot_dim<KT>(kk, g));
    qb[kk] = as_bf16x8(v);
  }
  const float wc = row0 ? rs.w[(int64_t)b * HI + c % HI] : 0.f;
  const bool writer = (c % HI) == 0 && row0;
  const int64_t e_end = e0 + kWave < n ? e0 + kWave : n;
  u32x4 kb[4][2];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int64_t s = e0 + u * 16 + c;
    load_key_tile<KT>(rs.kI, k_mx, e_base + s, s < e_end, g, kb[u][0], kb[u][1]);
  }
  float my_scale = 1.f;
  if (KT == kKeyFP8 && e0 + lane < e_end)
    my_scale = k_scale[fp8_scale_index<false>(PagedView{}, 0, rs.scale_off, b, e0 + lane, rs.scale_group)];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    float v[4];
    decode_score_tile<HI, KT>(kb[u][0], kb[u][1], qb, wc, v);
    if (writer) *reinterpret_cast<float4*>(&stage[u * 16 + 4 * g]) = make_float4(v[0], v[1], v[2], v[3]);
  }
  // each wave reads back only what it wrote: LDS operations of one wave complete in order
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  const float val = stage[lane] * my_scale;
  if (e0 + lane < n) srow[e0 + lane] = val;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// finish_row's Repair for scores on demand: each wave recomputes with its own 64 floats of LDS
struct RescoreRepair {
  static constexpr bool kActive = true;
  RescoreIn rs;
  const int64_t* ent_off;
  int b;
  float* srow;
  float* stage;  // 64 floats per wave
  __device__ __forceinline__ void wave(int64_t e0, int64_t n) const {
    float* st = stage + (threadIdx.x / kWave) * kWave;
#define CSL_RESCORE(H, KT) \
  case (KT) * 32 + (H): rescore_wave_hk<H, KT>(rs, ent_off, b, e0, n, srow, st); break;
    switch (rs.key_type * 32 + rs.HI) {
      CSL_RESCORE(1, kKeyBF16) CSL_RESCORE(2, kKeyBF16) CSL_RESCORE(4, kKeyBF16) CSL_RESCORE(8, kKeyBF16)
      CSL_RESCORE(16, kKeyBF16) CSL_RESCORE(1, kKeyFP8) CSL_RESCORE(2, kKeyFP8) CSL_RESCORE(4, kKeyFP8)
      CSL_RESCORE(8, kKeyFP8) CSL_RESCORE(16, kKeyFP8) CSL_RESCORE(1, kKeyFP4) CSL_RESCORE(2, kKeyFP4)
      CSL_RESCORE(4, kKeyFP4) CSL_RESCORE(8, kKeyFP4) CSL_RESCORE(16, kKeyFP4)
      default: break;
    }
#undef CSL_RESCORE
  }
};

// One workgroup of NT threads per row finishes the selection from the row's candidate lists
// (topk_finish.h); thread i owns CH consecutive chunks of 8 slots. RESCORE: the indexer
// kept no scores for list rows (scores on demand), and a row whose lists cannot prove its
// selection has them recomputed first.
template <int NT, int CH, bool RESCORE>
__global__ __launch_bounds__(NT) void topk_finish_kernel(float* __restrict__ scores, int64_t ld,
                                                             const int64_t* __restrict__ ent_off,
                                                             const int64_t* __restrict__ q_pos, int m, int T, int k,
                                                             int64_t max_entries, int32_t* __restrict__ idx, void* ws,
                                                             int budget, RescoreIn rs) {
  __shared__ FinishLds<NT> lds;
  __shared__ __align__(16) float stage[RESCORE ? NT : 1];
  const int row = blockIdx.x;
  const int b = row / T, t = row % T;
  const TopkRowWs rw = topk_row_ws(ws, row, max_entries, budget);
  float* srow = scores + (int64_t)row * ld;
  if constexpr (RESCORE) {
    finish_row<NT, CH>(srow, rw, [&] { return visible_entries(ent_off, q_pos, b, t, m, max_entries); },
                           max_entries, budget, k, idx + (int64_t)row * k, lds,
                           RescoreRepair{rs, ent_off, b, srow, stage});
  } else {
    finish_row<NT, CH>(srow, rw, [&] { return visible_entries(ent_off, q_pos, b, t, m, max_entries); },
                           max_entries, budget, k, idx + (int64_t)row * k, lds);
  }
}

template <int ITEMS>
hipError_t launch_row(const float* scores, int64_t ld, const int64_t* ent_off, const int64_t* q_pos, int m, int B,
                      int T, int k, int64_t max_entries, int32_t* idx, hipStream_t st) {
  topk_row_kernel<ITEMS><<<dim3((unsigned)(B * T)), 1024, 0, st>>>(scores, ld, ent_off, q_pos, m, T, k, max_entries, idx);
  return hipGetLastError();
}

}  // namespace

bool topk_uses_row_kernel(int64_t max_entries) { return max_entries <= kRowKernelMax; }

int64_t topk_max_entries() { return kMultiMaxEntries; }

size_t topk_workspace_bytes(int B, int T, int64_t max_entries, int k) {
  if (topk_uses_row_kernel(max_entries) || max_entries <= k || max_entries > kMultiMaxEntries) return 0;
  return (size_t)B * T * topk_row_stride(max_entries, topk_slot_budget(max_entries, k));
}

int topk_max_k() { return kTopkMaxK; }

bool topk_finish_can_rescore(int64_t max_entries, int k) {
  if (topk_uses_row_kernel(max_entries) || max_entries <= k || max_entries > kMultiMaxEntries) return false;
  return topk_num_slices(max_entries) * topk_slot_budget(max_entries, k) / 8 <= kFinNT;
}

hipError_t launch_topk(const float* scores, int64_t ld, const int64_t* ent_off, const int64_t* q_pos, int m, int B,
                       int T, int k, int64_t max_entries, int32_t* idx, void* ws, bool prepared, hipStream_t st,
                       const RescoreIn* rescore) {
  if (topk_uses_row_kernel(max_entries)) {
    if (max_entries <= 1024) return launch_row<1>(scores, ld, ent_off, q_pos, m, B, T, k, max_entries, idx, st);
    if (max_entries <= 4096) return launch_row<4>(scores, ld, ent_off, q_pos, m, B, T, k, max_entries, idx, st);
    if (max_entries <= 16384) return launch_row<16>(scores, ld, ent_off, q_pos, m, B, T, k, max_entries, idx, st);
    return launch_row<34>(scores, ld, ent_off, q_pos, m, B, T, k, max_entries, idx, st);
  }
  const int rows = B * T;
  const int budget = topk_slot_budget(max_entries, k);
  if (!prepared) {
    dim3 grid((unsigned)topk_num_slices(max_entries), (unsigned)rows);
    topk_prepare_kernel<<<grid, kSlice, 0, st>>>(scores, ld, ent_off, q_pos, m, T, k, max_entries, ws, budget);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  // chunks of 8 slots, CH per thread
  const int64_t chunks = topk_num_slices(max_entries) * budget / 8;
  const dim3 fg((unsigned)rows);
  float* sc = const_cast<float*>(scores);  // written only by the recomputing instance
  const RescoreIn none{};
  // rows of at most 2 * 512 chunks (8,192 slots): 512 threads with two chunks each. A
  // 1,024-thread workgroup needs most of a compute unit's wave slots and registers at once, so
  // beside other kernels' workgroups (decode steps of several micro-batches in flight) it waited
  // for a whole compute unit to drain; the 512-thread one starts sooner there (in-flight steps
  // 27.6 -> 26.9 us at 1M context) at ~1 us more on its own (256 threads: slower both ways)
  constexpr int NS = 512;
  if (rescore) {
    if (!prepared || T != 1 || chunks > 2 * NS) return hipErrorInvalidValue;
    topk_finish_kernel<NS, 2, true><<<fg, NS, 0, st>>>(sc, ld, ent_off, q_pos, m, T, k, max_entries, idx, ws, budget,
                                                       *rescore);
  } else if (chunks <= 2 * NS) {
    topk_finish_kernel<NS, 2, false><<<fg, NS, 0, st>>>(sc, ld, ent_off, q_pos, m, T, k, max_entries, idx, ws, budget,
                                                        none);
  } else if (chunks <= 2 * kFinNT) {
    topk_finish_kernel<kFinNT, 2, false><<<fg, kFinNT, 0, st>>>(sc, ld, ent_off, q_pos, m, T, k, max_entries, idx, ws,
                                                                budget, none);
  } else {  // at most kMaxRowSlots / 8 = 4 * kFinNT chunks
    topk_finish_kernel<kFinNT, 4, false><<<fg, kFinNT, 0, st>>>(sc, ld, ent_off, q_pos, m, T, k, max_entries, idx, ws,
                                                                budget, none);
  }
  return hipGetLastError();
}

}  // namespace csl
