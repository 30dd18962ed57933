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
#include "launch.h"
#include "topk_common.h"

namespace csl {

namespace {

__device__ __forceinline__ int64_t row_count(const int64_t* ent_off, const int64_t* q_pos, int b, int t, int m,
                                             int64_t max_entries) {
  const int64_t n_ent = ent_off[b + 1] - ent_off[b];
  int64_t n = (q_pos[b] + t) / m;
  n = n < n_ent ? n : n_ent;
  n = n < max_entries ? n : max_entries;
  return n < 0 ? 0 : n;
}

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
  const int64_t n = row_count(ent_off, q_pos, b, t, m, max_entries);
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

// One radix step of the finish: over BINS bins (hist in LDS), find the bin holding the
// need-th largest key counting from the top bin down. res = {bin, count above it, count in
// it, total}. Contains two workgroup barriers; the caller reads res after it returns.
template <int BINS>
__device__ __forceinline__ void fin_threshold(const uint32_t* hist, uint32_t need, uint32_t* wsum, uint32_t* res) {
  constexpr int PER = BINS / kFinNT;
  static_assert(PER * kFinNT == BINS, "bins per thread");
  const int tid = threadIdx.x;
  uint32_t v[PER];
  uint32_t local = 0;
#pragma unroll
  for (int q = 0; q < PER; ++q) {
    v[q] = hist[BINS - 1 - (tid * PER + q)];
    local += v[q];
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
  const int64_t n = row_count(ent_off, q_pos, b, t, m, max_entries);
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
    fin_threshold<2048>(hist_b, need, wsum, res);
    prefix = (prefix << wb) | res[0];
    shift = sb;
    need -= res[1];
    all_in = res[2] == need;
    if (!all_in && shift > 0) {  // shift <= 10 here
#pragma unroll
      for (int j = 0; j < ITEMS; ++j)
        if (key[j] && (key[j] >> shift) == prefix) atomicAdd(&hist_c[key[j] & ((1u << shift) - 1u)], 1u);
      __syncthreads();
      fin_threshold<1024>(hist_c, need, wsum, res);
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

// Exact selection over the whole row from its scores, for rows whose candidate lists cannot
// prove the selection and rows too dense for them. Passes over the row (from L2):
//   1. block min and max of the keys;
//   2. radix select of the keep-th largest key: 11 bits just below the keys' common prefix,
//      then the rest (usually one more pass);
//   3. ordered compaction in chunks of 8 * kFinNT ids with one packed block scan of the
//      (above, tied) counts per chunk, lower ids first among keys tied at the threshold.
// hist_a / hist_b: LDS [2048]; wsum: LDS [2 * kFinWaves]; res: LDS [4].
__device__ void finish_full_row(const float* __restrict__ srow, int64_t n, uint32_t keep, int32_t* __restrict__ out,
                                uint32_t* hist_a, uint32_t* hist_b, uint32_t* wsum, uint32_t* res) {
  const int tid = threadIdx.x;
  const int wave = tid / kWave;
  // visit every key of the row: 16 coalesced loads in flight per thread
  constexpr int U = 16;
  auto for_keys = [&](auto&& fn) {
    for (int64_t c0 = 0; c0 < n; c0 += (int64_t)U * kFinNT) {
      float v[U];
#pragma unroll
      for (int j = 0; j < U; ++j) {
        const int64_t i = c0 + (int64_t)j * kFinNT + tid;
        v[j] = srow[i < n ? i : n - 1];  // clamped: no branch per load
      }
#pragma unroll
      for (int j = 0; j < U; ++j)
        if (c0 + (int64_t)j * kFinNT + tid < n) fn(score_key(v[j]));
    }
  };
  for (int q = tid; q < 2048; q += kFinNT) {
    hist_a[q] = 0;
    hist_b[q] = 0;
  }
  uint32_t kmin = 0xffffffffu, kmax = 0u;
  for_keys([&](uint32_t x) {
    kmin = min(kmin, x);
    kmax = max(kmax, x);
  });
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
  // keys share their top `common` bits: bin the 11 below them first
  const int common = __clz(kmin ^ kmax);
  int shift = common >= 21 ? 0 : 21 - common;
  uint32_t need = keep;
  for_keys([&](uint32_t x) { atomicAdd(&hist_a[(x >> shift) & 2047u], 1u); });
  __syncthreads();
  fin_threshold<2048>(hist_a, need, wsum, res);
  uint32_t prefix = ((shift < 21 ? (kmin >> shift) : 0u) & ~2047u) | res[0];
  need -= res[1];
  bool all_in = res[2] == need;
  uint32_t* hist = hist_b;
  while (!all_in && shift > 0) {
    const int wb = shift < 11 ? shift : 11;
    const int sb = shift - wb;
    for_keys([&](uint32_t x) {
      if ((x >> shift) == prefix) atomicAdd(&hist[(x >> sb) & ((1u << wb) - 1u)], 1u);
    });
    __syncthreads();
    fin_threshold<2048>(hist, need, wsum, res);
    prefix = (prefix << wb) | res[0];
    shift = sb;
    need -= res[1];
    all_in = res[2] == need;
    // the other histogram is free again (its last reads ended before fin_threshold's barriers)
    uint32_t* other = (hist == hist_b) ? hist_a : hist_b;
    for (int q = tid; q < 2048; q += kFinNT) other[q] = 0;
    hist = other;
    __syncthreads();
  }
  const uint32_t need_eq = all_in ? 0u : need;

  constexpr int J = 16;
  uint32_t gbase = 0, ebase = 0;
  for (int64_t c0 = 0; c0 < n; c0 += (int64_t)J * kFinNT) {
    const int64_t i0 = c0 + (int64_t)J * tid;
    uint32_t gm = 0, em = 0;
    float v[J];
#pragma unroll
    for (int j = 0; j < J; ++j) v[j] = srow[i0 + j < n ? i0 + j : n - 1];  // clamped: no branch per load
#pragma unroll
    for (int j = 0; j < J; ++j) {
      if (i0 + j < n) {
        const uint32_t h = score_key(v[j]) >> shift;
        if (h > prefix || (all_in && h == prefix)) gm |= 1u << j;
        else if (h == prefix) em |= 1u << j;
      }
    }
    const uint32_t mine = (uint32_t)__popc(gm) | ((uint32_t)__popc(em) << 16);
    const uint32_t incl = wave_incl_scan(mine);
    if (lane_id() == kWave - 1) wsum[wave] = incl;
    __syncthreads();
    uint32_t before = 0, total = 0;
#pragma unroll
    for (int w = 0; w < kFinWaves; ++w) {
      const uint32_t x = wsum[w];
      before += (w < wave) ? x : 0u;
      total += x;
    }
    __syncthreads();  // wsum is rewritten by the next chunk
    const uint32_t ex = before + incl - mine;
    uint32_t gpos = gbase + (ex & 0xffffu), epos = ebase + (ex >> 16);
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const bool g = (gm >> j) & 1u, e = (em >> j) & 1u;
      if (g) {
        out[gpos + min(epos, need_eq)] = (int32_t)(i0 + j);
        ++gpos;
      } else if (e) {
        if (epos < need_eq) out[gpos + epos] = (int32_t)(i0 + j);
        ++epos;
      }
    }
    gbase += total & 0xffffu;
    ebase += total >> 16;
    if (gbase + min(ebase, need_eq) >= keep) break;  // every winner placed
  }
}

// One workgroup per row. Thread i owns CH consecutive chunks of 8 slots (a slice of the row's
// layout spans R / 8 chunks), so thread order is slot order is id order.
template <int CH>
__global__ __launch_bounds__(kFinNT) void topk_finish_kernel(const float* __restrict__ scores, int64_t ld,
                                                             const int64_t* __restrict__ ent_off,
                                                             const int64_t* __restrict__ q_pos, int m, int T, int k,
                                                             int64_t max_entries, int32_t* __restrict__ idx, void* ws,
                                                             int budget) {
  constexpr int PER = 8;  // slots per chunk
  static_assert(kMinSliceSlots % PER == 0, "a slice spans whole chunks");
  __shared__ uint32_t hist_a[2048];
  __shared__ uint32_t hist_b[2048];
  __shared__ uint32_t hist_c[1024];
  __shared__ uint32_t wsum[3 * kFinWaves];
  __shared__ uint32_t res[4];

  const int row = blockIdx.x;
  const int b = row / T, t = row % T;
  const int tid = threadIdx.x;
  const TopkRowWs rw = topk_row_ws(ws, row, max_entries, budget);
  const int n_chunks = (int)(topk_num_slices(max_entries) * budget / PER);
  // every slot load is issued up front, raw (unpacked only once all of them are out)
  // (a chunk past the row's slots reads the row's first chunk instead, so the loads carry no
  // branches; such a chunk also lies past the row's last slice and is masked below)
  u32x4 raw[CH][PER / 2];
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int j = tid * CH + c;
    const u32x4* src = reinterpret_cast<const u32x4*>(rw.slots + (j < n_chunks ? (int64_t)j * PER : 0));
#pragma unroll
    for (int q = 0; q < PER / 2; ++q) raw[c][q] = src[q];
  }
  // the cut of each chunk's slice for each possible layout (2, 4 or 8 chunks per slice; the
  // row's own layout is known only with n), also issued now and needed only at the end
  const int ns_max = (int)topk_num_slices(max_entries);
  uint32_t cut3[CH][3];
#pragma unroll
  for (int c = 0; c < CH; ++c)
#pragma unroll
    for (int l = 0; l < 3; ++l) cut3[c][l] = rw.cuts[min((tid * CH + c) >> (l + 1), ns_max - 1)];
  const int64_t n = row_count(ent_off, q_pos, b, t, m, max_entries);
  const uint32_t keep = (uint32_t)(n < k ? n : k);
  int32_t* out = idx + (int64_t)row * k;
  for (int q = tid; q < 2048; q += kFinNT) {
    hist_a[q] = 0;
    hist_b[q] = 0;
  }
  hist_c[tid] = 0;

  if ((int64_t)keep == n) {
    for (int p = tid; p < k; p += kFinNT) out[p] = p < n ? p : -1;
    return;
  }
  if (topk_row_dense(n, k)) {
    // winners too dense for candidate lists (more than 5 expected per wave of 64 entries):
    // the lists were not written, search the row directly
    finish_full_row(scores + (int64_t)row * ld, n, keep, out, hist_a, hist_b, wsum, res);
    for (int p = (int)keep + tid; p < k; p += kFinNT) out[p] = -1;
    return;
  }
  const int ns = (int)topk_num_slices(n);
  // chunks per slice in this row's layout: 2, 4 or 8
  const int cps_log2 = __ffs(topk_row_slots(n, max_entries, budget) / PER) - 1;
  uint64_t sl[CH][PER];
#pragma unroll
  for (int c = 0; c < CH; ++c)
#pragma unroll
    for (int q = 0; q < PER / 2; ++q) {
      sl[c][2 * q] = ((uint64_t)raw[c][q].y << 32) | raw[c][q].x;
      sl[c][2 * q + 1] = ((uint64_t)raw[c][q].w << 32) | raw[c][q].z;
    }
  uint32_t key[CH][PER];
  uint32_t kmin = 0xffffffffu, kmax = 0u;
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const bool in = ((tid * CH + c) >> cps_log2) < ns;
#pragma unroll
    for (int q = 0; q < PER; ++q) {
      const uint32_t x = in ? (uint32_t)(sl[c][q] >> 32) : 0u;
      key[c][q] = x;
      if (x) {
        kmin = min(kmin, x);
        kmax = max(kmax, x);
      }
    }
  }
  uint32_t cut[CH];
#pragma unroll
  for (int c = 0; c < CH; ++c)
    cut[c] = cps_log2 == 1 ? cut3[c][0] : (cps_log2 == 2 ? cut3[c][1] : cut3[c][2]);
  const int wave = tid / kWave;
  kmin = wave_min_u32(kmin);
  kmax = wave_max_u32(kmax);
  if (lane_id() == 0) {
    wsum[wave] = kmin;
    wsum[kFinWaves + wave] = kmax;
  }
  __syncthreads();  // histograms cleared, wave extremes posted
#pragma unroll
  for (int w = 0; w < kFinWaves; ++w) {
    kmin = min(kmin, wsum[w]);
    kmax = max(kmax, wsum[kFinWaves + w]);
  }

  // radix select of the keep-th largest listed key. The listed keys share their top
  // L = clz(kmin ^ kmax) bits, so the first pass bins the 11 bits below those (spreading the
  // keys over the bins instead of piling them into a few), the later passes the rest.
  bool ok = true;
  bool all_in = false;
  uint32_t need = keep;
  const int common = __clz(kmin ^ kmax);  // 32 when all keys are equal
  int shift = common >= 21 ? 0 : 21 - common;
  uint32_t prefix;  // value of key >> shift shared by the keys still in play
#pragma unroll
  for (int c = 0; c < CH; ++c)
#pragma unroll
    for (int q = 0; q < PER; ++q)
      if (key[c][q]) atomicAdd(&hist_a[(key[c][q] >> shift) & 2047u], 1u);
  __syncthreads();
  fin_threshold<2048>(hist_a, need, wsum, res);
  if (res[3] < keep) {
    ok = false;  // fewer listed entries than winners
  } else {
    prefix = ((shift < 21 ? (kmin >> shift) : 0u) & ~2047u) | res[0];
    need -= res[1];
    all_in = res[2] == need;
    if (!all_in && shift > 0) {
      const int wb = shift < 11 ? shift : 11;
      const int sb = shift - wb;
#pragma unroll
      for (int c = 0; c < CH; ++c)
#pragma unroll
        for (int q = 0; q < PER; ++q)
          if (key[c][q] && (key[c][q] >> shift) == prefix)
            atomicAdd(&hist_b[(key[c][q] >> sb) & ((1u << wb) - 1u)], 1u);
      __syncthreads();
      fin_threshold<2048>(hist_b, need, wsum, res);
      prefix = (prefix << wb) | res[0];
      shift = sb;
      need -= res[1];
      all_in = res[2] == need;
      if (!all_in && shift > 0) {  // shift <= 10 here
#pragma unroll
        for (int c = 0; c < CH; ++c)
#pragma unroll
          for (int q = 0; q < PER; ++q)
            if (key[c][q] && (key[c][q] >> shift) == prefix)
              atomicAdd(&hist_c[key[c][q] & ((1u << shift) - 1u)], 1u);
        __syncthreads();
        fin_threshold<1024>(hist_c, need, wsum, res);
        prefix = (prefix << shift) | res[0];
        shift = 0;
        need -= res[1];
        all_in = res[2] == need;
      }
    }
  }

  if (ok) {
    // winners: keys above the selected bin, plus (unless the whole bin is taken) the first
    // `need` keys equal to the exact key value, in id order
    const uint32_t lo = prefix << shift;  // lowest key a winner can have
    uint32_t gmask = 0, emask = 0, viol = 0;
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      if (((tid * CH + c) >> cps_log2) < ns && cut[c] > lo) viol = 1;
#pragma unroll
      for (int q = 0; q < PER; ++q) {
        const uint32_t x = key[c][q];
        const uint32_t h = x >> shift;
        const bool g = x != 0u && (h > prefix || (all_in && h == prefix));
        const bool e = x != 0u && !all_in && h == prefix;
        gmask |= (uint32_t)g << (c * PER + q);
        emask |= (uint32_t)e << (c * PER + q);
      }
    }
    // one block scan of (gt count | eq count << 16): a row lists at most 32768 keys
    const uint32_t mine = (uint32_t)__popc(gmask) | ((uint32_t)__popc(emask) << 16);
    const uint32_t incl = wave_incl_scan(mine);
    const bool wviol = __ballot(viol != 0u) != 0ull;
    if (lane_id() == kWave - 1) {
      wsum[wave] = incl;
      wsum[kFinWaves + wave] = wviol ? 1u : 0u;
    }
    __syncthreads();
    uint32_t before = 0, tv = 0;
#pragma unroll
    for (int w = 0; w < kFinWaves; ++w) {
      before += (w < wave) ? wsum[w] : 0u;
      tv |= wsum[kFinWaves + w];
    }
    if (tv != 0u) {
      ok = false;  // a slice may hide a winner below its cut
      __syncthreads();
    } else {
      const uint32_t ex = before + incl - mine;
      uint32_t gpos = ex & 0xffffu, epos = ex >> 16;
      const uint32_t need_eq = all_in ? 0u : need;
      const uint32_t wins = gmask | emask;
#pragma unroll
      for (int c = 0; c < CH; ++c)
#pragma unroll
        for (int q = 0; q < PER; ++q) {
          const int bit = c * PER + q;
          if ((wins >> bit) & 1u) {
            const bool g = (gmask >> bit) & 1u;
            const uint32_t e_before = min(epos, need_eq);
            if (g || epos < need_eq) out[gpos + e_before] = (int32_t)(uint32_t)sl[c][q];
            gpos += g ? 1u : 0u;
            epos += g ? 0u : 1u;
          }
        }
    }
  }
  if (!ok) {
    __syncthreads();  // every thread is done with the histograms and wsum
    finish_full_row(scores + (int64_t)row * ld, n, keep, out, hist_a, hist_b, wsum, res);
  }
  for (int p = (int)keep + tid; p < k; p += kFinNT) out[p] = -1;
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

hipError_t launch_topk(const float* scores, int64_t ld, const int64_t* ent_off, const int64_t* q_pos, int m, int B,
                       int T, int k, int64_t max_entries, int32_t* idx, void* ws, bool prepared, hipStream_t st) {
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
  if (chunks <= kFinNT)
    topk_finish_kernel<1><<<fg, kFinNT, 0, st>>>(scores, ld, ent_off, q_pos, m, T, k, max_entries, idx, ws, budget);
  else if (chunks <= 2 * kFinNT)
    topk_finish_kernel<2><<<fg, kFinNT, 0, st>>>(scores, ld, ent_off, q_pos, m, T, k, max_entries, idx, ws, budget);
  else  // at most kMaxRowSlots / 8 = 4 * kFinNT chunks
    topk_finish_kernel<4><<<fg, kFinNT, 0, st>>>(scores, ld, ent_off, q_pos, m, T, k, max_entries, idx, ws, budget);
  return hipGetLastError();
}

}  // namespace csl
