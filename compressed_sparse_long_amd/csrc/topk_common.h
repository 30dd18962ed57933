// Pieces of the top-k selection shared by the indexer (which can leave per-row candidate
// lists behind) and the top-k kernels: wave and block scans, radix threshold search, and the
// per-slice candidate lists.
//
// Slice candidates. A row of n scores is cut into slices of 512 consecutive entries. Every
// slice writes, with plain stores and no atomics, its cut -- a key value such that every entry
// of the slice whose key reaches the cut is listed -- and at most R listed (key << 32 | id)
// pairs, in ascending id order, into its own R slots (0 marks an empty slot). A row's slot
// budget is 16..64 per slice of the longest row of the call (about six times such a slice's
// expected share of the winners), and a shorter row gives each of its slices up to 64. The
// cut comes from two levels of order statistics taken
// with wave ballots: each wave of 64 entries keeps its 8 (or, where a wave expects more than
// 3/4 of a winner, 16) largest keys, and one wave keeps the `quota` largest of those (quota is
// 8..R, six times the slice's expected share of the k winners). Each level's cut is the r-th
// largest key or a bit prefix of it that already admits exactly r keys, and a value that ties
// across the boundary is dropped, so the lists stay honest. When the k-th largest listed key
// is at least every slice's cut, the k best listed entries are exactly the k best of the row:
// every entry left out lies strictly below its slice's cut. The finishing step checks that and
// searches the whole row otherwise; at 1M context a slice holds 12 or more of the k winners
// when it expects two with probability ~1.4e-6 (smaller slices would need a larger multiple
// of their expected share: the tail of a small count is fatter). Rows with more than 5
// expected winners per wave of 64 skip the lists.
#pragma once

#include "device_common.h"

namespace csl {

constexpr int kSlice = 512;        // entries per slice (one decode indexer workgroup)
constexpr int kMinSliceSlots = 16; // slots per slice of the longest row, at least
constexpr int kMaxSliceSlots = 64; // slots one slice may take
constexpr int kWaveListMax = 16;   // largest keys kept per wave of 64 entries, at most
constexpr int kMultiMaxEntries = 1 << 20;  // longest row of the multi-workgroup path
constexpr int kTopkMaxK = 4096;
constexpr int kRowKernelMax = 34 * 1024;   // rows up to this length use one workgroup (34 keys per thread)

__host__ __device__ inline int64_t topk_num_slices(int64_t entries) { return (entries + kSlice - 1) / kSlice; }

constexpr int64_t kMaxRowSlots = 32768;    // slots per row at most (4 x 8 per finishing thread)

// slots per slice of the longest row of a call: the power of two in [16, 64] at or above six
// times a slice's expected share of the k winners, within kMaxRowSlots per row
__host__ __device__ inline int topk_slot_budget(int64_t max_entries, int k) {
  const int64_t want = (6 * (int64_t)k * kSlice + max_entries - 1) / (max_entries > 0 ? max_entries : 1);
  const int64_t ns = topk_num_slices(max_entries);
  int R = kMinSliceSlots;
  while (R < kMaxSliceSlots && R < want && ns * 2 * R <= kMaxRowSlots) R *= 2;
  return R;
}

// per-row workspace: the cut of every slice (padded to 256 bytes), then the slots of the
// longest row's layout (budget = topk_slot_budget(max_entries, k), computed on the host and
// handed to the kernels)
__host__ __device__ inline size_t topk_cuts_bytes(int64_t max_entries) {
  return ((size_t)topk_num_slices(max_entries) * 4 + 255) & ~(size_t)255;
}
__host__ __device__ inline size_t topk_row_stride(int64_t max_entries, int budget) {
  return topk_cuts_bytes(max_entries) + (size_t)topk_num_slices(max_entries) * budget * 8;
}

struct TopkRowWs {
  uint32_t* cuts;
  uint64_t* slots;
};

__device__ __forceinline__ TopkRowWs topk_row_ws(void* ws, int64_t row, int64_t max_entries, int budget) {
  char* base = static_cast<char*>(ws) + (size_t)row * topk_row_stride(max_entries, budget);
  TopkRowWs r;
  r.cuts = reinterpret_cast<uint32_t*>(base);
  r.slots = reinterpret_cast<uint64_t*>(base + topk_cuts_bytes(max_entries));
  return r;
}

// slots per slice of a row of n entries: the largest of 16, 32, 64 inside the row's budget
// (a shorter row has fewer slices to share it)
__host__ __device__ inline int topk_row_slots(int64_t n, int64_t max_entries, int budget) {
  const int64_t ns = topk_num_slices(n), total = topk_num_slices(max_entries) * budget;
  int R = kMinSliceSlots;
  while (R < kMaxSliceSlots && ns * (2 * R) <= total) R *= 2;
  return R;
}

// keys listed per wave of 64 entries: 16 where a wave expects more than 3/4 of a winner
__host__ __device__ inline int topk_wave_list(int64_t n, int k) { return 4 * 64 * (int64_t)k > 3 * n ? 16 : 8; }

// rows with more than 5 expected winners per wave of 64 are searched whole
__host__ __device__ inline bool topk_row_dense(int64_t n, int k) { return 64 * (int64_t)k > 5 * n; }

// entries a slice aims to list: ~6x its expected share of the k winners, within [8, R]
__device__ __forceinline__ int slice_quota(int64_t n, int k, int R) {
  int64_t q = (6 * (int64_t)k * kSlice + n - 1) / (n > 0 ? n : 1);
  if (q < 8) q = 8;
  if (q > R) q = R;
  return (int)q;
}

__device__ __forceinline__ uint32_t lane_id() { return threadIdx.x % kWave; }

__device__ __forceinline__ uint32_t rank_in_wave(uint64_t mask) {
  const uint32_t l = lane_id();
  const uint64_t below = (l == 0) ? 0ull : (mask & ((~0ull) >> (64 - l)));
  return (uint32_t)__popcll(below);
}

// Inclusive prefix sum over the 64 lanes of a wave: row shifts (DPP) inside each row of 16
// lanes, then the totals of the lower rows read back with readlane.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xf, 0xf, true);  // row_shr:1
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xf, 0xf, true);  // row_shr:2
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xf, 0xf, true);  // row_shr:4
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xf, 0xf, true);  // row_shr:8
  const uint32_t r0 = (uint32_t)__builtin_amdgcn_readlane((int)v, 15);
  const uint32_t r1 = (uint32_t)__builtin_amdgcn_readlane((int)v, 31);
  const uint32_t r2 = (uint32_t)__builtin_amdgcn_readlane((int)v, 47);
  const uint32_t row = lane_id() >> 4;
  return v + (row >= 1 ? r0 : 0u) + (row >= 2 ? r1 : 0u) + (row >= 3 ? r2 : 0u);
}

// Maximum and minimum over the 64 lanes of a wave (wave-uniform results).
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xf, 0xf, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xf, 0xf, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xf, 0xf, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xf, 0xf, false));
  return max(max((uint32_t)__builtin_amdgcn_readlane((int)v, 15), (uint32_t)__builtin_amdgcn_readlane((int)v, 31)),
             max((uint32_t)__builtin_amdgcn_readlane((int)v, 47), (uint32_t)__builtin_amdgcn_readlane((int)v, 63)));
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) { return ~wave_max_u32(~v); }

// A threshold t with at least r of the wave's values x0, x1 (two per lane; pass 0 for an
// unused one) at or above it (r >= 1), found bit by bit from ballot counts: the r-th largest
// value, or -- as soon as a prefix of it already has exactly r values at or above it -- that
// prefix (every value >= t is then among those r). Wave-uniform.
template <bool TWO>
__device__ __forceinline__ uint32_t wave_rth_threshold(uint32_t x0, uint32_t x1, int r) {
  uint32_t t = 0;
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t c = t | (1u << bit);
    int n = (int)__popcll(__ballot(x0 >= c));
    if (TWO) n += (int)__popcll(__ballot(x1 >= c));
    if (n >= r) {
      t = c;
      if (n == r) break;
    }
  }
  return t;
}

// Exclusive prefix sum over a workgroup of NT threads. `wsum` holds >= NT/64 words.
template <int NT>
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, uint32_t* wsum, uint32_t* total) {
  const int lane = lane_id();
  const int wave = threadIdx.x / kWave;
  uint32_t incl = v;
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const uint32_t o = __shfl_up(incl, d, kWave);
    if (lane >= d) incl += o;
  }
  if (lane == kWave - 1) wsum[wave] = incl;
  __syncthreads();
  uint32_t before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < NT / kWave; ++w) {
    const uint32_t x = wsum[w];
    if (w < wave) before += x;
    all += x;
  }
  __syncthreads();
  if (total) *total = all;
  return before + incl - v;
}

template <int NT>
__device__ __forceinline__ uint32_t block_max_u32(uint32_t v, uint32_t* wsum) {
#pragma unroll
  for (int d = 32; d > 0; d >>= 1) v = max(v, (uint32_t)__shfl_xor(v, d, kWave));
  if (lane_id() == 0) wsum[threadIdx.x / kWave] = v;
  __syncthreads();
  uint32_t r = 0;
#pragma unroll
  for (int w = 0; w < NT / kWave; ++w) r = max(r, wsum[w]);
  __syncthreads();
  return r;
}

template <int NT>
__device__ __forceinline__ uint32_t block_min_u32(uint32_t v, uint32_t* wsum) {
#pragma unroll
  for (int d = 32; d > 0; d >>= 1) v = min(v, (uint32_t)__shfl_xor(v, d, kWave));
  if (lane_id() == 0) wsum[threadIdx.x / kWave] = v;
  __syncthreads();
  uint32_t r = 0xffffffffu;
#pragma unroll
  for (int w = 0; w < NT / kWave; ++w) r = min(r, wsum[w]);
  __syncthreads();
  return r;
}

// Scan a histogram (LDS) from its top bin down and find the bin where the running count
// first reaches `need`: out3 = {bin, count strictly above it, count in it}.
template <int NT, int BINS>
__device__ __forceinline__ void find_threshold_bin(const uint32_t* hist, uint32_t need, uint32_t* wsum,
                                                   uint32_t* out3) {
  constexpr int PER = BINS / NT > 0 ? BINS / NT : 1;
  uint32_t v[PER];
  uint32_t local = 0;
#pragma unroll
  for (int q = 0; q < PER; ++q) {
    const int bin = BINS - 1 - ((int)threadIdx.x * PER + q);
    v[q] = (bin >= 0) ? hist[bin] : 0u;
    local += v[q];
  }
  uint32_t excl = block_exclusive_scan<NT>(local, wsum, nullptr);
#pragma unroll
  for (int q = 0; q < PER; ++q) {
    if (excl < need && need <= excl + v[q]) {
      out3[0] = BINS - 1 - ((int)threadIdx.x * PER + q);
      out3[1] = excl;
      out3[2] = v[q];
    }
    excl += v[q];
  }
  __syncthreads();
}

static_assert(kSlice / kWave * kWaveListMax <= 2 * kWave, "the wave lists of a slice fit two values per lane");
static_assert(kMaxSliceSlots <= kWave, "one wave writes the slice's slots");

// LDS scratch of slice_candidates: every wave's list and cut
struct SliceScratch {
  uint32_t key[kSlice / kWave][kWaveListMax];
  uint32_t off[kSlice / kWave][kWaveListMax];
  uint32_t cut[kSlice / kWave];
};

// Write one slice's honest cut and its (at most R) listed (key << 32 | id) pairs in ascending
// id order, empty slots as 0. Called by all kSlice threads of a workgroup; thread i holds the
// key x of the slice's entry i (0 for no entry; keys of real scores are never 0), whose id is
// id_base + i. wl (8 or 16) keys are kept per wave, quota <= R <= 64 per slice. Contains one
// workgroup barrier; only wave 0 writes.
__device__ __forceinline__ void slice_candidates(uint32_t x, int quota, int wl, int R, SliceScratch& sc,
                                                 int64_t id_base, uint32_t* cut_out, uint64_t* slots_out) {
  const int lane = (int)lane_id();
  const int wave = threadIdx.x / kWave;
  // level 1: the wave's wl largest keys; all of the wave's entries at or above th are listed
  uint32_t th = wave_rth_threshold<false>(x, 0u, wl);
  uint64_t mk = __ballot(x != 0u && x >= th);
  if (__popcll(mk) > wl) {  // a tie across the boundary: list only the keys above it
    th += 1u;
    mk = __ballot(x >= th);
  }
  if ((mk >> lane) & 1ull) {
    const uint32_t r = rank_in_wave(mk);
    sc.key[wave][r] = x;
    sc.off[wave][r] = (uint32_t)threadIdx.x;
  }
  const int cw = __popcll(mk);
  if (lane >= cw && lane < wl) sc.key[wave][lane] = 0u;
  if (lane == 0) sc.cut[wave] = th;
  __syncthreads();
  if (wave != 0) return;
  // level 2: the quota largest of the wave lists (entry e = w * wl + j, ne of them; lane holds
  // e = lane and, when ne > 64, e = 64 + lane; lanes past ne hold no entry), and never below a
  // wave's own cut
  const int ne = wl * (kSlice / kWave);
  const bool two = ne > kWave;
  const int e0 = lane < ne ? lane : ne - 1, e1 = lane + kWave < ne ? lane + kWave : ne - 1;
  const uint32_t y0 = lane < ne ? sc.key[e0 / wl][e0 % wl] : 0u, o0 = sc.off[e0 / wl][e0 % wl];
  const uint32_t y1 = two && lane + kWave < ne ? sc.key[e1 / wl][e1 % wl] : 0u, o1 = sc.off[e1 / wl][e1 % wl];
  uint32_t cut = two ? wave_rth_threshold<true>(y0, y1, quota) : wave_rth_threshold<false>(y0, 0u, quota);
#pragma unroll
  for (int w = 0; w < kSlice / kWave; ++w) cut = max(cut, sc.cut[w]);
  uint64_t m0 = __ballot(y0 != 0u && y0 >= cut), m1 = __ballot(y1 != 0u && y1 >= cut);
  if (__popcll(m0) + __popcll(m1) > R) {
    cut += 1u;
    m0 = __ballot(y0 >= cut);
    m1 = __ballot(y1 >= cut);
  }
  const int c0 = __popcll(m0), cnt = c0 + __popcll(m1);
  if ((m0 >> lane) & 1ull) slots_out[rank_in_wave(m0)] = ((uint64_t)y0 << 32) | (uint32_t)(id_base + o0);
  if ((m1 >> lane) & 1ull) slots_out[c0 + rank_in_wave(m1)] = ((uint64_t)y1 << 32) | (uint32_t)(id_base + o1);
  if (lane >= cnt && lane < R) slots_out[lane] = 0ull;
  if (lane == 0) *cut_out = cut;
}

}  // namespace csl
