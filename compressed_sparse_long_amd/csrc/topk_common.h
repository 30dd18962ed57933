// Pieces of the top-k selection shared by the indexer (which can leave per-row candidate
// lists behind) and the top-k kernels: wave and block scans, radix threshold search, and the
// per-slice candidate lists.
//
// Slice candidates. A row of n scores is cut into slices of 512 consecutive entries. Every
// slice writes, with plain stores and no atomics, its cut -- a key value such that every entry
// of the slice whose key reaches the cut is listed -- and at most 16 listed (key << 32 | id)
// pairs, in ascending id order, into its own slots (0 marks an empty slot). The cut comes from
// two levels of order statistics taken with wave ballots: each wave of 64 entries keeps its 8
// largest keys, and one wave keeps the `quota` largest of those 64 (quota is 8..16, six times
// the slice's expected share of the k winners). Each level's cut is the r-th largest key or a
// bit prefix of it that already admits exactly r keys, and a value that ties across the
// boundary is dropped, so the lists stay honest. When the k-th largest listed key is at least
// every slice's cut, the k best listed entries are exactly the k best of the row: every entry
// left out lies strictly below its slice's cut. The finishing step checks that and searches
// the whole row otherwise; a slice holds 12 or more of the k winners when it expects two with
// probability ~1.4e-6.
#pragma once

#include "device_common.h"

namespace csl {

constexpr int kSlice = 512;        // entries per slice (one decode indexer workgroup)
constexpr int kSliceSlots = 16;    // listed candidates per slice at most
constexpr int kWaveList = 8;       // largest keys kept per wave of 64 entries
constexpr int kMultiMaxEntries = 1 << 20;  // longest row of the multi-workgroup path
constexpr int kTopkMaxK = 4096;
constexpr int kRowKernelMax = 40 * 1024;   // rows up to this length use one workgroup

__host__ __device__ inline int64_t topk_num_slices(int64_t entries) { return (entries + kSlice - 1) / kSlice; }

// per-row workspace: the cut of every slice (padded to 256 bytes), then kSliceSlots slots per slice
__host__ __device__ inline size_t topk_cuts_bytes(int64_t max_entries) {
  return ((size_t)topk_num_slices(max_entries) * 4 + 255) & ~(size_t)255;
}
__host__ __device__ inline size_t topk_row_stride(int64_t max_entries) {
  return topk_cuts_bytes(max_entries) + (size_t)topk_num_slices(max_entries) * kSliceSlots * 8;
}

struct TopkRowWs {
  uint32_t* cuts;
  uint64_t* slots;
};

__device__ __forceinline__ TopkRowWs topk_row_ws(void* ws, int64_t row, int64_t max_entries) {
  char* base = static_cast<char*>(ws) + (size_t)row * topk_row_stride(max_entries);
  TopkRowWs r;
  r.cuts = reinterpret_cast<uint32_t*>(base);
  r.slots = reinterpret_cast<uint64_t*>(base + topk_cuts_bytes(max_entries));
  return r;
}

// entries a slice aims to list: ~6x its expected share of the k winners, within [8, 16]
__device__ __forceinline__ int slice_quota(int64_t n, int k) {
  int64_t q = (6 * (int64_t)k * kSlice + n - 1) / (n > 0 ? n : 1);
  if (q < kWaveList) q = kWaveList;
  if (q > kSliceSlots) q = kSliceSlots;
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

// A threshold t with at least r lanes holding x >= t (r >= 1), found bit by bit from ballot
// counts: the r-th largest x of the wave, or -- as soon as a prefix of it already has exactly
// r lanes at or above it -- that prefix (every x >= t is then among those r). Wave-uniform.
__device__ __forceinline__ uint32_t wave_rth_threshold(uint32_t x, int r) {
  uint32_t t = 0;
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t c = t | (1u << bit);
    const int n = (int)__popcll(__ballot(x >= c));
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

static_assert(kSlice / kWave * kWaveList == kWave, "the wave lists of a slice fill one wave");
static_assert(kSliceSlots <= kWave, "one wave writes the slice's slots");

// LDS scratch of slice_candidates: every wave's list and cut
struct SliceScratch {
  uint32_t key[kSlice / kWave][kWaveList];
  uint32_t off[kSlice / kWave][kWaveList];
  uint32_t cut[kSlice / kWave];
};

// Write one slice's honest cut and its listed (key << 32 | id) pairs in ascending id order,
// empty slots as 0. Called by all kSlice threads of a workgroup; thread i holds the key x of
// the slice's entry i (0 for no entry; keys of real scores are never 0), whose id is
// id_base + i. Contains one workgroup barrier; only wave 0 writes.
__device__ __forceinline__ void slice_candidates(uint32_t x, int quota, SliceScratch& sc, int64_t id_base,
                                                 uint32_t* cut_out, uint64_t* slots_out) {
  const int lane = (int)lane_id();
  const int wave = threadIdx.x / kWave;
  // level 1: the wave's kWaveList largest keys; all of the wave's entries at or above th are listed
  uint32_t th = wave_rth_threshold(x, kWaveList);
  uint64_t mk = __ballot(x != 0u && x >= th);
  if (__popcll(mk) > kWaveList) {  // a tie across the boundary: list only the keys above it
    th += 1u;
    mk = __ballot(x >= th);
  }
  if ((mk >> lane) & 1ull) {
    const uint32_t r = rank_in_wave(mk);
    sc.key[wave][r] = x;
    sc.off[wave][r] = (uint32_t)threadIdx.x;
  }
  const int cw = __popcll(mk);
  if (lane >= cw && lane < kWaveList) sc.key[wave][lane] = 0u;
  if (lane == 0) sc.cut[wave] = th;
  __syncthreads();
  if (wave != 0) return;
  // level 2: the quota largest of the wave lists, and never below a wave's own cut
  const uint32_t y = sc.key[lane / kWaveList][lane % kWaveList];
  const uint32_t yo = sc.off[lane / kWaveList][lane % kWaveList];
  uint32_t cut = wave_rth_threshold(y, quota);
#pragma unroll
  for (int w = 0; w < kSlice / kWave; ++w) cut = max(cut, sc.cut[w]);
  uint64_t ms = __ballot(y != 0u && y >= cut);
  if (__popcll(ms) > kSliceSlots) {
    cut += 1u;
    ms = __ballot(y >= cut);
  }
  const int cnt = __popcll(ms);
  if ((ms >> lane) & 1ull) slots_out[rank_in_wave(ms)] = ((uint64_t)y << 32) | (uint32_t)(id_base + yo);
  if (lane >= cnt && lane < kSliceSlots) slots_out[lane] = 0ull;
  if (lane == 0) *cut_out = cut;
}

}  // namespace csl
