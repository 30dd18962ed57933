// Pieces of the top-k selection shared by the indexer (which can leave per-row candidate
// lists behind) and the top-k kernels: block scans, radix threshold search, and the
// per-slice candidate cut.
//
// Slice candidates. A row of n scores is cut into slices of S consecutive entries
// (S = 512 for rows up to 2^18 entries, doubling beyond). Every slice writes, with plain
// stores and no atomics, its cut -- a key value such that all of the slice's entries with
// key >= cut are listed -- and up to R = 24 listed (key, id) pairs into its own slots. The
// cut is chosen so that `quota` entries pass (16..20, about 8x the slice's expected share of
// the k winners) but never more than R; it is honest either way. Every entry of the row whose
// key reaches the largest cut of all slices is therefore listed, so whenever at least k listed
// entries reach that largest cut, the k best of them are exactly the k best of the row.
// Otherwise the finishing step searches the whole row. A slice holds 16 or more of the
// k winners when it expects two with probability ~2e-9.
#pragma once

#include "device_common.h"

namespace csl {

constexpr int kSliceMin = 512;                 // slice of the indexer-prepared path (one block)
constexpr int kSliceR = 24;                    // candidate slots per slice
constexpr int kMaxRowSlots = (1 << 18) / kSliceMin * kSliceR;  // 12288 slots per row
constexpr int kMultiMaxEntries = 1 << 20;      // longest row of the multi-workgroup path
constexpr int kTopkMaxK = 4096;
constexpr int kRowKernelMax = 40 * 1024;       // rows up to this length use one workgroup

__host__ __device__ inline int topk_slice_size(int64_t max_entries) {
  int S = kSliceMin;
  while ((max_entries + S - 1) / S * kSliceR > kMaxRowSlots) S *= 2;
  return S;
}
__host__ __device__ inline int64_t topk_num_slices(int64_t entries, int S) { return (entries + S - 1) / S; }

// per-row workspace: cut per slice (padded to 256 bytes), then kSliceR slots per slice
__host__ __device__ inline size_t topk_cuts_bytes(int64_t max_entries) {
  const int64_t ns = topk_num_slices(max_entries, topk_slice_size(max_entries));
  return ((size_t)ns * 4 + 255) & ~(size_t)255;
}
__host__ __device__ inline size_t topk_row_stride(int64_t max_entries) {
  const int64_t ns = topk_num_slices(max_entries, topk_slice_size(max_entries));
  return topk_cuts_bytes(max_entries) + (size_t)ns * kSliceR * 8;
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

// entries a slice of S aims to list: ~8x its expected share of the k winners, within [16, 20]
__device__ __forceinline__ int slice_quota(int64_t n, int k, int S) {
  int64_t q = (8 * (int64_t)k * S + n - 1) / (n > 0 ? n : 1);
  if (q < 16) q = 16;
  if (q > 20) q = 20;
  return (int)q;
}

__device__ __forceinline__ uint32_t lane_id() { return threadIdx.x % kWave; }

__device__ __forceinline__ uint32_t rank_in_wave(uint64_t mask) {
  const uint32_t l = lane_id();
  const uint64_t below = (l == 0) ? 0ull : (mask & ((~0ull) >> (64 - l)));
  return (uint32_t)__popcll(below);
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

// Choose a slice's honest cut (at most kSliceR entries at or above it, about `quota` when
// the keys allow) and write the cut and the listed (key << 32 | id) pairs, empty slots as 0.
// keys: LDS [S], slots [0, nv) valid, slot s is entry id id_base + s. hist: LDS [2048];
// wsum: LDS [NT/64]; res: LDS [4]. Keys of real scores are never 0 (0 marks an empty slot).
template <int NT, int PER>
__device__ void slice_cut_to_slots(const uint32_t* keys, int nv, int64_t id_base, int quota, uint32_t* hist,
                                   uint32_t* wsum, uint32_t* res, uint32_t* cut_out, uint64_t* slots_out) {
  const int tid = threadIdx.x;
  uint32_t cut = 0;
  if (nv > quota) {
    for (int q = tid; q < 2048; q += NT) hist[q] = 0;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int s = j * NT + tid;
      if (s < nv) atomicAdd(&hist[keys[s] >> 21], 1u);
    }
    __syncthreads();
    find_threshold_bin<NT, 2048>(hist, (uint32_t)quota, wsum, res);
    const uint32_t b1 = res[0], above = res[1], inbin = res[2];
    __syncthreads();
    if (above + inbin <= (uint32_t)kSliceR) {
      cut = b1 << 21;
    } else {
      // the coarse bin holds too many: refine inside it on the next 11 key bits
      for (int q = tid; q < 2048; q += NT) hist[q] = 0;
      __syncthreads();
#pragma unroll
      for (int j = 0; j < PER; ++j) {
        const int s = j * NT + tid;
        if (s < nv && (keys[s] >> 21) == b1) atomicAdd(&hist[(keys[s] >> 10) & 2047u], 1u);
      }
      __syncthreads();
      find_threshold_bin<NT, 2048>(hist, (uint32_t)quota - above, wsum, res);
      const uint32_t b2 = res[0], above2 = res[1], inbin2 = res[2];
      __syncthreads();
      cut = (b1 << 21) | (b2 << 10);
      if (above + above2 + inbin2 > (uint32_t)kSliceR) cut += 1u << 10;  // drop the tied bin: fewer, still honest
    }
  }
  uint32_t mine = 0;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int s = j * NT + tid;
    if (s < nv && keys[s] >= cut) ++mine;
  }
  uint32_t total;
  uint32_t pos = block_exclusive_scan<NT>(mine, wsum, &total);
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int s = j * NT + tid;
    if (s < nv && keys[s] >= cut) {
      if (pos < (uint32_t)kSliceR) slots_out[pos] = ((uint64_t)keys[s] << 32) | (uint64_t)(uint32_t)(id_base + s);
      ++pos;
    }
  }
  for (int q = (int)total + tid; q < kSliceR; q += NT) slots_out[q] = 0ull;
  if (tid == 0) *cut_out = cut;
}

}  // namespace csl
