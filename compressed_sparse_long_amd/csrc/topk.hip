// topk_select: the k highest indexer scores of every query row, lower id first on ties,
// written as ascending ids padded with -1 ([P2] "Deep Dive", CSA top-k selection).
//
// Scores are compared through an order-preserving 32-bit key; a tie on the key is broken
// by the lower id, so (key descending, id ascending) is a strict total order and the top-k
// set is unique. Two paths:
//
//   * short rows (n <= 40960, e.g. a 4K-context decode or a prefill chunk over a 131K
//     prefix): one 1024-thread workgroup per row holds the row's keys in registers
//     (element i = j*1024 + tid), radix-selects the k-th best on a 48-bit composite
//     C(i) = key << 16 | (0xffff - i), and writes the selection with a block-wide ordered
//     compaction, so the output is ascending by construction;
//
//   * long rows (decode at 1M context: 262144 scores per row): every slice of the row lists
//     its own candidates above an honest slice cut (topk_common.h) -- either inside
//     indexer_scores, which already holds the scores, or in a prepare kernel here -- and one
//     workgroup per row finishes: it keeps the listed entries whose key reaches the row's
//     largest cut (exactly the row's entries at or above that cut), radix-selects the k
//     best of them with the candidates held in registers, marks the winners in an LDS bitmap
//     of the row and scans it to emit ascending ids. If fewer than k entries reach the cut
//     it runs an exact pass over the whole row instead.
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
// Short rows: one workgroup per row, keys in registers.
// ---------------------------------------------------------------------------------------
template <int ITEMS>
__global__ __launch_bounds__(1024) void topk_row_kernel(const float* __restrict__ scores, int64_t ld,
                                                        const int64_t* __restrict__ ent_off,
                                                        const int64_t* __restrict__ q_pos, int m, int T, int k,
                                                        int64_t max_entries, int32_t* __restrict__ idx) {
  constexpr int NT = 1024;
  constexpr int NW = NT / kWave;
  __shared__ uint32_t hist[2048];
  __shared__ uint32_t wsum[NW];
  __shared__ uint32_t res[4];
  __shared__ uint32_t cnt[ITEMS * NW];

  const int row = blockIdx.x;
  const int b = row / T, t = row % T;
  const int tid = threadIdx.x;
  const int64_t n = row_count(ent_off, q_pos, b, t, m, max_entries);
  const int keep = (int)(n < k ? n : k);
  int32_t* out = idx + (int64_t)row * k;
  const float* srow = scores + (int64_t)row * ld;

  if (keep == n) {  // everything visible is selected
    for (int p = tid; p < k; p += NT) out[p] = p < n ? p : -1;
    return;
  }

  uint32_t key[ITEMS];
#pragma unroll
  for (int j = 0; j < ITEMS; ++j) {
    const int i = j * NT + tid;
    key[j] = (i < n) ? score_key(srow[i]) : 0u;
  }
  auto comp = [&](int j) -> uint64_t {
    const int i = j * NT + tid;
    return ((uint64_t)key[j] << 16) | (uint64_t)(0xffffu - (uint32_t)i);
  };

  uint64_t prefix = 0;
  int pbits = 0;
  uint32_t need = (uint32_t)keep;
  for (int pass = 0; pass < 5; ++pass) {
    const int width = pass < 2 ? 11 : (pass == 2 ? 10 : 8);
    const int shift = 48 - pbits - width;
    for (int q = tid; q < 2048; q += NT) hist[q] = 0;
    __syncthreads();
    for (int j = 0; j < ITEMS; ++j) {
      const int i = j * NT + tid;
      if (i < n) {
        const uint64_t C = comp(j);
        if (pbits == 0 || (C >> (48 - pbits)) == prefix)
          atomicAdd(&hist[(uint32_t)(C >> shift) & ((1u << width) - 1u)], 1u);
      }
    }
    __syncthreads();
    find_threshold_bin<NT, 2048>(hist, need, wsum, res);
    const uint32_t d = res[0], above = res[1], in_bin = res[2];
    prefix = (prefix << width) | d;
    pbits += width;
    need -= above;
    __syncthreads();
    if (in_bin == need) break;  // the whole bin is taken
  }

  // ordered compaction of sel(i) = (C(i) >> (48 - pbits)) >= prefix
  const int wave = tid / kWave;
  for (int j = 0; j < ITEMS; ++j) {
    const int i = j * NT + tid;
    const bool s = (i < n) && ((comp(j) >> (48 - pbits)) >= prefix);
    const uint64_t mask = __ballot(s);
    if (lane_id() == 0) cnt[j * NW + wave] = (uint32_t)__popcll(mask);
  }
  __syncthreads();
  {
    const uint32_t v = (tid < ITEMS * NW) ? cnt[tid] : 0u;
    __syncthreads();
    const uint32_t e = block_exclusive_scan<NT>(v, wsum, nullptr);
    if (tid < ITEMS * NW) cnt[tid] = e;
    __syncthreads();
  }
  for (int j = 0; j < ITEMS; ++j) {
    const int i = j * NT + tid;
    const bool s = (i < n) && ((comp(j) >> (48 - pbits)) >= prefix);
    const uint64_t mask = __ballot(s);
    if (s) {
      const uint32_t pos = cnt[j * NW + wave] + rank_in_wave(mask);
      if (pos < (uint32_t)keep) out[pos] = i;
    }
  }
  for (int p = keep + tid; p < k; p += NT) out[p] = -1;
}

// ---------------------------------------------------------------------------------------
// Long rows: slice candidates, then one finishing workgroup per row.
// ---------------------------------------------------------------------------------------
template <int S>
__global__ __launch_bounds__(256) void topk_prepare_kernel(const float* __restrict__ scores, int64_t ld,
                                                           const int64_t* __restrict__ ent_off,
                                                           const int64_t* __restrict__ q_pos, int m, int T, int k,
                                                           int64_t max_entries, void* ws) {
  __shared__ uint32_t keys[S];
  __shared__ uint32_t hist[2048];
  __shared__ uint32_t wsum[256 / kWave];
  __shared__ uint32_t res[4];
  const int row = blockIdx.y;
  const int b = row / T, t = row % T;
  const int64_t n = row_count(ent_off, q_pos, b, t, m, max_entries);
  if (n <= k) return;  // the finishing kernel selects everything
  const int64_t lo = (int64_t)blockIdx.x * S;
  if (lo >= n) return;
  const float* srow = scores + (int64_t)row * ld;
  const int nv = (int)((n - lo) < S ? (n - lo) : S);
#pragma unroll
  for (int j = 0; j < S / 256; ++j) {
    const int s = j * 256 + threadIdx.x;
    keys[s] = (s < nv) ? score_key(srow[lo + s]) : 0u;
  }
  __syncthreads();
  const TopkRowWs rw = topk_row_ws(ws, row, max_entries);
  slice_cut_to_slots<256, S / 256>(keys, nv, lo, slice_quota(n, k, S), hist, wsum, res, &rw.cuts[blockIdx.x],
                                   rw.slots + (int64_t)blockIdx.x * kSliceR);
}

constexpr int kFinNT = 1024;
constexpr int kFinPer = (kMaxRowSlots + kFinNT - 1) / kFinNT;  // candidate slots per thread
constexpr int kBitmapIds = 1 << 18;  // rows up to this length are ordered through an LDS bitmap

__global__ __launch_bounds__(kFinNT) void topk_finish_kernel(const float* __restrict__ scores, int64_t ld,
                                                             const int64_t* __restrict__ ent_off,
                                                             const int64_t* __restrict__ q_pos, int m, int T, int k,
                                                             int64_t max_entries, int32_t* __restrict__ idx, void* ws) {
  __shared__ uint32_t hist[2048];
  __shared__ uint32_t bitmap[kBitmapIds / 32];  // also the id buffer of very long rows
  __shared__ uint32_t wsum[kFinNT / kWave];
  __shared__ uint32_t res[4];

  const int row = blockIdx.x;
  const int b = row / T, t = row % T;
  const int tid = threadIdx.x;
  const TopkRowWs rw = topk_row_ws(ws, row, max_entries);
  const int S = topk_slice_size(max_entries);
  const int ns_max = (int)topk_num_slices(max_entries, S);
  // every global read is issued up front: row geometry, all slice cuts and all slots (those
  // of slices past this row's length are ignored below)
  const uint32_t my_cut = (tid < ns_max) ? rw.cuts[tid] : 0u;
  uint64_t cv[kFinPer];
#pragma unroll
  for (int q = 0; q < kFinPer; ++q) {
    const int j = q * kFinNT + tid;
    cv[q] = (j < ns_max * kSliceR) ? rw.slots[j] : 0ull;
  }
  const int64_t n = row_count(ent_off, q_pos, b, t, m, max_entries);
  const uint32_t keep = (uint32_t)(n < k ? n : k);
  int32_t* out = idx + (int64_t)row * k;
  const float* srow = scores + (int64_t)row * ld;
  const int words = (int)(n <= kBitmapIds ? (n + 31) / 32 : 0);
  for (int w = tid; w < words; w += kFinNT) bitmap[w] = 0;

  if ((int64_t)keep == n) {
    for (int p = tid; p < k; p += kFinNT) out[p] = p < n ? p : -1;
    return;
  }

  // the listed entries whose key reaches the largest slice cut are exactly the row's entries
  // at or above that cut
  const int ns = (int)topk_num_slices(n, S);
  const uint32_t max_cut = block_max_u32<kFinNT>(tid < ns ? my_cut : 0u, wsum);
  uint32_t vmask = 0, kmax = 0;
#pragma unroll
  for (int q = 0; q < kFinPer; ++q) {
    const int j = q * kFinNT + tid;
    const uint32_t key = (uint32_t)(cv[q] >> 32);
    if (j < ns * kSliceR && key != 0u && key >= max_cut) {
      vmask |= 1u << q;
      kmax = max(kmax, key);
    }
  }
  const uint32_t max_key = block_max_u32<kFinNT>(kmax, wsum);
  const uint32_t range = max_key - max_cut;
  const int start_bit = 32 + (range ? 32 - __clz(range) : 0);
  uint64_t v[kFinPer];  // (max_key - key) << 32 | id: the k smallest are the k best
#pragma unroll
  for (int q = 0; q < kFinPer; ++q) v[q] = ((uint64_t)(max_key - (uint32_t)(cv[q] >> 32)) << 32) | (uint32_t)cv[q];
  bool ok = true;
  uint64_t prefix = 0;
  int pbits = 0;
  {
    uint32_t need = keep;
    while (pbits < start_bit) {
      const int width = (start_bit - pbits) < 11 ? (start_bit - pbits) : 11;
      const int shift = start_bit - pbits - width;
      for (int q = tid; q < 2048; q += kFinNT) hist[q] = 0;
      __syncthreads();
#pragma unroll
      for (int q = 0; q < kFinPer; ++q)
        if (((vmask >> q) & 1u) && (pbits == 0 || (v[q] >> (start_bit - pbits)) == prefix))
          atomicAdd(&hist[2047u - ((uint32_t)(v[q] >> shift) & ((1u << width) - 1u))], 1u);
      __syncthreads();
      if (pbits == 0) {  // total of the first histogram = listed entries at or above max_cut
        uint32_t tot;
        block_exclusive_scan<kFinNT>(hist[2 * tid] + hist[2 * tid + 1], wsum, &tot);
        if (tot < keep) {
          ok = false;
          break;
        }
      }
      find_threshold_bin<kFinNT, 2048>(hist, need, wsum, res);  // top-down over reversed bins
      const uint32_t d = 2047u - res[0], below = res[1], in_bin = res[2];
      prefix = (prefix << width) | d;
      pbits += width;
      need -= below;
      __syncthreads();
      if (in_bin == need) break;
    }
  }

  if (ok && n <= kBitmapIds) {
    // mark the winners in a bitmap of the row and emit them in id order
    constexpr int WPT = kBitmapIds / 32 / kFinNT;  // bitmap words per thread
#pragma unroll
    for (int q = 0; q < kFinPer; ++q)
      if (((vmask >> q) & 1u) && (v[q] >> (start_bit - pbits)) <= prefix) {
        const uint32_t id = (uint32_t)v[q];
        atomicOr(&bitmap[id >> 5], 1u << (id & 31));
      }
    __syncthreads();
    uint32_t wv[WPT];
    uint32_t c = 0;
#pragma unroll
    for (int q = 0; q < WPT; ++q) {
      const int w = tid * WPT + q;
      wv[q] = (w < words) ? bitmap[w] : 0u;
      c += __popc(wv[q]);
    }
    uint32_t pos = block_exclusive_scan<kFinNT>(c, wsum, nullptr);
#pragma unroll
    for (int q = 0; q < WPT; ++q) {
      uint32_t bits = wv[q];
      while (bits) {
        const int bit = __ffs(bits) - 1;
        bits &= bits - 1;
        if (pos < keep) out[pos] = (tid * WPT + q) * 32 + bit;
        ++pos;
      }
    }
  } else if (ok) {
    // very long rows: gather the winners and sort their ids
    uint32_t* ids = bitmap;
    if (tid == 0) res[3] = 0;
    __syncthreads();
#pragma unroll
    for (int q = 0; q < kFinPer; ++q)
      if (((vmask >> q) & 1u) && (v[q] >> (start_bit - pbits)) <= prefix) {
        const uint32_t p = atomicAdd(&res[3], 1u);
        if (p < keep) ids[p] = (uint32_t)v[q];
      }
    __syncthreads();
    uint32_t np2 = 1;
    while (np2 < keep) np2 <<= 1;
    for (uint32_t q = keep + tid; q < np2; q += kFinNT) ids[q] = 0xffffffffu;
    __syncthreads();
    for (uint32_t size = 2; size <= np2; size <<= 1) {
      for (uint32_t stride = size >> 1; stride > 0; stride >>= 1) {
        for (uint32_t i = tid; i < np2 / 2; i += kFinNT) {
          const uint32_t a = 2 * i - (i & (stride - 1));
          const uint32_t c2 = a + stride;
          const bool up = (a & size) == 0;
          const uint32_t x = ids[a], y = ids[c2];
          if ((x > y) == up) {
            ids[a] = y;
            ids[c2] = x;
          }
        }
        __syncthreads();
      }
    }
    for (uint32_t q = tid; q < keep; q += kFinNT) out[q] = (int32_t)ids[q];
  } else {
    // the lists cannot prove the selection: exact radix select on key << 32 | (~id) over
    // the whole row
    uint64_t pre = 0;
    int pb = 0;
    uint32_t need = keep;
    while (pb < 64) {
      const int width = (64 - pb) < 11 ? (64 - pb) : 11;
      const int shift = 64 - pb - width;
      for (int q = tid; q < 2048; q += kFinNT) hist[q] = 0;
      __syncthreads();
      for (int64_t i = tid; i < n; i += kFinNT) {
        const uint64_t C = ((uint64_t)score_key(srow[i]) << 32) | (uint64_t)(0xffffffffu - (uint32_t)i);
        if (pb == 0 || (C >> (64 - pb)) == pre) atomicAdd(&hist[(uint32_t)(C >> shift) & ((1u << width) - 1u)], 1u);
      }
      __syncthreads();
      find_threshold_bin<kFinNT, 2048>(hist, need, wsum, res);
      const uint32_t d = res[0], above = res[1], in_bin = res[2];
      pre = (pre << width) | d;
      pb += width;
      need -= above;
      __syncthreads();
      if (in_bin == need) break;
    }
    uint32_t base = 0;
    for (int64_t c0 = 0; c0 < n; c0 += kFinNT) {
      const int64_t i = c0 + tid;
      bool s = false;
      if (i < n) {
        const uint64_t C = ((uint64_t)score_key(srow[i]) << 32) | (uint64_t)(0xffffffffu - (uint32_t)i);
        s = (C >> (64 - pb)) >= pre;
      }
      uint32_t tot;
      const uint32_t e = block_exclusive_scan<kFinNT>(s ? 1u : 0u, wsum, &tot);
      if (s && base + e < keep) out[base + e] = (int32_t)i;
      base += tot;
    }
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
  return (size_t)B * T * topk_row_stride(max_entries);
}

int topk_max_k() { return kTopkMaxK; }

hipError_t launch_topk(const float* scores, int64_t ld, const int64_t* ent_off, const int64_t* q_pos, int m, int B,
                       int T, int k, int64_t max_entries, int32_t* idx, void* ws, bool prepared, hipStream_t st) {
  if (topk_uses_row_kernel(max_entries)) {
    if (max_entries <= 1024) return launch_row<1>(scores, ld, ent_off, q_pos, m, B, T, k, max_entries, idx, st);
    if (max_entries <= 4096) return launch_row<4>(scores, ld, ent_off, q_pos, m, B, T, k, max_entries, idx, st);
    if (max_entries <= 16384) return launch_row<16>(scores, ld, ent_off, q_pos, m, B, T, k, max_entries, idx, st);
    return launch_row<40>(scores, ld, ent_off, q_pos, m, B, T, k, max_entries, idx, st);
  }
  const int rows = B * T;
  if (!prepared) {
    const int S = topk_slice_size(max_entries);
    dim3 grid((unsigned)topk_num_slices(max_entries, S), (unsigned)rows);
    if (S == 512)
      topk_prepare_kernel<512><<<grid, 256, 0, st>>>(scores, ld, ent_off, q_pos, m, T, k, max_entries, ws);
    else if (S == 1024)
      topk_prepare_kernel<1024><<<grid, 256, 0, st>>>(scores, ld, ent_off, q_pos, m, T, k, max_entries, ws);
    else
      topk_prepare_kernel<2048><<<grid, 256, 0, st>>>(scores, ld, ent_off, q_pos, m, T, k, max_entries, ws);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  topk_finish_kernel<<<dim3((unsigned)rows), kFinNT, 0, st>>>(scores, ld, ent_off, q_pos, m, T, k, max_entries, idx,
                                                               ws);
  return hipGetLastError();
}

}  // namespace csl
