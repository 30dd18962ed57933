// topk_select: the k highest indexer scores of every query row, lower id first on ties,
// written as ascending ids padded with -1 ([P2] "Deep Dive", CSA top-k selection).
//
// Selection is a radix select on a unique composite key
//     C(i) = score_key(score_i) << IDX_BITS | (IDX_MASK - i)
// where score_key is an order-preserving 32-bit image of the fp32 score. Larger C means a
// larger score, or an equal score at a lower id, so the k largest composites are exactly
// the wanted set and no two elements tie. The kernels find the k-th largest composite
// digit by digit from the top with LDS histograms and stop as soon as the threshold bin
// holds exactly the number still needed.
//
// Two paths:
//   * row kernel (n <= 40960): one 1024-thread workgroup per row keeps the row's keys in
//     registers (element i = j*1024 + tid), radix-selects on a 48-bit composite (16 id
//     bits) and writes the selection with a block-wide ordered compaction, so the output
//     is already ascending.
//   * multi-workgroup path (long rows, e.g. 262144 scores at 1M context): G workgroups per
//     row first add their slices into a per-row 2048-bin histogram of the top 11 key bits
//     (global atomics). A second launch re-reads the slices, appends every element above
//     the threshold bin to a per-row list and every element inside it to a candidate
//     buffer; the last workgroup of the row (atomic ticket after a device-scope fence)
//     finishes the radix select on the candidates in LDS, sorts the k ids ascending and
//     returns the row's workspace to zero. If the threshold bin is larger than the
//     candidate buffer, the last workgroup refines over the whole row instead.
#include "device_common.h"
#include "launch.h"

namespace csl {

namespace {

constexpr int kHistBins = 2048;     // first digit: top 11 bits of the 32-bit score key
constexpr int kCandCap = 4096;      // candidate buffer per row (multi-workgroup path)
constexpr int kMaxK = 4096;
constexpr int kSegThreads = 256;
constexpr int kSegItems = 16;
constexpr int kSeg = kSegThreads * kSegItems;  // scores per workgroup slice

__device__ __forceinline__ int64_t row_count(const int64_t* ent_off, const int64_t* q_pos, int b, int t, int m,
                                             int64_t max_entries) {
  const int64_t n_ent = ent_off[b + 1] - ent_off[b];
  int64_t n = (q_pos[b] + t) / m;
  n = n < n_ent ? n : n_ent;
  n = n < max_entries ? n : max_entries;
  return n < 0 ? 0 : n;
}

__device__ __forceinline__ uint32_t lane_id() { return threadIdx.x % kWave; }

__device__ __forceinline__ uint32_t rank_in_wave(uint64_t mask) {
  const uint32_t l = lane_id();
  const uint64_t below = (l == 0) ? 0ull : (mask & ((~0ull) >> (64 - l)));
  return (uint32_t)__popcll(below);
}

// Exclusive prefix sum over a workgroup of NT threads (NT/64 waves). `wsum` holds >= NT/64 words.
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

// Given a histogram (LDS) whose bins are scanned from the top, find the bin where the
// running count from the top first reaches `need`. Writes digit / count-above / bin count.
template <int NT, int BINS>
__device__ __forceinline__ void find_threshold_bin(const uint32_t* hist, uint32_t need, uint32_t* wsum,
                                                   uint32_t* out3) {
  constexpr int PER = BINS / NT;
  uint32_t v[PER];
  uint32_t local = 0;
#pragma unroll
  for (int q = 0; q < PER; ++q) {
    v[q] = hist[BINS - 1 - (threadIdx.x * PER + q)];
    local += v[q];
  }
  uint32_t excl = block_exclusive_scan<NT>(local, wsum, nullptr);
#pragma unroll
  for (int q = 0; q < PER; ++q) {
    if (excl < need && need <= excl + v[q]) {
      out3[0] = BINS - 1 - (threadIdx.x * PER + q);
      out3[1] = excl;
      out3[2] = v[q];
    }
    excl += v[q];
  }
  __syncthreads();
}

// ---------------------------------------------------------------------------------------
// Row kernel: one workgroup per row, keys in registers.
// ---------------------------------------------------------------------------------------
template <int ITEMS>
__global__ __launch_bounds__(1024) void topk_row_kernel(const float* __restrict__ scores, int64_t ld,
                                                        const int64_t* __restrict__ ent_off,
                                                        const int64_t* __restrict__ q_pos, int m, int T, int k,
                                                        int64_t max_entries, int32_t* __restrict__ idx) {
  constexpr int NT = 1024;
  constexpr int NW = NT / kWave;
  __shared__ uint32_t hist[kHistBins];
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
  // composite C = key << 16 | (0xffff - i), 48 bits, handled as (key, low16)
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
    for (int q = tid; q < kHistBins; q += NT) hist[q] = 0;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < ITEMS; ++j) {
      const int i = j * NT + tid;
      if (i < n) {
        const uint64_t C = comp(j);
        if (pbits == 0 || (C >> (48 - pbits)) == prefix)
          atomicAdd(&hist[(uint32_t)(C >> shift) & ((1u << width) - 1u)], 1u);
      }
    }
    __syncthreads();
    find_threshold_bin<NT, kHistBins>(hist, need, wsum, res);
    const uint32_t d = res[0], above = res[1], in_bin = res[2];
    prefix = (prefix << width) | d;
    pbits += width;
    need -= above;
    __syncthreads();
    if (in_bin == need) break;  // the whole bin is taken
  }

  // ordered compaction of sel(i) = (C(i) >> (48 - pbits)) >= prefix
  const int wave = tid / kWave;
#pragma unroll
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
#pragma unroll
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
// Multi-workgroup path.
// ---------------------------------------------------------------------------------------
struct RowWs {
  uint32_t* hist;      // [kHistBins]
  uint32_t* ctr;       // [4]: n_def, n_cand, done, unused
  int32_t* def;        // [k]
  uint64_t* cand;      // [kCandCap]
};

__host__ __device__ inline size_t row_ws_stride(int k) {
  size_t s = (size_t)kHistBins * 4 + 16 + (size_t)k * 4;
  s = (s + 15) & ~(size_t)15;
  return s + (size_t)kCandCap * 8;
}

__device__ __forceinline__ RowWs row_ws(void* ws, int row, int k) {
  char* base = static_cast<char*>(ws) + (size_t)row * row_ws_stride(k);
  RowWs r;
  r.hist = reinterpret_cast<uint32_t*>(base);
  r.ctr = reinterpret_cast<uint32_t*>(base + kHistBins * 4);
  r.def = reinterpret_cast<int32_t*>(base + kHistBins * 4 + 16);
  size_t off = (size_t)kHistBins * 4 + 16 + (size_t)k * 4;
  off = (off + 15) & ~(size_t)15;
  r.cand = reinterpret_cast<uint64_t*>(base + off);
  return r;
}

__global__ __launch_bounds__(kSegThreads) void topk_hist_kernel(const float* __restrict__ scores, int64_t ld,
                                                                const int64_t* __restrict__ ent_off,
                                                                const int64_t* __restrict__ q_pos, int m, int T,
                                                                int k, int64_t max_entries, void* ws) {
  __shared__ uint32_t lh[kHistBins];
  const int row = blockIdx.y;
  const int b = row / T, t = row % T;
  const int64_t n = row_count(ent_off, q_pos, b, t, m, max_entries);
  if (n <= k) return;
  const int64_t lo = (int64_t)blockIdx.x * kSeg;
  if (lo >= n) return;
  for (int q = threadIdx.x; q < kHistBins; q += kSegThreads) lh[q] = 0;
  __syncthreads();
  const float* srow = scores + (int64_t)row * ld;
#pragma unroll
  for (int j = 0; j < kSegItems; ++j) {
    const int64_t i = lo + j * kSegThreads + threadIdx.x;
    if (i < n) atomicAdd(&lh[score_key(srow[i]) >> 21], 1u);
  }
  __syncthreads();
  RowWs r = row_ws(ws, row, k);
  for (int q = threadIdx.x; q < kHistBins; q += kSegThreads)
    if (lh[q]) atomicAdd(&r.hist[q], lh[q]);
}

// LDS layout of the select kernel (bytes): the last workgroup reuses it for candidates.
constexpr int kSelLds = kCandCap * 8 + kMaxK * 4 + kHistBins * 4;

__device__ void bitonic_sort_ascending(int32_t* a, int n_pow2) {
  for (int size = 2; size <= n_pow2; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = threadIdx.x; i < n_pow2 / 2; i += kSegThreads) {
        const int lo = 2 * i - (i & (stride - 1));
        const int hi = lo + stride;
        const bool up = ((lo & size) == 0);
        const int32_t x = a[lo], y = a[hi];
        if ((x > y) == up) {
          a[lo] = y;
          a[hi] = x;
        }
      }
      __syncthreads();
    }
  }
}

__global__ __launch_bounds__(kSegThreads) void topk_select_kernel(const float* __restrict__ scores, int64_t ld,
                                                                  const int64_t* __restrict__ ent_off,
                                                                  const int64_t* __restrict__ q_pos, int m, int T,
                                                                  int k, int64_t max_entries, int32_t* __restrict__ idx,
                                                                  void* ws) {
  constexpr int NT = kSegThreads;
  constexpr int NW = NT / kWave;
  extern __shared__ __align__(16) unsigned char lds[];
  __shared__ uint32_t wsum[NW];
  __shared__ uint32_t res[4];
  __shared__ uint32_t sh_base[2];
  __shared__ int sh_last;

  const int row = blockIdx.y;
  const int b = row / T, t = row % T;
  const int tid = threadIdx.x;
  const int64_t n = row_count(ent_off, q_pos, b, t, m, max_entries);
  int32_t* out = idx + (int64_t)row * k;
  const float* srow = scores + (int64_t)row * ld;
  const int64_t lo = (int64_t)blockIdx.x * kSeg;

  if (n <= k) {  // every visible entry is selected; ids are written in place
    for (int j = 0; j < kSegItems; ++j) {
      const int64_t i = lo + j * NT + tid;
      if (i < k) out[i] = i < n ? (int32_t)i : -1;
    }
    return;
  }
  const uint32_t keep = (uint32_t)k;
  RowWs r = row_ws(ws, row, k);
  uint32_t* h = reinterpret_cast<uint32_t*>(lds + kCandCap * 8 + kMaxK * 4);
  for (int q = tid; q < kHistBins; q += NT) h[q] = r.hist[q];
  __syncthreads();
  find_threshold_bin<NT, kHistBins>(h, keep, wsum, res);
  const uint32_t d1 = res[0], above1 = res[1], cnt1 = res[2];
  const bool big = cnt1 > (uint32_t)kCandCap;
  const uint32_t need1 = keep - above1;

  if (lo < n) {
#pragma unroll 1
    for (int j = 0; j < kSegItems; ++j) {
      const int64_t i = lo + j * NT + tid;
      uint32_t key = 0;
      const bool v = i < n;
      if (v) key = score_key(srow[i]);
      const uint32_t dig = key >> 21;
      const bool is_def = v && dig > d1;
      const bool is_cand = v && !big && dig == d1;
      // workgroup-aggregated appends: one atomic per list per workgroup and step
      const uint64_t md = __ballot(is_def), mc = __ballot(is_cand);
      __shared__ uint32_t wcnt[2][NW];
      const int wave = tid / kWave;
      if (lane_id() == 0) {
        wcnt[0][wave] = (uint32_t)__popcll(md);
        wcnt[1][wave] = (uint32_t)__popcll(mc);
      }
      __syncthreads();
      if (tid == 0) {
        uint32_t td = 0, tc = 0;
        for (int w = 0; w < NW; ++w) {
          td += wcnt[0][w];
          tc += wcnt[1][w];
        }
        sh_base[0] = td ? atomicAdd(&r.ctr[0], td) : 0u;
        sh_base[1] = tc ? atomicAdd(&r.ctr[1], tc) : 0u;
      }
      __syncthreads();
      uint32_t bd = sh_base[0], bc = sh_base[1];
      for (int w = 0; w < wave; ++w) {
        bd += wcnt[0][w];
        bc += wcnt[1][w];
      }
      if (is_def) {
        const uint32_t pos = bd + rank_in_wave(md);
        if (pos < keep) r.def[pos] = (int32_t)i;
      }
      if (is_cand) {
        const uint32_t pos = bc + rank_in_wave(mc);
        if (pos < (uint32_t)kCandCap) r.cand[pos] = ((uint64_t)key << 32) | (uint64_t)(0xffffffffu - (uint32_t)i);
      }
      __syncthreads();
    }
  }

  // ticket: the last workgroup of the row finishes it
  __threadfence();
  __syncthreads();
  if (tid == 0) sh_last = (atomicAdd(&r.ctr[2], 1u) == gridDim.x - 1) ? 1 : 0;
  __syncthreads();
  if (!sh_last) return;
  __threadfence();

  int32_t* ids = reinterpret_cast<int32_t*>(lds + kCandCap * 8);
  uint32_t* h8 = h;  // reused as a 256-bin histogram
  if (!big) {
    // ---- refine inside the candidate set (all share the top 11 key bits) ----
    uint64_t* cand = reinterpret_cast<uint64_t*>(lds);
    const uint32_t nc = cnt1 < (uint32_t)kCandCap ? cnt1 : (uint32_t)kCandCap;
    for (uint32_t q = tid; q < nc; q += NT) cand[q] = r.cand[q];
    for (uint32_t q = tid; q < above1 && q < keep; q += NT) ids[q] = r.def[q];
    __syncthreads();
    uint64_t prefix = 0;  // over the low 53 bits
    int pbits = 0;
    uint32_t need = need1;
    for (int pass = 0; pass < 7; ++pass) {
      const int width = pass == 2 ? 5 : 8;
      const int shift = 53 - pbits - width;
      for (int q = tid; q < 256; q += NT) h8[q] = 0;
      __syncthreads();
      for (uint32_t q = tid; q < nc; q += NT) {
        const uint64_t c = cand[q] & ((1ull << 53) - 1);
        if (pbits == 0 || (c >> (53 - pbits)) == prefix) atomicAdd(&h8[(uint32_t)(c >> shift) & ((1u << width) - 1)], 1u);
      }
      __syncthreads();
      find_threshold_bin<NT, 256>(h8, need, wsum, res);
      const uint32_t d = res[0], above = res[1], in_bin = res[2];
      prefix = (prefix << width) | d;
      pbits += width;
      need -= above;
      __syncthreads();
      if (in_bin == need) break;
    }
    // append chosen candidates after the definite ids (order fixed by the sort below)
    __shared__ uint32_t app;
    if (tid == 0) app = above1;
    __syncthreads();
    for (uint32_t q = tid; q < nc; q += NT) {
      const uint64_t c = cand[q] & ((1ull << 53) - 1);
      if ((c >> (53 - pbits)) >= prefix) {
        const uint32_t pos = atomicAdd(&app, 1u);
        if (pos < keep) ids[pos] = (int32_t)(0xffffffffu - (uint32_t)(cand[q] & 0xffffffffull));
      }
    }
    __syncthreads();
    int np2 = 1;
    while (np2 < (int)keep) np2 <<= 1;
    for (int q = keep + tid; q < np2; q += NT) ids[q] = 0x7fffffff;
    __syncthreads();
    bitonic_sort_ascending(ids, np2);
    for (int q = tid; q < k; q += NT) out[q] = q < (int)keep ? ids[q] : -1;
  } else {
    // ---- threshold bin too large for the buffer: refine over the whole row ----
    uint64_t prefix = d1;  // known top 11 bits of the 64-bit composite
    int pbits = 11;
    uint32_t need = need1;
    for (int pass = 0; pass < 7; ++pass) {
      const int width = pass == 2 ? 5 : 8;
      const int shift = 64 - pbits - width;
      for (int q = tid; q < 256; q += NT) h8[q] = 0;
      __syncthreads();
      for (int64_t i = tid; i < n; i += NT) {
        const uint64_t C = ((uint64_t)score_key(srow[i]) << 32) | (uint64_t)(0xffffffffu - (uint32_t)i);
        if ((C >> (64 - pbits)) == prefix) atomicAdd(&h8[(uint32_t)(C >> shift) & ((1u << width) - 1)], 1u);
      }
      __syncthreads();
      find_threshold_bin<NT, 256>(h8, need, wsum, res);
      const uint32_t d = res[0], above = res[1], in_bin = res[2];
      prefix = (prefix << width) | d;
      pbits += width;
      need -= above;
      __syncthreads();
      if (in_bin == need) break;
    }
    // ordered compaction over the row, chunk by chunk
    uint32_t base = 0;
    for (int64_t c0 = 0; c0 < n; c0 += NT) {
      const int64_t i = c0 + tid;
      bool s = false;
      if (i < n) {
        const uint64_t C = ((uint64_t)score_key(srow[i]) << 32) | (uint64_t)(0xffffffffu - (uint32_t)i);
        s = (C >> (64 - pbits)) >= prefix;
      }
      uint32_t tot;
      const uint32_t e = block_exclusive_scan<NT>(s ? 1u : 0u, wsum, &tot);
      if (s && base + e < keep) out[base + e] = (int32_t)i;
      base += tot;
    }
    for (int q = keep + tid; q < k; q += NT) out[q] = -1;
  }
  // return the row's workspace to zero for the next call
  for (int q = tid; q < kHistBins; q += NT) r.hist[q] = 0;
  if (tid < 3) r.ctr[tid] = 0;
}

template <int ITEMS>
hipError_t launch_row(const float* scores, int64_t ld, const int64_t* ent_off, const int64_t* q_pos, int m, int B,
                      int T, int k, int64_t max_entries, int32_t* idx, hipStream_t st) {
  topk_row_kernel<ITEMS><<<dim3((unsigned)(B * T)), 1024, 0, st>>>(scores, ld, ent_off, q_pos, m, T, k, max_entries, idx);
  return hipGetLastError();
}

}  // namespace

bool topk_uses_row_kernel(int64_t max_entries) { return max_entries <= 40 * 1024; }

size_t topk_workspace_bytes(int B, int T, int64_t max_entries, int k) {
  if (topk_uses_row_kernel(max_entries) || max_entries <= k) return 0;
  return (size_t)B * T * row_ws_stride(k);
}

int topk_max_k() { return kMaxK; }

hipError_t launch_topk(const float* scores, int64_t ld, const int64_t* ent_off, const int64_t* q_pos, int m, int B,
                       int T, int k, int64_t max_entries, int32_t* idx, void* ws, hipStream_t st) {
  if (topk_uses_row_kernel(max_entries)) {
    if (max_entries <= 1024) return launch_row<1>(scores, ld, ent_off, q_pos, m, B, T, k, max_entries, idx, st);
    if (max_entries <= 4096) return launch_row<4>(scores, ld, ent_off, q_pos, m, B, T, k, max_entries, idx, st);
    if (max_entries <= 16384) return launch_row<16>(scores, ld, ent_off, q_pos, m, B, T, k, max_entries, idx, st);
    return launch_row<40>(scores, ld, ent_off, q_pos, m, B, T, k, max_entries, idx, st);
  }
  const int64_t G = (max_entries + kSeg - 1) / kSeg;
  dim3 grid((unsigned)G, (unsigned)(B * T));
  if (max_entries > k) {
    topk_hist_kernel<<<grid, kSegThreads, 0, st>>>(scores, ld, ent_off, q_pos, m, T, k, max_entries, ws);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  topk_select_kernel<<<grid, kSegThreads, kSelLds, st>>>(scores, ld, ent_off, q_pos, m, T, k, max_entries, idx, ws);
  return hipGetLastError();
}

}  // namespace csl
