// The top-k selection of one short row by a whole workgroup ([P2] "Deep Dive", CSA top-k
// selection), for launches that already give each query row one workgroup: the k best of the
// row's n visible scores by (score descending, id ascending), in ascending id order and -1
// padded. That is the selection csl_topk_select makes, so the two give the same ids.
//
// Thread tid holds the keys of ids j * NT + tid (j < ITEMS), so n <= ITEMS * NT. The k-th key
// is found by a radix search over the 8-bit digits of the 32-bit keys, most significant first,
// counted in one LDS histogram (it stops at the first digit whose bin holds exactly the keys
// still needed); one scan of per-(item, wave) counts then places every winner: the keys above
// the threshold, and the lowest ids among the keys equal to it.
#pragma once

#include "device_common.h"
#include "topk_common.h"

namespace csl {

template <int NT, int ITEMS>
struct ShortTopkLds {
  uint32_t hist[256];
  uint32_t cnt[ITEMS * (NT / kWave)];
  uint32_t res[4];
};

// The visible entries of query row (b, t): floor(p / m) at position p = q_pos[b] + t, capped at
// the sequence's entries and at max_entries (every top-k kernel counts a row's entries so).
__device__ __forceinline__ int64_t visible_entries(const int64_t* __restrict__ ent_off,
                                                  const int64_t* __restrict__ q_pos, int b, int t, int m,
                                                  int64_t max_entries) {
  const int64_t n_ent = ent_off[b + 1] - ent_off[b];
  int64_t n = (q_pos[b] + t) / m;
  n = n < n_ent ? n : n_ent;
  n = n < max_entries ? n : max_entries;
  return n < 0 ? 0 : n;
}

// Writes the selection to sel[0, k) (LDS) and out[0, k) (global). srow holds at least cap >= n
// readable scores (the row's stride allows max_entries), so the score loads need not wait for
// n, whose own loads may still be in flight. Every thread of the workgroup calls it; it holds
// workgroup barriers, and the caller puts one more between it and the first read of sel.
template <int NT, int ITEMS>
__device__ __forceinline__ void short_row_topk(const float* __restrict__ srow, int64_t cap, int64_t n, int k,
                                               int32_t* __restrict__ sel, int32_t* __restrict__ out,
                                               ShortTopkLds<NT, ITEMS>& L) {
  constexpr int NW = NT / kWave;
  static_assert(NT >= 256 && NT % kWave == 0, "one histogram bin per thread");
  static_assert(ITEMS * NW <= kWave, "one wave scans the per-(item, wave) counts");
  const int tid = threadIdx.x;
  const int wave = tid / kWave;
  const int lane = tid % kWave;
  // the scores first, from ids clamped to cap (no branch per load); the ids past the row are
  // then marked invalid
  float sv[ITEMS];
  if (cap > 0) {
#pragma unroll
    for (int j = 0; j < ITEMS; ++j) {
      const int64_t i = j * NT + tid;
      sv[j] = srow[i < cap ? i : cap - 1];
    }
  }
  const uint32_t keep = (uint32_t)(n < k ? n : (int64_t)k);
  if ((int64_t)keep == n) {  // everything visible is selected
    for (int p = tid; p < k; p += NT) {
      const int32_t v = p < n ? p : -1;
      sel[p] = v;
      out[p] = v;
    }
    return;
  }
  uint32_t key[ITEMS];
  bool valid[ITEMS];
#pragma unroll
  for (int j = 0; j < ITEMS; ++j) {
    const int i = j * NT + tid;
    valid[j] = i < n;
    key[j] = valid[j] ? score_key(sv[j]) : 0u;
  }
  uint32_t prefix = 0u, need = keep;
  bool all_in = false;
  int shift = 32;
  for (int pass = 0; pass < 4; ++pass) {  // uniform
    shift -= 8;
    if (tid < 256) L.hist[tid] = 0u;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < ITEMS; ++j)
      if (valid[j] && (pass == 0 || (key[j] >> (shift + 8)) == prefix))
        atomicAdd(&L.hist[(key[j] >> shift) & 255u], 1u);
    __syncthreads();
    if (wave == 0) {
      // bins from the top down, 4 per lane: lane l holds bins 255 - 4l .. 252 - 4l
      uint32_t c[4], local = 0u;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        c[q] = L.hist[255 - 4 * lane - q];
        local += c[q];
      }
      uint32_t excl = wave_incl_scan(local) - local;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (excl < need && need <= excl + c[q]) {
          L.res[0] = (uint32_t)(255 - 4 * lane - q);
          L.res[1] = excl;
          L.res[2] = c[q];
        }
        excl += c[q];
      }
    }
    __syncthreads();
    prefix = (prefix << 8) | L.res[0];
    need -= L.res[1];
    if (L.res[2] == need) {  // every key of the bin is in
      all_in = true;
      break;
    }
  }
  // without all_in the search ran to the last digit: prefix is the k-th key itself, and the
  // need lowest ids among the keys equal to it are in
  const uint32_t need_eq = all_in ? 0u : need;
  auto above = [&](int j) {
    const uint32_t h = key[j] >> shift;
    return valid[j] && (h > prefix || (all_in && h == prefix));
  };
  auto tied = [&](int j) { return valid[j] && !all_in && key[j] == prefix; };
  {
    uint32_t mycnt = 0u;  // lane j: (above | tied << 16) count of item j in this wave
#pragma unroll
    for (int j = 0; j < ITEMS; ++j) {
      const uint32_t c = (uint32_t)__popcll(__ballot(above(j))) | ((uint32_t)__popcll(__ballot(tied(j))) << 16);
      mycnt = (lane == j) ? c : mycnt;
    }
    if (lane < ITEMS) L.cnt[lane * NW + wave] = mycnt;
  }
  __syncthreads();
  if (wave == 0) {  // exclusive prefix of the counts in id order (item, then wave)
    const uint32_t v = (lane < ITEMS * NW) ? L.cnt[lane] : 0u;
    const uint32_t incl = wave_incl_scan(v);
    if (lane < ITEMS * NW) L.cnt[lane] = incl - v;
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < ITEMS; ++j) {
    const uint32_t base = L.cnt[j * NW + wave];
    const bool g = above(j), e = tied(j);
    const uint32_t gb = (base & 0xffffu) + rank_in_wave(__ballot(g));
    const uint32_t eb = (base >> 16) + rank_in_wave(__ballot(e));
    const int32_t id = j * NT + tid;
    int pos = -1;
    if (g) pos = (int)(gb + min(eb, need_eq));  // every tie taken before it precedes it
    else if (e && eb < need_eq) pos = (int)(gb + eb);
    if (pos >= 0) {
      sel[pos] = id;
      out[pos] = id;
    }
  }
  for (int p = (int)keep + tid; p < k; p += NT) {
    sel[p] = -1;
    out[p] = -1;
  }
}

}  // namespace csl
