// The finishing step of the long-row top-k selection ([P2] "Deep Dive", CSA top-k selection),
// as workgroup-level device functions of NT threads, which the finishing kernel runs with 1024
// threads, one workgroup per query row.
//
// From the row's slice candidate lists (topk_common.h) it radix-selects the k best listed
// entries on their 32-bit keys (lower id first within the last tied key), checks that the k-th
// best listed key reaches every slice's cut (then the selection is the row's), and writes the
// winners in ascending id order straight from the slot order with one block-wide scan. If the
// check fails, or the row is too dense for lists, it runs an exact pass over the row's scores.
#pragma once

#include "device_common.h"
#include "topk_common.h"

namespace csl {

template <int NT>
struct FinishLds {
  uint32_t hist_a[2048];
  uint32_t hist_b[2048];
  uint32_t hist_c[1024];
  uint32_t wsum[3 * (NT / kWave)];
  uint32_t res[4];
};

// One radix step: over BINS bins (hist in LDS), find the bin holding the need-th largest key
// counting from the top bin down. res = {bin, count above it, count in it, total}. Contains two
// workgroup barriers; the caller reads res after it returns.
template <int NT, int BINS>
__device__ __forceinline__ void fin_threshold(const uint32_t* hist, uint32_t need, uint32_t* wsum, uint32_t* res) {
  constexpr int PER = BINS / NT;
  constexpr int NW = NT / kWave;
  static_assert(PER * NT == BINS, "bins per thread");
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
  for (int w = 0; w < NW; ++w) {
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

// Exact selection over the whole row from its scores, for rows whose candidate lists cannot
// prove the selection and rows too dense for them. Passes over the row (from L2):
//   1. block min and max of the keys;
//   2. radix select of the keep-th largest key: 11 bits just below the keys' common prefix,
//      then the rest (usually one more pass);
//   3. ordered compaction in chunks of J * NT ids with one packed block scan of the
//      (above, tied) counts per chunk, lower ids first among keys tied at the threshold.
template <int NT>
__device__ __forceinline__ void finish_full_row(const float* __restrict__ srow, int64_t n, uint32_t keep, int32_t* __restrict__ out,
                                FinishLds<NT>& L) {
  constexpr int NW = NT / kWave;
  const int tid = threadIdx.x;
  const int wave = tid / kWave;
  uint32_t* hist_a = L.hist_a;
  uint32_t* hist_b = L.hist_b;
  uint32_t* wsum = L.wsum;
  uint32_t* res = L.res;
  // visit every key of the row: 16 coalesced loads in flight per thread
  constexpr int U = 16;
  auto for_keys = [&](auto&& fn) {
    for (int64_t c0 = 0; c0 < n; c0 += (int64_t)U * NT) {
      float v[U];
#pragma unroll
      for (int j = 0; j < U; ++j) {
        const int64_t i = c0 + (int64_t)j * NT + tid;
        v[j] = srow[i < n ? i : n - 1];  // clamped: no branch per load
      }
#pragma unroll
      for (int j = 0; j < U; ++j)
        if (c0 + (int64_t)j * NT + tid < n) {
          const uint32_t x = score_key(v[j]);
          if (x) fn(x);  // key 0 marks no entry (kNoScoreBits below)
        }
    }
  };
  for (int q = tid; q < 2048; q += NT) {
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
    wsum[NW + wave] = kmax;
  }
  __syncthreads();
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    kmin = min(kmin, wsum[w]);
    kmax = max(kmax, wsum[NW + w]);
  }
  // keys share their top `common` bits: bin the 11 below them first
  const int common = __clz(kmin ^ kmax);
  int shift = common >= 21 ? 0 : 21 - common;
  uint32_t need = keep;
  for_keys([&](uint32_t x) { atomicAdd(&hist_a[(x >> shift) & 2047u], 1u); });
  __syncthreads();
  fin_threshold<NT, 2048>(hist_a, need, wsum, res);
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
    fin_threshold<NT, 2048>(hist, need, wsum, res);
    prefix = (prefix << wb) | res[0];
    shift = sb;
    need -= res[1];
    all_in = res[2] == need;
    // the other histogram is free again (its last reads ended before fin_threshold's barriers)
    uint32_t* other = (hist == hist_b) ? hist_a : hist_b;
    for (int q = tid; q < 2048; q += NT) other[q] = 0;
    hist = other;
    __syncthreads();
  }
  const uint32_t need_eq = all_in ? 0u : need;

  constexpr int J = 16;
  uint32_t gbase = 0, ebase = 0;
  for (int64_t c0 = 0; c0 < n; c0 += (int64_t)J * NT) {
    const int64_t i0 = c0 + (int64_t)J * tid;
    uint32_t gm = 0, em = 0;
    float v[J];
#pragma unroll
    for (int j = 0; j < J; ++j) v[j] = srow[i0 + j < n ? i0 + j : n - 1];  // clamped: no branch per load
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const uint32_t x = score_key(v[j]);
      if (i0 + j < n && x) {
        const uint32_t h = x >> shift;
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
    for (int w = 0; w < NW; ++w) {
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

// The whole selection of one row of n = row_n() visible entries (k best, ascending ids, -1
// padded into out[0..k)), by NT threads: everything visible when n <= k, the exact row pass when the row
// is too dense for lists, else the k best listed entries with the cut check (and the row pass
// when the check fails). Thread i owns CH consecutive chunks of 8 slots of the row's layout
// (a slice spans R / 8 chunks), so thread order is slot order is id order; the row's layout
// must fit: topk_num_slices(max_entries) * budget <= 8 * CH * NT.
// What finish_row does before the exact row pass when the lists cannot prove a row's
// selection: nothing (the row's scores are in place), or, when the indexer left no scores
// for the row (scores on demand), build them: a Repair with kActive recomputes the scores of
// entries [e0, min(e0 + 64, n)) with one wave (wave(e0, n)).
struct NoRepair {
  static constexpr bool kActive = false;
  __device__ void wave(int64_t, int64_t) const {}
};

// A value in a score row that the exact row pass skips: the one float whose key is 0 (a NaN
// with every bit set, which no score is)
constexpr uint32_t kNoScoreBits = 0xffffffffu;

// The float whose score_key is x (score_key is one-to-one on floats other than -0)
__device__ __forceinline__ float key_score(uint32_t x) {
  return __uint_as_float((x & 0x80000000u) ? (x & 0x7fffffffu) : ~x);
}

template <int NT, int CH, typename RowN, typename Repair = NoRepair>
__device__ __forceinline__ void finish_row(const float* __restrict__ srow, TopkRowWs rw, RowN row_n,
                                           int64_t max_entries, int budget, int k, int32_t* __restrict__ out,
                                           FinishLds<NT>& L, Repair repair = Repair{}) {
  constexpr int PER = 8;  // slots per chunk
  constexpr int NW = NT / kWave;
  static_assert(kMinSliceSlots % PER == 0, "a slice spans whole chunks");
  uint32_t* hist_a = L.hist_a;
  uint32_t* hist_b = L.hist_b;
  uint32_t* hist_c = L.hist_c;
  uint32_t* wsum = L.wsum;
  uint32_t* res = L.res;
  const int tid = threadIdx.x;
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
  // the cut of each chunk's slice for each possible layout (2, 4 or 8 chunks per slice; which
  // one is the row's depends on n, whose loads may still be in flight), also issued now and
  // needed only at the end: the loads of the step all go out together
  const int ns_max = (int)topk_num_slices(max_entries);
  uint32_t cut3[CH][3];
#pragma unroll
  for (int c = 0; c < CH; ++c)
#pragma unroll
    for (int l = 0; l < 3; ++l) cut3[c][l] = rw.cuts[min((tid * CH + c) >> (l + 1), ns_max - 1)];
  const int64_t n = row_n();  // the row's visible entries (its own loads go out after the slots')
  const uint32_t keep = (uint32_t)(n < k ? n : k);
  for (int q = tid; q < 2048; q += NT) {
    hist_a[q] = 0;
    hist_b[q] = 0;
  }
  for (int q = tid; q < 1024; q += NT) hist_c[q] = 0;

  if ((int64_t)keep == n) {
    for (int p = tid; p < k; p += NT) out[p] = p < n ? p : -1;
    return;
  }
  if (topk_row_dense(n, k)) {
    // winners too dense for candidate lists (more than 5 expected per wave of 64 entries):
    // the lists were not written, search the row directly
    finish_full_row<NT>(srow, n, keep, out, L);
    for (int p = (int)keep + tid; p < k; p += NT) out[p] = -1;
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
    wsum[NW + wave] = kmax;
  }
  __syncthreads();  // histograms cleared, wave extremes posted
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    kmin = min(kmin, wsum[w]);
    kmax = max(kmax, wsum[NW + w]);
  }

  // radix select of the keep-th largest listed key. The listed keys share their top
  // L = clz(kmin ^ kmax) bits, so the first pass bins the 11 bits below those (spreading the
  // keys over the bins instead of piling them into a few), the later passes the rest.
  bool ok = true;
  bool all_in = false;
  uint32_t need = keep;
  const int common = __clz(kmin ^ kmax);  // 32 when all keys are equal
  int shift = common >= 21 ? 0 : 21 - common;
  uint32_t prefix = 0;  // value of key >> shift shared by the keys still in play
#pragma unroll
  for (int c = 0; c < CH; ++c)
#pragma unroll
    for (int q = 0; q < PER; ++q)
      if (key[c][q]) atomicAdd(&hist_a[(key[c][q] >> shift) & 2047u], 1u);
  __syncthreads();
  fin_threshold<NT, 2048>(hist_a, need, wsum, res);
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
      fin_threshold<NT, 2048>(hist_b, need, wsum, res);
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
        fin_threshold<NT, 1024>(hist_c, need, wsum, res);
        prefix = (prefix << shift) | res[0];
        shift = 0;
        need -= res[1];
        all_in = res[2] == need;
      }
    }
  }

  const bool listed_enough = ok;  // the lists hold at least `keep` keys
  uint32_t lo = 0;                 // lowest key a listed winner can have
  if (ok) {
    // winners: keys above the selected bin, plus (unless the whole bin is taken) the first
    // `need` keys equal to the exact key value, in id order
    lo = prefix << shift;
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
      wsum[NW + wave] = wviol ? 1u : 0u;
    }
    __syncthreads();
    uint32_t before = 0, tv = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      before += (w < wave) ? wsum[w] : 0u;
      tv |= wsum[NW + w];
    }
    if (tv != 0u) {
      ok = false;  // a slice may hide a winner below its cut
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
    if constexpr (Repair::kActive) {
      // no scores from the indexer: build the row the exact pass reads. With fewer listed keys
      // than winners, recompute every entry. Otherwise the true threshold is at or above the
      // k-th listed key lo, so a slice whose cut is at or below lo lists every entry that can
      // win: its listed entries take their listed keys and the rest kNoScoreBits, which the
      // exact pass skips;
      // the slices whose cut is above lo are recomputed whole.
      float* row = const_cast<float*>(srow);
      const int wave = tid / kWave;
      if (!listed_enough) {
        for (int64_t e0 = (int64_t)wave * kWave; e0 < n; e0 += NT) repair.wave(e0, n);
      } else {
        uint32_t* redo = hist_a;  // per slice: recompute it (ns <= 2048)
        for (int64_t i = tid; i < n; i += NT) row[i] = __uint_as_float(kNoScoreBits);
        for (int q = tid; q < ns; q += NT) redo[q] = 0u;
        __threadfence();  // stores of every wave done before the next writes to the same row
        __syncthreads();
#pragma unroll
        for (int c = 0; c < CH; ++c) {
          const int slice = (tid * CH + c) >> cps_log2;
          if (slice >= ns) continue;
          if (cut[c] > lo) redo[slice] = 1u;
#pragma unroll
          for (int q = 0; q < PER; ++q)
            if (key[c][q]) row[(uint32_t)sl[c][q]] = key_score(key[c][q]);
        }
        __threadfence();  // stores of every wave done before the next writes to the same row
        __syncthreads();
        constexpr int WPS = kSlice / kWave;  // wave-sized parts of a slice
        for (int t = wave; t < ns * WPS; t += NW)
          if (redo[t / WPS]) repair.wave((int64_t)t * kWave, n);
      }
      // the exact pass reads the row back through global memory (a rare path: the fences are
      // device-wide, so no wave's store can land after another wave's read or write)
      __threadfence();
      __syncthreads();
    }
    finish_full_row<NT>(srow, n, keep, out, L);
  }
  for (int p = (int)keep + tid; p < k; p += NT) out[p] = -1;
}

}  // namespace csl
