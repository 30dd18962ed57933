// Softmax-weighted pooling of m consecutive raw K=V rows into one compressed entry, as a
// workgroup-level device function shared by compress_kv's own kernel and the fused decode
// step (which runs it in spare workgroups of the indexer launch).
//
// Each compressed entry is, per dimension d, a softmax over the m chunk rows of the
// logits z[:, d] applied to kv[:, d] ([P3] section 3: per-dimension weights of the chunk
// tokens; [P2] "Deep Dive", CSA step 2 and HCA "How it works").
//
// With DUAL (CSA's overlapped compression, [P2] "Deep Dive", dual-series KV compression;
// [P1] section 4.3) entry i pools 2m rows under one softmax per dimension: rows
// [m*i, m*i + m) of series a (kv, z) and rows [m*(i-1), m*i) of series b (kv_b, z_b), the
// block before it. Entry 0 has no earlier block and pools its m series-a rows alone. The
// 2m rows are one virtual chunk, series a first, split over the lanes like a plain chunk.
//
// Layout: a thread owns 8 consecutive dimensions (16 bytes of bf16) of one entry and a
// strided subset of its rows; TPE = D/8 threads cover one row, RS row-splits of the same
// entry sit TPE lanes apart inside a wave and merge their partial softmax states with
// xor-shuffles; for long chunks RSX waves split the rows further (an m = 128 entry then
// loads in one round trip) and merge in two passes, through lane swaps and LDS. Loads are
// 16-byte, row-contiguous across the TPE lanes, so a wave reads whole 256-byte rows. It reads
// 2*m*D*2 bytes and writes D*4 (fp32) or D*2 (bf16) bytes per entry (twice the reads with DUAL).
#pragma once

#include "device_common.h"
#include "launch.h"

namespace csl {

// Where a finished entry goes: row orow of out (bf16 or fp32), 8 dims per thread.
template <bool OUT_BF16>
struct StoreEntry {
  void* out;
  int D;
  __device__ __forceinline__ void operator()(int64_t /*i*/, int64_t orow, int dg, const float (&o)[8]) const {
    if (OUT_BF16) {
      u32x4 v;
      v.x = pack_bf16x2(o[0], o[1]);
      v.y = pack_bf16x2(o[2], o[3]);
      v.z = pack_bf16x2(o[4], o[5]);
      v.w = pack_bf16x2(o[6], o[7]);
      *reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(out) + orow * D + dg * 8) = v;
    } else {
      float* op = reinterpret_cast<float*>(out) + orow * D + dg * 8;
      *reinterpret_cast<float4*>(op) = make_float4(o[0], o[1], o[2], o[3]);
      *reinterpret_cast<float4*>(op + 4) = make_float4(o[4], o[5], o[6], o[7]);
    }
  }
};

// Maximum (MAX) or sum of v over the RS in-wave row-splits of an entry, which sit TPE, 2 TPE,
// 4 TPE lanes apart; every lane of the entry gets the same bits.
template <int TPE, int RS>
__device__ __forceinline__ float splits_reduce(float v, bool MAX) {
  static_assert(RS == 1 || RS == 2 || RS == 4 || RS == 8, "power-of-two in-wave splits");
  if constexpr (RS >= 2) v = MAX ? xor_max<TPE>(v) : xor_sum<TPE>(v);
  if constexpr (RS >= 4) v = MAX ? xor_max<2 * TPE>(v) : xor_sum<2 * TPE>(v);
  if constexpr (RS >= 8) v = MAX ? xor_max<4 * TPE>(v) : xor_sum<4 * TPE>(v);
  return v;
}

// One workgroup of NT threads compresses the NT / (TPE * RS * RSX) entries first_entry[b] +
// blk * that .. of sequence b (entries past max_new or past the sequence end are skipped) and
// hands each finished entry i (8 dims per thread dg, its cache row orow) to store. Each thread
// loads ROWS of its rows at a time. With RSX > 1 every thread of the workgroup must call this
// (it holds a workgroup barrier).
template <int NT, int TPE, int RS, bool HAS_Z, int ROWS, int RSX, bool DUAL, class Store>
__device__ __forceinline__ void compress_block_to(
    const uint16_t* __restrict__ kv, const uint16_t* __restrict__ z,
    const int64_t* __restrict__ kv_off, const int64_t* __restrict__ ent_off,
    const int64_t* __restrict__ first_entry, int D, int m, int64_t max_new, const Store& store, int b,
    int64_t blk, const uint16_t* __restrict__ kv_b, const uint16_t* __restrict__ z_b, PagedView pg) {
  static_assert(TPE * RS <= kWave, "in-wave row-splits merge by shuffles");
  static_assert(RSX == 1 || TPE * RS == kWave, "cross-wave splits take whole waves");
  constexpr int EPB = NT / (TPE * RS * RSX);  // entries per block
  constexpr int NSPLIT = RS * RSX;           // row-splits per entry
  const int t = threadIdx.x;
  const int dg = t % TPE;
  const int rsw = (t / TPE) % RS;              // split inside the wave
  const int rsx = (t / (TPE * RS)) % RSX;      // wave of the entry
  const int rs = rsx * RS + rsw;               // row-split index of this lane
  const int el = t / (TPE * RS * RSX);

  const int64_t row0 = kv_off[b];
  const int64_t n_rows = kv_off[b + 1] - row0;
  const int64_t n_ent = n_rows / m;
  int64_t first = first_entry ? first_entry[b] : 0;
  if (first < 0) first = 0;
  const int64_t rel = blk * EPB + el;
  const int64_t i = first + rel;
  const bool valid = (rel < max_new) && (i < n_ent);
  // the entry's cache row, ent_off[b] + i or its pool row in the paged layout, loaded with the
  // row offsets so that the store does not wait for another round trip
  int64_t orow = ent_off[b] + i;
  if (pg.table) {
    int64_t j = i >> pg.eb_shift;
    j = j < pg.max_blocks ? j : pg.max_blocks - 1;
    j = j > 0 ? j : 0;
    orow = ((int64_t)pg.table[(int64_t)b * pg.max_blocks + j] << pg.eb_shift) | (i & ((1 << pg.eb_shift) - 1));
  }

  float mu[8], s[8], acc[8];
#pragma unroll
  for (int d = 0; d < 8; ++d) {
    mu[d] = -INFINITY;
    s[d] = 0.f;
    acc[d] = 0.f;
  }

  if (valid) {
    // virtual chunk rows v < m are series-a raw rows m*i + v of the sequence; with DUAL, rows
    // m <= v < 2m are series-b raw rows m*i + v - 2m (absent for entry 0). Raw row r sits at
    // kv_off[b] + r, or in the paged layout at ring row b * R + (r mod R).
    const bool ring = pg.ring_rows > 0;
    const int64_t rbase = ring ? (int64_t)b * pg.ring_rows : row0;
    const int64_t rmask = ring ? (int64_t)pg.ring_rows - 1 : -1;
    const int64_t base_rel = i * (int64_t)m;
    const int nv = (DUAL && i > 0) ? 2 * m : m;
    // rows handled by this lane: v = rs + NSPLIT * j
    const int my_rows = (nv > rs) ? (nv - rs + NSPLIT - 1) / NSPLIT : 0;
    for (int j0 = 0; j0 < my_rows; j0 += ROWS) {
      u32x4 kr[ROWS], zr[ROWS];
      const int cnt = min(ROWS, my_rows - j0);
#pragma unroll
      for (int u = 0; u < ROWS; ++u) {
        if (u < cnt) {
          const int v = rs + NSPLIT * (j0 + u);
          const bool in_b = DUAL && v >= m;
          const int64_t e = (rbase + ((base_rel + v - (in_b ? 2 * m : 0)) & rmask)) * D + dg * 8;
          kr[u] = *reinterpret_cast<const u32x4*>((in_b ? kv_b : kv) + e);
          if (HAS_Z) zr[u] = *reinterpret_cast<const u32x4*>((in_b ? z_b : z) + e);
        }
      }
      if (HAS_Z) {
        float zl[ROWS][8];
#pragma unroll
        for (int u = 0; u < ROWS; ++u) {
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            zl[u][2 * w] = bf16lo(zr[u][w]) * kLog2e;
            zl[u][2 * w + 1] = bf16hi(zr[u][w]) * kLog2e;
          }
        }
#pragma unroll
        for (int d = 0; d < 8; ++d) {
          float cmax = zl[0][d];
#pragma unroll
          for (int u = 1; u < ROWS; ++u)
            if (u < cnt) cmax = fmaxf(cmax, zl[u][d]);
          const float nmu = fmaxf(mu[d], cmax);
          const float alpha = __builtin_amdgcn_exp2f(mu[d] - nmu);  // 0 on the first step
          s[d] *= alpha;
          acc[d] *= alpha;
          mu[d] = nmu;
        }
#pragma unroll
        for (int u = 0; u < ROWS; ++u) {
          if (u < cnt) {
#pragma unroll
            for (int w = 0; w < 4; ++w) {
              const float e0 = __builtin_amdgcn_exp2f(zl[u][2 * w] - mu[2 * w]);
              const float e1 = __builtin_amdgcn_exp2f(zl[u][2 * w + 1] - mu[2 * w + 1]);
              s[2 * w] += e0;
              s[2 * w + 1] += e1;
              acc[2 * w] = fmaf(e0, bf16lo(kr[u][w]), acc[2 * w]);
              acc[2 * w + 1] = fmaf(e1, bf16hi(kr[u][w]), acc[2 * w + 1]);
            }
          }
        }
      } else {
#pragma unroll
        for (int u = 0; u < ROWS; ++u) {
          if (u < cnt) {
#pragma unroll
            for (int w = 0; w < 4; ++w) {
              acc[2 * w] += bf16lo(kr[u][w]);
              acc[2 * w + 1] += bf16hi(kr[u][w]);
              s[2 * w] += 1.f;
              s[2 * w + 1] += 1.f;
            }
          }
        }
        if (cnt > 0) {
#pragma unroll
          for (int d = 0; d < 8; ++d) mu[d] = 0.f;
        }
      }
    }
  }

  if constexpr (RSX == 1) {
    // one wave per entry: merge the RS partial states pairwise inside the wave (lanes TPE*2^j
    // apart), each pair with its own rescale
#pragma unroll
    for (int step = 1; step < RS; step <<= 1) {
      const int mask = TPE * step;
#pragma unroll
      for (int d = 0; d < 8; ++d) {
        const float mu2 = shfl_xor_f(mu[d], mask);
        const float s2 = shfl_xor_f(s[d], mask);
        const float a2 = shfl_xor_f(acc[d], mask);
        const float M = fmaxf(mu[d], mu2);
        if (M == -INFINITY) continue;  // neither side saw a row
        const float f1 = __builtin_amdgcn_exp2f(mu[d] - M);
        const float f2 = __builtin_amdgcn_exp2f(mu2 - M);
        s[d] = s[d] * f1 + s2 * f2;
        acc[d] = acc[d] * f1 + a2 * f2;
        mu[d] = M;
      }
    }
  } else {
    // an entry split over RSX waves (the few-entry layout of a decode step): merge its NSPLIT
    // partial states in two passes, the maximum logit of each dimension over all splits and
    // then each split's sums rescaled to it once and added up. Inside a wave the splits combine
    // through lane swaps, the waves meet in LDS.
    float M[8];
#pragma unroll
    for (int d = 0; d < 8; ++d) M[d] = splits_reduce<TPE, RS>(mu[d], true);
    __shared__ __align__(16) float xm[EPB][RSX][TPE][8];
    if (rsw == 0) {
#pragma unroll
      for (int d = 0; d < 8; ++d) xm[el][rsx][dg][d] = M[d];
    }
    __syncthreads();
#pragma unroll
    for (int d = 0; d < 8; ++d) M[d] = xm[el][0][dg][d];
#pragma unroll
    for (int w = 1; w < RSX; ++w) {
#pragma unroll
      for (int d = 0; d < 8; ++d) M[d] = fmaxf(M[d], xm[el][w][dg][d]);
    }
#pragma unroll
    for (int d = 0; d < 8; ++d) {
      // a split that saw no row (mu = -inf) adds nothing
      const float f = mu[d] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mu[d] - M[d]);
      s[d] = splits_reduce<TPE, RS>(s[d] * f, false);
      acc[d] = splits_reduce<TPE, RS>(acc[d] * f, false);
    }
    __shared__ __align__(16) float xs[EPB][RSX][TPE][2][8];
    if (rsw == 0 && rsx > 0) {
#pragma unroll
      for (int d = 0; d < 8; ++d) {
        xs[el][rsx][dg][0][d] = s[d];
        xs[el][rsx][dg][1][d] = acc[d];
      }
    }
    __syncthreads();
    if (rsx == 0 && rsw == 0) {
#pragma unroll
      for (int w = 1; w < RSX; ++w) {
#pragma unroll
        for (int d = 0; d < 8; ++d) {
          s[d] += xs[el][w][dg][0][d];
          acc[d] += xs[el][w][dg][1][d];
        }
      }
    }
  }

  if (valid && rs == 0) {
    float o[8];
#pragma unroll
    for (int d = 0; d < 8; ++d) o[d] = acc[d] / s[d];
    store(i, orow, dg, o);
  }
}

// compress_block_to with the entries written to their rows of out (bf16 or fp32)
template <int NT, int TPE, int RS, bool HAS_Z, bool OUT_BF16, int ROWS = 4, int RSX = 1, bool DUAL = false>
__device__ __forceinline__ void compress_block(
    const uint16_t* __restrict__ kv, const uint16_t* __restrict__ z,
    const int64_t* __restrict__ kv_off, const int64_t* __restrict__ ent_off,
    const int64_t* __restrict__ first_entry, int D, int m, int64_t max_new, void* __restrict__ out, int b,
    int64_t blk, const uint16_t* __restrict__ kv_b = nullptr, const uint16_t* __restrict__ z_b = nullptr,
    PagedView pg = PagedView{}) {
  compress_block_to<NT, TPE, RS, HAS_Z, ROWS, RSX, DUAL>(kv, z, kv_off, ent_off, first_entry, D, m, max_new,
                                                         StoreEntry<OUT_BF16>{out, D}, b, blk, kv_b, z_b, pg);
}

}  // namespace csl
