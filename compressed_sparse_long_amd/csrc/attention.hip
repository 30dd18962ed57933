// sparse_attn_decode / hca_attn_decode: shared-KV multi-query attention over a gathered
// key list (selected or all visible compressed entries, then the raw sliding window),
// one softmax over the whole list ([P2] "Deep Dive", CSA core attention and sliding-window
// branch; [P2] "Heavily Compressed Attention"; [P5] the attention formula).
//
// Split-K flash decoding:
//   * a workgroup takes one query row (b, t) and a contiguous range of the row's key list;
//     it has one wave per 16 query heads, all waves sharing one gathered tile;
//   * each 64-key tile is gathered from HBM into LDS twice: row-major K[key][d] for the
//     logits and transposed V^T[d][key] for the value product (K = V), so both MFMA
//     operands are read as contiguous 16- and 8-byte LDS words;
//   * S^T = K Q^T runs as 16x16x32 bf16 MFMAs with keys on M and heads on N, so each
//     lane holds 16 keys of one head and the softmax statistics stay per lane;
//   * an fp32 online softmax in base 2 rescales the O^T accumulators, and the
//     probabilities, rounded to bf16, feed O^T += V^T P^T without leaving registers;
//   * with several splits per row each workgroup writes a normalised partial (o, lse) and
//     a merge kernel combines them with log-sum-exp weights.
#include "device_common.h"
#include "launch.h"

namespace csl {

namespace {

constexpr int kD = 128;
constexpr int kKT = 64;               // keys per tile
constexpr int kKsStride = kD + 8;     // bf16 elements per LDS key row (pad breaks bank aliasing)
constexpr int kVtStride = kKT + 8;    // bf16 elements per LDS transposed row

struct RowGeom {
  int64_t ent_base, n_ent, kv_base, win_lo, win_cnt, nvis;
};

__device__ __forceinline__ RowGeom row_geom(const int64_t* kv_off, const int64_t* ent_off, const int64_t* q_pos,
                                            int b, int t, int m, int n_win, int64_t max_entries) {
  RowGeom g;
  g.ent_base = ent_off[b];
  g.n_ent = ent_off[b + 1] - g.ent_base;
  g.kv_base = kv_off[b];
  const int64_t n_rows = kv_off[b + 1] - g.kv_base;
  const int64_t p = q_pos[b] + t;
  const int64_t hi = p < n_rows - 1 ? p : n_rows - 1;
  if (n_win > 0 && hi >= 0) {
    const int64_t lo = hi - n_win + 1;
    g.win_lo = lo > 0 ? lo : 0;
    g.win_cnt = hi - g.win_lo + 1;
  } else {
    g.win_lo = 0;
    g.win_cnt = 0;
  }
  int64_t nv = (m > 0) ? p / m : 0;
  nv = nv < g.n_ent ? nv : g.n_ent;
  nv = nv < max_entries ? nv : max_entries;
  g.nvis = nv < 0 ? 0 : nv;
  return g;
}

// 16-byte load through a pointer known to address global memory (a pointer that passed
// through LDS as an integer would otherwise become a flat access)
__device__ __forceinline__ u32x4 load_global16(const uint16_t* p) {
  return *(const __attribute__((address_space(1))) u32x4*)(p);
}

template <int NHG, bool SPARSE>
__global__ __launch_bounds__(NHG * 64) void attn_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ ckv, const int32_t* __restrict__ idx, int k,
    const uint16_t* __restrict__ kv, const int64_t* __restrict__ kv_off, const int64_t* __restrict__ ent_off,
    const int64_t* __restrict__ q_pos, int m, int n_win, int T, float scale_log2, int64_t max_entries,
    int keys_per_split, float* __restrict__ out, float* __restrict__ lse_out, float* __restrict__ ws_o,
    float* __restrict__ ws_lse) {
  constexpr int NT = NHG * 64;
  constexpr int H = NHG * 16;
  __shared__ __align__(16) uint16_t Ks[kKT * kKsStride];
  __shared__ __align__(16) uint16_t Vt[kD * kVtStride];
  __shared__ uint64_t rowp[kKT];  // row addresses as integers (0 = masked)
  __shared__ uint64_t tile_valid;  // bit v: slot v of the current tile holds a key

  const int split = blockIdx.x;
  const int row = blockIdx.y;
  const int nrows = gridDim.y;
  const int b = row / T, t = row % T;
  const int tid = threadIdx.x;
  const int wave = tid / kWave;
  const int lane = tid % kWave;
  const int g = lane / 16;
  const int c = lane % 16;

  const int64_t k_lo = (int64_t)split * keys_per_split;
  // the first tile's selected ids do not depend on the row geometry: load them right away.
  // Every thread loads, from a clamped slot (or from q when there is no list), so the load
  // carries no branch and is only awaited where the ids are used.
  const bool has_ids = SPARSE && k > 0;
  const int32_t* id_src = has_ids ? idx + (int64_t)row * k + (k_lo + tid < k ? k_lo + tid : k - 1)
                                  : reinterpret_cast<const int32_t*>(q);
  const int32_t first_raw = *id_src;
  const RowGeom geo = row_geom(kv_off, ent_off, q_pos, b, t, m, n_win, max_entries);
  const int64_t n_comp = SPARSE ? (int64_t)k : geo.nvis;  // compressed slots in the list
  const int64_t L = n_comp + geo.win_cnt;
  const int64_t k_hi = (k_lo + keys_per_split < L) ? k_lo + keys_per_split : L;

  // queries of this wave's 16 heads as MFMA B operands (d-slots 8g..8g+7 of each 32-chunk)
  const int head = wave * 16 + c;
  bf16x8 qb[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk)
    qb[kk] = as_bf16x8(*reinterpret_cast<const u32x4*>(q + ((int64_t)row * H + head) * kD + kk * 32 + g * 8));

  f32x4 oacc[8];
#pragma unroll
  for (int db = 0; db < 8; ++db) oacc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY;
  float l_run = 0.f;

  for (int64_t t0 = k_lo; t0 < k_hi; t0 += kKT) {
    // ---- resolve the 64 slots of this tile to row pointers (nullptr = masked) ----
    if (tid < kKT) {  // kKT slots, one per thread of the first wave
      const int v = tid;
      const int64_t slot = t0 + v;
      const uint16_t* p = nullptr;
      if (slot < k_hi) {
        if (slot < n_comp) {
          int64_t id = slot;
          if (SPARSE) id = (t0 == k_lo) ? (int64_t)(has_ids ? first_raw : -1) : (int64_t)idx[(int64_t)row * k + slot];
          if (id >= 0 && id < geo.n_ent) p = ckv + (geo.ent_base + id) * kD;
        } else {
          const int64_t w = slot - n_comp;
          p = kv + (geo.kv_base + geo.win_lo + w) * kD;
        }
      }
      rowp[v] = reinterpret_cast<uint64_t>(p);
      const uint64_t vb = __ballot(p != nullptr);
      if (v == 0) tile_valid = vb;
    }
    __syncthreads();
    // ---- gather: each thread moves a 4-key x 8-dim block into both LDS layouts ----
    for (int blk = tid; blk < 16 * 16; blk += NT) {
      const int kg = blk / 16;  // keys 4kg..4kg+3
      const int dg = blk % 16;  // dims 8dg..8dg+7
      const uint16_t* pp[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) pp[u] = reinterpret_cast<const uint16_t*>(rowp[4 * kg + u]);
      u32x4 r[4];
#pragma unroll
      for (int u = 0; u < 4; ++u)  // unconditional loads (a masked slot reads row 0) keep all four in flight
        r[u] = load_global16((pp[u] ? pp[u] : ckv) + dg * 8);
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (!pp[u]) r[u] = u32x4{0, 0, 0, 0};
#pragma unroll
      for (int u = 0; u < 4; ++u)
        *reinterpret_cast<u32x4*>(&Ks[(4 * kg + u) * kKsStride + dg * 8]) = r[u];
      // transpose: dim 8dg+2w (low halves) and 8dg+2w+1 (high halves) across the 4 keys
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const uint32_t a0 = r[0][w], a1 = r[1][w], a2 = r[2][w], a3 = r[3][w];
        u32x2 lo, hi;
        lo.x = (a0 & 0xffffu) | (a1 << 16);
        lo.y = (a2 & 0xffffu) | (a3 << 16);
        hi.x = (a0 >> 16) | (a1 & 0xffff0000u);
        hi.y = (a2 >> 16) | (a3 & 0xffff0000u);
        *reinterpret_cast<u32x2*>(&Vt[(dg * 8 + 2 * w) * kVtStride + 4 * kg]) = lo;
        *reinterpret_cast<u32x2*>(&Vt[(dg * 8 + 2 * w + 1) * kVtStride + 4 * kg]) = hi;
      }
    }
    __syncthreads();

    // ---- S^T = K Q^T: 4 key blocks x 4 d-chunks ----
    // all 16 key fragments are read before the first product so LDS latency overlaps
    bf16x8 ka[4][4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
        ka[kk][mb] = as_bf16x8(*reinterpret_cast<const u32x4*>(&Ks[(16 * mb + c) * kKsStride + kk * 32 + g * 8]));
    f32x4 sacc[4];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) sacc[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) sacc[mb] = mfma16x16x32(ka[kk][mb], qb[kk], sacc[mb]);
    // ---- online softmax (base 2) for head c over keys 16mb + 4g + i ----
    const uint64_t valid = tile_valid;
    float x[4][4];
    float mx = -INFINITY;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool ok = (valid >> (16 * mb + 4 * g + i)) & 1ull;
        x[mb][i] = ok ? sacc[mb][i] * scale_log2 : -INFINITY;
        mx = fmaxf(mx, x[mb][i]);
      }
    }
    mx = fmaxf(mx, shfl_xor_f(mx, 16));
    mx = fmaxf(mx, shfl_xor_f(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    float alpha = 1.f;
    float p[4][4];
    if (m_new == -INFINITY) {
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int i = 0; i < 4; ++i) p[mb][i] = 0.f;
    } else {
      alpha = __builtin_amdgcn_exp2f(m_run - m_new);
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int i = 0; i < 4; ++i) p[mb][i] = __builtin_amdgcn_exp2f(x[mb][i] - m_new);
    }
    m_run = m_new;
    float psum = 0.f;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int i = 0; i < 4; ++i) psum += p[mb][i];
    l_run = l_run * alpha + psum;
#pragma unroll
    for (int db = 0; db < 8; ++db) oacc[db] *= alpha;

    // ---- O^T += V^T P^T: 8 d-blocks x 2 key chunks of 32 ----
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      u32x4 pw;
      pw.x = pack_bf16x2(p[2 * s][0], p[2 * s][1]);
      pw.y = pack_bf16x2(p[2 * s][2], p[2 * s][3]);
      pw.z = pack_bf16x2(p[2 * s + 1][0], p[2 * s + 1][1]);
      pw.w = pack_bf16x2(p[2 * s + 1][2], p[2 * s + 1][3]);
      const bf16x8 pb = as_bf16x8(pw);
#pragma unroll
      for (int db = 0; db < 8; ++db) {
        const uint16_t* vr = &Vt[(16 * db + c) * kVtStride + 32 * s + 4 * g];
        const u32x2 v0 = *reinterpret_cast<const u32x2*>(vr);
        const u32x2 v1 = *reinterpret_cast<const u32x2*>(vr + 16);
        const bf16x8 va = as_bf16x8(u32x4{v0.x, v0.y, v1.x, v1.y});
        oacc[db] = mfma16x16x32(va, pb, oacc[db]);
      }
    }
    __syncthreads();  // the next tile overwrites Ks / Vt / rowp
  }

  // ---- finish: reduce the lane-partial denominators across the 4 lane groups ----
  float l = l_run;
  l += shfl_xor_f(l, 16);
  l += shfl_xor_f(l, 32);
  const bool empty = !(l > 0.f);
  const float inv = empty ? 0.f : 1.f / l;
  const float lse = empty ? -INFINITY : (m_run + __log2f(l)) * kLn2;

  const bool single = (gridDim.x == 1);
  float* o_dst = single ? out + ((int64_t)row * H + head) * kD
                        : ws_o + (((int64_t)split * nrows + row) * H + head) * kD;
#pragma unroll
  for (int db = 0; db < 8; ++db) {
    const f32x4 v = oacc[db] * inv;
    *reinterpret_cast<float4*>(o_dst + 16 * db + 4 * g) = make_float4(v[0], v[1], v[2], v[3]);
  }
  if (g == 0) {
    if (single) {
      if (lse_out) lse_out[(int64_t)row * H + head] = lse;
    } else {
      ws_lse[((int64_t)split * nrows + row) * H + head] = lse;
    }
  }
}

// Log-sum-exp merge of the split partials: one thread per (query row, head, dim). Splits are
// consumed 8 at a time with all their loads issued together and an online rescale.
__global__ __launch_bounds__(256) void attn_merge_kernel(const float* __restrict__ ws_o, const float* __restrict__ ws_lse,
                                                         int nsplit, int nrows, int H, float* __restrict__ out,
                                                         float* __restrict__ lse_out) {
  constexpr int CH = 8;
  const int row = blockIdx.x;
  const int e = blockIdx.y * 256 + threadIdx.x;  // (head, dim) index inside the row
  if (e >= H * kD) return;
  const int h = e / kD;
  const int d = e % kD;
  const float* lse_p = ws_lse + (int64_t)row * H + h;
  const float* o_p = ws_o + ((int64_t)row * H + h) * kD + d;
  const int64_t lse_stride = (int64_t)nrows * H;
  const int64_t o_stride = lse_stride * kD;
  float M = -INFINITY, acc = 0.f, wsum = 0.f;
  for (int c0 = 0; c0 < nsplit; c0 += CH) {
    float ls[CH], o[CH];
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      const int s = c0 + j;
      ls[j] = (s < nsplit) ? lse_p[s * lse_stride] : -INFINITY;
      o[j] = (s < nsplit) ? o_p[s * o_stride] : 0.f;
    }
    float cm = -INFINITY;
#pragma unroll
    for (int j = 0; j < CH; ++j) cm = fmaxf(cm, ls[j]);
    const float Mn = fmaxf(M, cm);
    if (Mn == -INFINITY) continue;  // no split so far saw a key
    const float r = __expf(M - Mn);  // 0 while M is still -inf
    acc *= r;
    wsum *= r;
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      const float wgt = (ls[j] == -INFINITY) ? 0.f : __expf(ls[j] - Mn);
      acc = fmaf(wgt, o[j], acc);
      wsum += wgt;
    }
    M = Mn;
  }
  out[((int64_t)row * H + h) * kD + d] = (M == -INFINITY) ? 0.f : acc / wsum;
  if (d == 0 && lse_out) lse_out[(int64_t)row * H + h] = (M == -INFINITY) ? -INFINITY : M + __logf(wsum);
}

template <bool SPARSE>
hipError_t launch_nhg(int H, dim3 grid, hipStream_t st, const uint16_t* q, const uint16_t* ckv, const int32_t* idx,
                      int k, const uint16_t* kv, const int64_t* kv_off, const int64_t* ent_off, const int64_t* q_pos,
                      int m, int n_win, int T, float scale_log2, int64_t max_entries, int kps, float* out,
                      float* lse, float* ws_o, float* ws_lse) {
#define CSL_ATTN_CASE(NHG)                                                                                   \
  case NHG:                                                                                                  \
    attn_kernel<NHG, SPARSE><<<grid, NHG * 64, 0, st>>>(q, ckv, idx, k, kv, kv_off, ent_off, q_pos, m, n_win, \
                                                        T, scale_log2, max_entries, kps, out, lse, ws_o, ws_lse); \
    break;
  switch (H / 16) {
    CSL_ATTN_CASE(1)
    CSL_ATTN_CASE(2)
    CSL_ATTN_CASE(3)
    CSL_ATTN_CASE(4)
    CSL_ATTN_CASE(5)
    CSL_ATTN_CASE(6)
    CSL_ATTN_CASE(7)
    CSL_ATTN_CASE(8)
    default: return hipErrorInvalidValue;
  }
#undef CSL_ATTN_CASE
  return hipGetLastError();
}

}  // namespace

AttnPlan attn_plan(int B, int T, int64_t max_keys) {
  AttnPlan p;
  const int64_t rows = (int64_t)B * T;
  const int64_t tiles = max_keys > 0 ? (max_keys + kKT - 1) / kKT : 1;
  int64_t want = rows >= 512 ? 1 : (1024 + rows - 1) / rows;  // aim for ~1024 workgroups
  if (want > tiles) want = tiles;
  if (want < 1) want = 1;
  const int64_t tps = (tiles + want - 1) / want;
  p.keys_per_split = (int)(tps * kKT);
  p.nsplit = (int)((tiles + tps - 1) / tps);
  return p;
}

size_t attn_workspace_bytes(int B, int T, int H, int64_t max_keys) {
  const AttnPlan p = attn_plan(B, T, max_keys);
  if (p.nsplit <= 1) return 0;
  return (size_t)p.nsplit * B * T * H * (kD + 1) * sizeof(float);
}

hipError_t launch_attention(bool sparse, const void* q, const void* ckv, const int32_t* idx, int k, const void* kv,
                            const int64_t* kv_off, const int64_t* ent_off, const int64_t* q_pos, int m, int n_win,
                            int B, int T, int H, float scale, int64_t max_entries, int64_t max_keys, float* out,
                            float* lse, void* ws, hipStream_t st) {
  const AttnPlan p = attn_plan(B, T, max_keys);
  const int rows = B * T;
  float* ws_o = static_cast<float*>(ws);
  float* ws_lse = ws_o ? ws_o + (size_t)p.nsplit * rows * H * kD : nullptr;
  dim3 grid((unsigned)p.nsplit, (unsigned)rows);
  const float sl2 = scale * kLog2e;
  const uint16_t* q16 = static_cast<const uint16_t*>(q);
  const uint16_t* c16 = static_cast<const uint16_t*>(ckv);
  const uint16_t* k16 = static_cast<const uint16_t*>(kv);
  hipError_t e = sparse ? launch_nhg<true>(H, grid, st, q16, c16, idx, k, k16, kv_off, ent_off, q_pos, m, n_win, T, sl2,
                                           max_entries, p.keys_per_split, out, lse, ws_o, ws_lse)
                        : launch_nhg<false>(H, grid, st, q16, c16, idx, k, k16, kv_off, ent_off, q_pos, m, n_win, T,
                                            sl2, max_entries, p.keys_per_split, out, lse, ws_o, ws_lse);
  if (e != hipSuccess || p.nsplit <= 1) return e;
  attn_merge_kernel<<<dim3((unsigned)rows, (unsigned)((H * kD + 255) / 256)), 256, 0, st>>>(ws_o, ws_lse, p.nsplit,
                                                                                             rows, H, out, lse);
  return hipGetLastError();
}

}  // namespace csl
