// The attention kernels of sparse_attn_decode / hca_attn_decode, shared by attention.hip and
// attention_fused.hip (the launches that also carry an HCA step's compression): shared-KV
// multi-query attention over a gathered key list (selected or all visible compressed entries,
// then the raw sliding window), one softmax over the whole list ([P2] "Deep Dive", CSA core
// attention and sliding-window branch; [P2] "Heavily Compressed Attention"; [P5] the
// attention formula).
//
// Split-K flash decoding:
//   * a workgroup takes one query row (b, t) and a contiguous range of the row's key list;
//     it has one wave per 16 query heads, all waves sharing one gathered tile;
//   * each 64-key tile is gathered from HBM into one row-major LDS tile K[key][d] (K = V),
//     XOR-swizzled by 16-byte units so that its writes and both kinds of reads are free of
//     bank conflicts;
//   * S^T = K Q^T runs as 16x16x32 bf16 MFMAs with keys on M and heads on N, so each
//     lane holds 16 keys of one head and the softmax statistics stay per lane;
//   * an fp32 online softmax in base 2 (rescaling only when the maximum grows by more than
//     2^8) feeds the probabilities, each split into a bf16 high part and a bf16 residual, to
//     O^T += V^T P^T; the V^T operand comes from the same tile through gfx950's
//     transposing LDS reads;
//   * a split of one or two tiles gathers all its rows in one round trip; a workgroup that
//     walks more tiles loads the next tile's rows while the current one is multiplied;
//   * with several splits per row each workgroup writes a normalised partial (o, lse) and
//     a merge kernel combines them with log-sum-exp weights;
//   * optional per-query extras ([P1] sections 7 and 8): the attention sink, a per-head logit
//     whose exponential joins the final softmax denominator with no value, and partial RoPE:
//     the query's last 64 dims are rotated at its position p before the scores (kept exact
//     as a bf16 pair, like the probabilities) and the output's last 64 dims at -p after
//     normalisation. Both act where the row's result is final: in the single-split
//     epilogue or in the merge;
//   * FUSED (an HCA step): rows of the grid before the query rows are workgroups that pool the
//     step's new entries into the cache, and a workgroup whose keys include an entry being
//     rewritten pools it from the raw rows into its tile instead of reading the cache;
//   * TOPK (a CSA step whose rows each fit one workgroup): the workgroup selects its row's
//     top-k from the indexer's scores itself (topk_short.h), into LDS and the id buffer, and
//     gathers from that selection.
#pragma once

#include <type_traits>

#include "compress_common.h"
#include "device_common.h"
#include "launch.h"
#include "topk_short.h"

namespace csl {

// The paged cache as the attention reads it: entry e of sequence b at pool row
// table[b * max_blocks + (e >> eb_shift)] << eb_shift | (e & mask); raw rows in rings
struct AttnLayout {
  const int32_t* table = nullptr;
  int max_blocks = 0;
  int eb_shift = 0;
  int ring_rows = 0;                         // 0: raw rows packed in kv; else a power-of-two ring
};

namespace {


constexpr int kD = 128;
constexpr int kKT = 64;               // keys per tile
constexpr int kRope = 64;             // partial RoPE: the last 64 dims ([P1] section 8)
constexpr int kRopeOff = kD - kRope;  // first rotated dim
constexpr int kRopeKK = kRopeOff / 32;  // first rotated 32-dim chunk of the query operand
constexpr int kHzMax = 4;  // FUSED: most entries a split can find rewritten (max_new <= this)
constexpr int kSelItems = 4;   // TOPK: scores per thread, so rows of up to 4 * threads entries
constexpr int kSelMax = 256;   // TOPK: most selected slots (a one-workgroup plan holds 4 tiles)

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

// The K tile in LDS: 64 rows of 256 bytes (16 units of 16 bytes, no padding); unit U of row r
// sits at position U ^ ks_swz(r). The swizzle keeps every LDS access of the kernel free of
// bank conflicts: the gather's writes (4 rows x 64 contiguous bytes per 16 lanes), the 16-byte
// K-operand reads (16 rows of one unit) and the transposing 8-byte V-operand reads (4 rows x
// 2 units per 16 lanes). It is linear over the row's low 4 bits.
__device__ __forceinline__ int ks_swz(int r) {
  return ((r & 1) ? 4 : 0) ^ ((r & 2) ? 10 : 0) ^ ((r & 4) ? 1 : 0) ^ ((r & 8) ? 2 : 0);
}

// gfx950 transposing LDS read: within each 16-lane group, lanes 4j..4j+3 name 4 consecutive
// 16-bit values each (row j, 16 values), and lane i receives value i of rows 0..3.
__device__ __forceinline__ u32x2 lds_read_tr16(const uint8_t* lds_base, int byte_off) {
  typedef short v4s __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) v4s lds_v4s;
  lds_v4s* p = (lds_v4s*)((__attribute__((address_space(3))) uint8_t*)(lds_base) + byte_off);
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(p));
}

// (cos, sin) of RoPE pair j at position p: the angle p * theta1^j (theta1 = base^(-2/R)) is
// formed in double, in revolutions, and reduced to [-1/2, 1/2] there (p reaches 2^20 and
// more, where a float angle would be off by hundredths of a radian); the hardware sine and
// cosine, which take revolutions, finish in float. theta1^j comes from square-and-multiply
// over j's 6 bits.
__device__ __forceinline__ float2 rope_cs(int64_t p, int j, double theta1) {
  double th = 1.0, sq = theta1;
#pragma unroll
  for (int bit = 0; bit < 6; ++bit) {
    if (j & (1 << bit)) th *= sq;
    sq *= sq;
  }
  double rev = (double)p * th * 0.15915494309189535;  // 1 / (2 pi)
  rev -= rint(rev);
  const float f = (float)rev;
  return make_float2(__builtin_amdgcn_cosf(f), __builtin_amdgcn_sinf(f));
}

// A score must exceed the running maximum (base-2 logits) by more than this before the
// accumulators are rescaled; in between, probabilities are taken relative to the stale
// maximum and stay below 2^8, which fp32 sums and bf16 probabilities hold without loss.
constexpr float kRescaleSlack = 8.f;

// One 64-key tile from LDS for this wave's 16 heads: S^T = K Q^T (keys on M, heads on N), the
// online softmax in base 2 (vld[v] != 0: slot v holds a key), and O^T += V^T P^T with each
// probability split into two bf16 terms. V^T comes from the same row-major tile through
// transposing reads.
template <bool ROPE>
__device__ __forceinline__ void tile_compute(const uint8_t* Ks, const uint8_t* vld, const bf16x8 (&qb)[4],
                                             const bf16x8 (&ql)[4], float scale_log2, f32x4 (&oacc)[8],
                                             float& m_run, float& l_run, int c, int g) {
  // K operand: lane (c, g) takes key 16mb + c, dims 32kk + 8g.. (unit 4kk + g); every row
  // 16mb + c shares the swizzle of row c
  const int swc = ks_swz(c);
  f32x4 sacc[4];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) sacc[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
  bf16x8 ka[4][4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    const int koff = c * 256 + 16 * ((4 * kk + g) ^ swc);
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      ka[kk][mb] = as_bf16x8(*reinterpret_cast<const u32x4*>(Ks + koff + mb * 16 * 256));
      sacc[mb] = mfma16x16x32(ka[kk][mb], qb[kk], sacc[mb]);
    }
  }
  if (ROPE) {
    // rotated query chunks carry a bf16 residual: a second product per block keeps q.k exact
    // to fp32 (issued after all the main products, so no product waits on its own block's)
#pragma unroll
    for (int kk = kRopeKK; kk < 4; ++kk)
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) sacc[mb] = mfma16x16x32(ka[kk][mb], ql[kk], sacc[mb]);
  }
  // this lane's 16 keys are 16mb + 4g + i; a tile with every slot filled skips the masking
  uint32_t okw[4];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) okw[mb] = *reinterpret_cast<const uint32_t*>(&vld[16 * mb + 4 * g]);
  const bool full = __builtin_amdgcn_ballot_w64((okw[0] & okw[1] & okw[2] & okw[3]) != 0x01010101u) == 0;
  float mx = -INFINITY;
  if (full) {
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int i = 0; i < 4; ++i) mx = fmaxf(mx, sacc[mb][i]);
  } else {
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool ok = (okw[mb] >> (8 * i)) & 0xffu;
        sacc[mb][i] = ok ? sacc[mb][i] : -INFINITY;
        mx = fmaxf(mx, sacc[mb][i]);
      }
  }
  mx = xor_max<16>(mx);
  mx = xor_max<32>(mx);
  mx *= scale_log2;  // scale > 0, so the maximum commutes with the scaling
  if (__builtin_amdgcn_ballot_w64(mx > m_run + kRescaleSlack) != 0) {
    const float m_new = fmaxf(m_run, mx);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);  // 0 while nothing was seen
    l_run *= alpha;
#pragma unroll
    for (int db = 0; db < 8; ++db) oacc[db] *= alpha;
    m_run = m_new;
  }
  // p = 2^(s * scale - m); before the first key m is -inf and every p of the tile is masked
  const float nm = m_run == -INFINITY ? 0.f : -m_run;
  float p[4][4];
  float psum = 0.f;
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      p[mb][i] = __builtin_amdgcn_exp2f(fmaf(sacc[mb][i], scale_log2, nm));
      psum += p[mb][i];
    }
  l_run += psum;
  // O^T += V^T P^T: 8 d-blocks x 2 key chunks of 32. The A operand of lane (c, g) holds dim
  // 16db + c of keys 32s + 4g + 0..3 and 32s + 16 + 4g + 0..3 (the key order of P's k-slots);
  // in the transposing read the lane names row 32s (+16) + 4g + c/4 and dims 16db + 4(c%4)..
  const int rv = 4 * g + (c >> 2);
  const int swv = ks_swz(rv);
  // Each probability enters as a bf16 pair p = hi + lo (lo = bf16(p - hi)), two products per
  // block: the pair carries p to about 2^-16 relative, so the value product is as exact as
  // its fp32 accumulation, where one bf16 would round every weight by up to 2^-9.
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const float* pp0 = p[2 * s];
    const float* pp1 = p[2 * s + 1];
    u32x4 hw, lw;
    hw.x = pack_bf16x2(pp0[0], pp0[1]);
    hw.y = pack_bf16x2(pp0[2], pp0[3]);
    hw.z = pack_bf16x2(pp1[0], pp1[1]);
    hw.w = pack_bf16x2(pp1[2], pp1[3]);
    auto lo_pair = [](uint32_t h, float a, float b) {
      return pack_bf16x2(a - __uint_as_float(h << 16), b - __uint_as_float(h & 0xffff0000u));
    };
    lw.x = lo_pair(hw.x, pp0[0], pp0[1]);
    lw.y = lo_pair(hw.y, pp0[2], pp0[3]);
    lw.z = lo_pair(hw.z, pp1[0], pp1[1]);
    lw.w = lo_pair(hw.w, pp1[2], pp1[3]);
    const bf16x8 ph = as_bf16x8(hw), pl = as_bf16x8(lw);
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      const int voff = rv * 256 + 8 * (c & 1) + 16 * ((2 * db + ((c >> 1) & 1)) ^ swv) + 32 * s * 256;
      const u32x2 v0 = lds_read_tr16(Ks, voff);
      const u32x2 v1 = lds_read_tr16(Ks, voff + 16 * 256);
      const bf16x8 va = as_bf16x8(u32x4{v0.x, v0.y, v1.x, v1.y});
      oacc[db] = mfma16x16x32(va, ph, oacc[db]);
      oacc[db] = mfma16x16x32(va, pl, oacc[db]);
    }
  }
}

// Common epilogue: normalise and write the output (one split) or the partial (o, lse). The
// single-split output is final: the sink joins its denominator and its last R dims rotate
// at -p (rcs holds the (cos, sin) of the row's R/2 RoPE pairs).
template <bool ROPE>
__device__ __forceinline__ void attn_write(const f32x4 (&oacc)[8], float m_run, float l_run, int row, int nrows,
                                           int split, int H, int head, int g, float* __restrict__ out,
                                           float* __restrict__ lse_out, float* __restrict__ ws_o,
                                           float* __restrict__ ws_lse, const float* __restrict__ sink,
                                           const float2* rcs) {
  // reduce the lane-partial denominators across the 4 lane groups
  float l = l_run;
  l = xor_sum<16>(l);
  l = xor_sum<32>(l);
  const bool single = (gridDim.x == 1);
  // sink logit in base 2 (-inf without a sink; partials never take it)
  const float zs = (single && sink) ? sink[head] * kLog2e : -INFINITY;
  const float M = fmaxf(l > 0.f ? m_run : -INFINITY, zs);
  float inv = 0.f, lse = -INFINITY;
  if (M != -INFINITY) {
    const float a = l > 0.f ? __builtin_amdgcn_exp2f(m_run - M) : 0.f;
    const float den = l * a + __builtin_amdgcn_exp2f(zs - M);
    inv = a / den;
    lse = (M + __log2f(den)) * kLn2;
  }
  float* o_dst = single ? out + ((int64_t)row * H + head) * kD : ws_o + (((int64_t)split * nrows + row) * H + head) * kD;
#pragma unroll
  for (int db = 0; db < 8; ++db) {
    f32x4 v = oacc[db] * inv;
    if (ROPE && single && 16 * db >= kRopeOff) {
      // dims 16db + 4g + 0..3 are two pairs; rotate each at -p
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const float2 cs = rcs[(16 * db + 4 * g + 2 * i - kRopeOff) >> 1];
        const float x0 = v[2 * i], x1 = v[2 * i + 1];
        v[2 * i] = x0 * cs.x + x1 * cs.y;
        v[2 * i + 1] = x1 * cs.x - x0 * cs.y;
      }
    }
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

// Merge of one wave's online-softmax state (o, m, l; base-2 logits) into another's: the two
// states cover disjoint key sets of the same 16 heads.
__device__ __forceinline__ void merge_state(f32x4 (&o)[8], float& m, float& l, const float (&o2)[32], float m2,
                                            float l2) {
  const float M = fmaxf(m, m2);
  if (M == -INFINITY) return;  // neither side saw a key
  const float f1 = __builtin_amdgcn_exp2f(m - M), f2 = __builtin_amdgcn_exp2f(m2 - M);
#pragma unroll
  for (int db = 0; db < 8; ++db)
#pragma unroll
    for (int i = 0; i < 4; ++i) o[db][i] = o[db][i] * f1 + o2[4 * db + i] * f2;
  l = l * f1 + l2 * f2;
  m = M;
}

// Attention over one query row's key range. Each thread gathers whole 64-byte pieces of rows:
// pair p = j * NT + tid takes row p / 4, units 4q + p % 4 (q = 0..3), so 4 lanes read 64
// contiguous bytes per load and a thread resolves one row address per row it gathers.
// MODE 1 or 2: the range is at most that many tiles, all gathered at once (one round trip)
// and then multiplied; this is the decode shape, where a lone workgroup would otherwise wait
// for each tile's rows in turn. MODE 0: the workgroup walks many tiles and loads the next
// tile's rows (and the selected ids of the one after) into registers while the current tile
// is multiplied.
// NSUB > 1 (with MODE 1): the workgroup holds NSUB tiles at once and its waves are NSUB groups
// of NHG, group s multiplying tile s, so the tiles' latencies overlap; the groups' states are
// then merged through LDS into group 0, which writes the result.
template <int NHG, int NSUB, bool SPARSE, int MODE, bool ROPE, bool PAGED, bool FUSED = false, bool TOPK = false>
__global__ __launch_bounds__(NHG * NSUB * 64) void attn_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ ckv, const int32_t* __restrict__ idx, int k,
    const uint16_t* __restrict__ kv, const int64_t* __restrict__ kv_off, const int64_t* __restrict__ ent_off,
    const int64_t* __restrict__ q_pos, int m, int n_win, int T, int H, float scale_log2, int64_t max_entries,
    int keys_per_split, float* __restrict__ out, float* __restrict__ lse_out, float* __restrict__ ws_o,
    float* __restrict__ ws_lse, const float* __restrict__ sink, double rope_theta1,
    float2* __restrict__ ws_rope, AttnLayout lay, int nrows, HcaJob job, TopkIn tk) {
  constexpr bool MULTI = MODE == 0;
  static_assert(NSUB == 1 || MODE == 1, "parallel tiles take single-round splits of one tile each");
  static_assert(!FUSED || (NSUB == 1 && !SPARSE), "a fused launch is dense, one tile per wave group");
  static_assert(!TOPK || (SPARSE && !FUSED && !MULTI), "the selection feeds a one-round sparse gather");
  constexpr int NTL = MULTI ? 1 : (NSUB > 1 ? NSUB : MODE);  // tiles held in LDS at once
  constexpr int NT = NHG * NSUB * 64;
  constexpr int NV = kKT * NTL;            // rows gathered per round
  constexpr int NP = 4 * NV;               // gather pairs per round
  constexpr int RPT = (NP + NT - 1) / NT;  // pairs (rows) per thread
  static_assert(RPT <= 32, "one mask bit per gathered row");
  constexpr size_t kTileBytes = (size_t)kKT * kD * 2;
  constexpr size_t kTilesBytes = NTL * kTileBytes;
  // the tiles' LDS, shared at the end with the states of wave groups 1..NSUB-1 for the merge:
  // per wave 32 output values, m and l, for each of 64 lanes
  constexpr size_t kMergeBytes = (size_t)(NSUB - 1) * NHG * 34 * kWave * 4;
  constexpr size_t kKsBytes = kTilesBytes > kMergeBytes ? kTilesBytes : kMergeBytes;
  __shared__ __align__(16) uint8_t Ks_raw[kKsBytes];
  uint8_t (*Ks)[kTileBytes] = reinterpret_cast<uint8_t (*)[kTileBytes]>(Ks_raw);
  __shared__ __align__(16) uint8_t vld[NTL][kKT];  // slot v of a tile holds a key
  __shared__ __align__(16) uint8_t hz_rows[FUSED ? kHzMax : 1][kD * 2];  // FUSED: entries pooled here
  __shared__ float2 rcs_all[ROPE ? NHG * NSUB : 1][kRope / 2];  // RoPE (cos, sin) per pair at the row's position, per wave

  const int split = blockIdx.x;
  // FUSED: the grid's first rows are the step's compression (dispatched first, so that it
  // starts with the attention rather than after it), then the query rows
  const int njob = FUSED ? (int)gridDim.y - nrows : 0;
  const int row = (int)blockIdx.y - njob;
  const PagedView jpg{lay.table, lay.max_blocks, lay.eb_shift, lay.ring_rows};
  if (FUSED && row < 0) {
    // workgroup (0, j) takes new entry j % max_new of sequence j / max_new, written to its
    // cache row
    if (split == 0) {
      const int jb = (int)blockIdx.y;
      const int bj = (int)(jb / job.max_new);
      const int64_t blk = jb % job.max_new;
      if (job.z)
        compress_block_to<NT, 16, 4, true, 8, NT / 64, false>(job.kv, job.z, kv_off, ent_off, job.first_entry, kD,
                                                             m, job.max_new, StoreEntry<true>{job.ckv, kD}, bj, blk,
                                                             nullptr, nullptr, jpg);
      else
        compress_block_to<NT, 16, 4, false, 8, NT / 64, false>(job.kv, job.z, kv_off, ent_off, job.first_entry, kD,
                                                              m, job.max_new, StoreEntry<true>{job.ckv, kD}, bj, blk,
                                                              nullptr, nullptr, jpg);
    }
    return;
  }
  const int b = row / T, t = row % T;
  const int tid = threadIdx.x;
  const int wave = tid / kWave;
  const int lane = tid % kWave;
  const int g = lane / 16;
  const int c = lane % 16;
  const int hg = wave % NHG;   // head group: heads 16 hg .. 16 hg + 15
  const int sub = wave / NHG;  // tile of the round this wave multiplies (NSUB > 1)

  const int64_t k_lo = (int64_t)split * keys_per_split;
  // TOPK: the row's selection, made below while the window rows are in flight, into LDS (and
  // the id buffer, for the caller)
  __shared__ int32_t sel[TOPK ? kSelMax : 1];
  __shared__ std::conditional_t<TOPK, ShortTopkLds<NT, kSelItems>, char> sel_lds;
  // selected ids do not depend on the row geometry: the first ones load right away, from
  // clamped slots (or from q when there is no list), so the loads carry no branch
  const bool has_ids = SPARSE && k > 0;
  const int32_t* idx_row = has_ids ? idx + (int64_t)row * k : reinterpret_cast<const int32_t*>(q);
  auto load_ids = [&](int64_t t0, int32_t (&ids)[RPT]) {
#pragma unroll
    for (int j = 0; j < RPT; ++j) {
      const int64_t slot = t0 + (j * NT + tid) / 4;
      const int64_t cs = has_ids ? (slot < k ? slot : k - 1) : 0;
      ids[j] = TOPK ? sel[cs] : idx_row[cs];
    }
  };
  int32_t ids_cur[RPT], ids_nxt[RPT];
  if (TOPK) {
#pragma unroll
    for (int j = 0; j < RPT; ++j) ids_cur[j] = 0;  // (the window rows issued first read no id)
  } else {
    load_ids(k_lo, ids_cur);
  }
  if (MULTI) load_ids(k_lo + NV, ids_nxt);
  const RowGeom geo = row_geom(kv_off, ent_off, q_pos, b, t, m, n_win, max_entries);
  const int64_t n_comp = SPARSE ? (int64_t)k : geo.nvis;  // compressed slots in the list
  // first entry this launch's compression rewrites (FUSED)
  int64_t f_new = 0;
  if (FUSED && job.first_entry) {
    f_new = job.first_entry[b];
    f_new = f_new > 0 ? f_new : 0;
  }
  const int64_t L = n_comp + geo.win_cnt;
  const int64_t k_hi = (k_lo + keys_per_split < L) ? k_lo + keys_per_split : L;

  // Row addresses as integers, computed without branches. Slot t0 + v of a round (v < NV) is
  // a compressed entry while v < n_comp - t0 and holds a key while v < k_hi - t0; both limits
  // are clamped to [0, NV] so the per-slot tests are 32-bit.
  // Entry e of the sequence is ckv row ent_off[b] + e or, in the paged layout, the pool row
  // its block table gives (looked up here, between the id and the row loads). Window slot
  // s (s >= n_comp) is raw row win_lo + s - n_comp of the sequence: kv row kv_off[b] + that,
  // or ring row b * R + (that mod R) in the paged layout.
  const uint64_t ckv_a = reinterpret_cast<uint64_t>(ckv);
  const uint64_t ent_a = ckv_a + (uint64_t)(PAGED ? 0 : geo.ent_base) * (kD * 2);
  const uint32_t n_ent32 = (uint32_t)(geo.n_ent < 0x7fffffff ? geo.n_ent : 0x7fffffff);
  const int32_t* tbl = PAGED ? lay.table + (int64_t)b * lay.max_blocks : nullptr;
  const uint32_t emask = PAGED ? (1u << lay.eb_shift) - 1u : 0u;
  const bool ring = PAGED && lay.ring_rows > 0;
  const uint64_t wmask = ring ? (uint64_t)(lay.ring_rows - 1) : ~0ull;
  const uint64_t wrow0 = ring ? (uint64_t)b * lay.ring_rows : (uint64_t)(geo.kv_base + geo.win_lo - n_comp);
  const uint64_t woff = ring ? (uint64_t)(geo.win_lo - n_comp) : 0ull;  // wraps for compressed slots: unused there
  const uint64_t kv_a = reinterpret_cast<uint64_t>(kv);
  const uint64_t win_a = kv_a + wrow0 * (kD * 2);  // packed layout: slot s at win_a + s rows
  auto clamp_round = [](int64_t x) { return (int)(x < 0 ? 0 : (x > NV ? NV : x)); };
  u32x4 r[RPT][4];
  uint32_t okm = 0;  // bit j: pair j's row holds a key
  // part 0: every row of the round; 1: its window rows only; 2: its compressed entries only
  auto issue = [&](int64_t t0, const int32_t (&ids)[RPT], int part) {
    const int lim_c = clamp_round(n_comp - t0), lim_h = clamp_round(k_hi - t0);

    if (part != 2) okm = 0;
#pragma unroll
    for (int j = 0; j < RPT; ++j) {
      const int pr = j * NT + tid;
      const bool in = (j + 1) * NT <= NP || pr < NP;
      const int v = pr / 4;
      const uint32_t e = SPARSE ? (uint32_t)ids[j] : (uint32_t)(t0 + v);  // negative ids wrap to huge
      const bool comp = v < lim_c;
      if (part != 0 && comp != (part == 2)) continue;
      const bool ok = in && v < lim_h && (!comp || e < n_ent32);
      uint64_t erow = e;
      if (PAGED) {  // the entry's pool row (a clamped table slot where it is not used)
        uint32_t j = (comp && ok) ? (e >> lay.eb_shift) : 0u;
        j = j < (uint32_t)lay.max_blocks ? j : (uint32_t)lay.max_blocks - 1u;
        erow = ((uint64_t)(uint32_t)tbl[j] << lay.eb_shift) | (e & emask);
      }
      const uint64_t a = comp ? ent_a + erow * (kD * 2)
                              : (PAGED ? kv_a + (wrow0 + ((woff + (uint64_t)(t0 + v)) & wmask)) * (kD * 2)
                                       : win_a + (uint64_t)(t0 + v) * (kD * 2));
      okm |= (ok ? 1u : 0u) << j;
      const uint16_t* src = reinterpret_cast<const uint16_t*>(ok ? a : ckv_a) + 8 * (pr % 4);
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) r[j][qq] = load_global16(src + 32 * qq);  // unconditional: masked rows read row 0
    }
  };

  // FUSED: entries of this split that the launch's compression rewrites (at most max_new <=
  // kHzMax) are not read from the cache. The workgroup pools them itself first, with the same
  // arithmetic and before its own state is live, into a side buffer that the gather copies
  // into their tile slots in whichever round holds them.
  int64_t hz_lo = 0, hz_hi = 0;
  if (FUSED) {
    hz_lo = k_lo > f_new ? k_lo : f_new;
    hz_hi = f_new + job.max_new;
    hz_hi = hz_hi < n_comp ? hz_hi : n_comp;
    hz_hi = hz_hi < k_hi ? hz_hi : k_hi;
    for (int64_t e = hz_lo; e < hz_hi; ++e) {  // uniform
      auto to_tile = [&](int64_t i, int64_t, int dg, const float (&o)[8]) {
        u32x4 w;
        w.x = pack_bf16x2(o[0], o[1]);
        w.y = pack_bf16x2(o[2], o[3]);
        w.z = pack_bf16x2(o[4], o[5]);
        w.w = pack_bf16x2(o[6], o[7]);
        *reinterpret_cast<u32x4*>(hz_rows[i - hz_lo] + 16 * dg) = w;
      };
      if (job.z)
        compress_block_to<NT, 16, 4, true, 8, NT / 64, false>(job.kv, job.z, kv_off, ent_off, job.first_entry, kD, m,
                                                             job.max_new, to_tile, b, e - f_new, nullptr, nullptr,
                                                             jpg);
      else
        compress_block_to<NT, 16, 4, false, 8, NT / 64, false>(job.kv, job.z, kv_off, ent_off, job.first_entry, kD,
                                                              m, job.max_new, to_tile, b, e - f_new, nullptr, nullptr,
                                                              jpg);
    }
    if (hz_lo < hz_hi) __syncthreads();  // the side rows are read by other threads of the gather
  }

  // queries of this wave's 16 heads as MFMA B operands (d-slots 8g..8g+7 of each 32-chunk)
  const int head = hg * 16 + c;
  bf16x8 qb[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk)
    qb[kk] = as_bf16x8(*reinterpret_cast<const u32x4*>(q + ((int64_t)row * H + head) * kD + kk * 32 + g * 8));
  // with prefetching, the query and id loads complete before the first row loads: inside the
  // tile loop the compiler then knows the query operands have arrived and the products do not
  // wait for the prefetch
  if (MULTI) __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));

  f32x4 oacc[8];
#pragma unroll
  for (int db = 0; db < 8; ++db) oacc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY;
  float l_run = 0.f;

  if constexpr (TOPK) {
    // the window rows depend on no selection: they are in flight while the workgroup selects
    // the row's entries (no store precedes the selection's barriers, so they wait for no
    // load), then the selected entries follow
    if (k_lo < k_hi) issue(k_lo, ids_cur, 1);
    const int64_t n = visible_entries(ent_off, q_pos, b, t, tk.m, tk.max_entries);
    short_row_topk<NT, kSelItems>(tk.scores + (int64_t)row * tk.ld, tk.max_entries, n, k, sel,
                                  tk.idx + (int64_t)row * k, sel_lds);
    __syncthreads();
    load_ids(k_lo, ids_cur);
    if (k_lo < k_hi) issue(k_lo, ids_cur, 2);
  } else {
    if (k_lo < k_hi) issue(k_lo, ids_cur, 0);
  }

  // partial RoPE: the row's (cos, sin) table, then the rotated query chunks as bf16 pairs.
  // Every wave builds its own copy, so no workgroup barrier (which would also wait for the
  // gathered rows in flight) stands between the table and its readers; the first split
  // also leaves the table in the workspace for the merge. The table needs only the row's
  // position, so it is built while the rows are in flight; the rotation needs the query,
  // whose loads may be queued behind the rows', so a single-round kernel rotates once the
  // rows have landed (the prefetching loop has its query in registers before the rows go
  // out).
  float2* rcs = rcs_all[ROPE ? wave : 0];
  bf16x8 ql[4];
  if (ROPE) {
    const int64_t p = q_pos[b] + t;
    if (lane < kRope / 2) {
      const float2 cs = rope_cs(p, lane, rope_theta1);
      rcs[lane] = cs;
      if (ws_rope && split == 0 && wave == 0) ws_rope[(int64_t)row * (kRope / 2) + lane] = cs;
    }
    // the wave's own LDS writes, ordered before its reads (in-wave: no hardware wait needed)
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    __builtin_amdgcn_wave_barrier();
  }
  auto rotate_q = [&]() {
#pragma unroll
    for (int kk = kRopeKK; kk < 4; ++kk) {
      const u32x4 w = __builtin_bit_cast(u32x4, qb[kk]);
      const uint32_t wv[4] = {w.x, w.y, w.z, w.w};
      uint32_t hv[4], lv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {  // dims 32kk + 8g + 2i, +1: pair (32kk + 8g + 2i - kRopeOff) / 2
        const float2 cs = rcs[(32 * kk + 8 * g + 2 * i - kRopeOff) >> 1];
        const float x0 = bf16lo(wv[i]), x1 = bf16hi(wv[i]);
        const float y0 = x0 * cs.x - x1 * cs.y;
        const float y1 = x0 * cs.y + x1 * cs.x;
        const uint32_t h = pack_bf16x2(y0, y1);
        hv[i] = h;
        lv[i] = pack_bf16x2(y0 - bf16lo(h), y1 - bf16hi(h));
      }
      qb[kk] = as_bf16x8(u32x4{hv[0], hv[1], hv[2], hv[3]});
      ql[kk] = as_bf16x8(u32x4{lv[0], lv[1], lv[2], lv[3]});
    }
  };
  if (ROPE && MULTI) rotate_q();

  for (int64_t t0 = k_lo; t0 < k_hi; t0 += NV) {
    // this round's rows (in flight since the previous round) into the swizzled K tiles
#pragma unroll
    for (int j = 0; j < RPT; ++j) {
      const int pr = j * NT + tid;
      if ((j + 1) * NT > NP && pr >= NP) break;
      const int v = pr / 4, u = pr % 4;
      const int tl = v / kKT, vr = v % kKT;
      const bool ok = (okm >> j) & 1u;
      const int sw = ks_swz(vr);
      // (FUSED: a slot the workgroup pooled itself takes its row from the side buffer)
      const bool own = FUSED && t0 + v >= hz_lo && t0 + v < hz_hi;
      if (own) {
        const uint8_t* src = hz_rows[FUSED ? t0 + v - hz_lo : 0];
#pragma unroll
        for (int qq = 0; qq < 4; ++qq)
          *reinterpret_cast<u32x4*>(Ks[tl] + vr * 256 + 16 * ((4 * qq + u) ^ sw)) =
              *reinterpret_cast<const u32x4*>(src + 16 * (4 * qq + u));
      } else {
#pragma unroll
        for (int qq = 0; qq < 4; ++qq)
          *reinterpret_cast<u32x4*>(Ks[tl] + vr * 256 + 16 * ((4 * qq + u) ^ sw)) = ok ? r[j][qq] : u32x4{0, 0, 0, 0};
      }
      if (u == 0) vld[tl][vr] = ok ? 1 : 0;
    }
    __syncthreads();
    if (ROPE && !MULTI) rotate_q();  // single round: the rows (and so the query) have landed
    // the next round's rows and the ids two rounds ahead go out while this one computes
    if (MULTI && t0 + NV < k_hi) {
      issue(t0 + NV, ids_nxt, 0);
      if (SPARSE && t0 + 2 * NV < k_hi) load_ids(t0 + 2 * NV, ids_nxt);
    }
    if (NSUB > 1) {
      if (sub == 0 || t0 + sub * kKT < k_hi)
        tile_compute<ROPE>(Ks[sub], vld[sub], qb, ql, scale_log2, oacc, m_run, l_run, c, g);
    } else {
#pragma unroll
      for (int tl = 0; tl < NTL; ++tl)
        if (tl == 0 || t0 + tl * kKT < k_hi)
          tile_compute<ROPE>(Ks[tl], vld[tl], qb, ql, scale_log2, oacc, m_run, l_run, c, g);
    }
    if (!MULTI) break;  // the launch gives single-round kernels at most NTL tiles
    __syncthreads();    // the next tile overwrites Ks / vld
  }
  if (NSUB > 1) {
    // groups 1..NSUB-1 post their states (lane-major, so each LDS access is one contiguous row
    // of 64 words) over the tiles, which every wave has finished reading; group 0 merges them
    float* ms = reinterpret_cast<float*>(Ks_raw);
    __syncthreads();
    if (sub > 0) {
      float* dst = ms + (size_t)((sub - 1) * NHG + hg) * 34 * kWave + lane;
#pragma unroll
      for (int db = 0; db < 8; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i) dst[(4 * db + i) * kWave] = oacc[db][i];
      dst[32 * kWave] = m_run;
      dst[33 * kWave] = l_run;
    }
    __syncthreads();
    if (sub > 0) return;
#pragma unroll
    for (int s2 = 1; s2 < NSUB; ++s2) {
      const float* src = ms + (size_t)((s2 - 1) * NHG + hg) * 34 * kWave + lane;
      float o2[32];
#pragma unroll
      for (int i = 0; i < 32; ++i) o2[i] = src[i * kWave];
      merge_state(oacc, m_run, l_run, o2, src[32 * kWave], src[33 * kWave]);
    }
  }
  attn_write<ROPE>(oacc, m_run, l_run, row, nrows, split, H, head, g, out, lse_out, ws_o, ws_lse, sink, rcs);
}

// Log-sum-exp merge of the split partials: one thread per (query row, head, dim). Splits are
// consumed CH at a time with all their loads issued together and an online rescale; the
// launch picks CH >= nsplit when it can, so the merge waits on memory once.
// The merged row is final: the sink joins the denominator and, with RoPE, each thread's dim
// is rotated at -p together with its pair partner (the neighbouring lane), with the row's
// (cos, sin) table that the attention kernel left in the workspace.
template <int CH>
__global__ __launch_bounds__(256) void attn_merge_kernel(const float* __restrict__ ws_o, const float* __restrict__ ws_lse,
                                                         int nsplit, int nrows, int H, float* __restrict__ out,
                                                         float* __restrict__ lse_out, const float* __restrict__ sink,
                                                         bool rope, const float2* __restrict__ ws_rope) {
  const int row = blockIdx.x;
  const int e = blockIdx.y * 256 + threadIdx.x;  // (head, dim) index inside the row
  if (e >= H * kD) return;
  const int h = e / kD;
  const int d = e % kD;
  // issued with the partials' loads: the pair's (cos, sin), read once the merge is done
  const float2 cs = (rope && d >= kRopeOff) ? ws_rope[(int64_t)row * (kRope / 2) + ((d - kRopeOff) >> 1)]
                                            : make_float2(1.f, 0.f);
  const float* lse_p = ws_lse + (int64_t)row * H + h;
  const float* o_p = ws_o + ((int64_t)row * H + h) * kD + d;
  const int64_t lse_stride = (int64_t)nrows * H;
  const int64_t o_stride = lse_stride * kD;
  float M = -INFINITY, acc = 0.f, wsum = 0.f;
  for (int c0 = 0; c0 < nsplit; c0 += CH) {
    float ls[CH], o[CH];
#pragma unroll
    for (int j = 0; j < CH; ++j) {  // clamped split index: every load is issued, none branches
      const int s = c0 + j < nsplit ? c0 + j : nsplit - 1;
      ls[j] = lse_p[s * lse_stride];
      o[j] = o_p[s * o_stride];
    }
#pragma unroll
    for (int j = 0; j < CH; ++j)
      if (c0 + j >= nsplit) ls[j] = -INFINITY;
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
  float den = wsum;
  if (sink) {  // the sink joins the denominator with no value
    const float z = sink[h];
    const float Mf = fmaxf(M, z);
    if (Mf != -INFINITY) {
      const float a = (M == -INFINITY) ? 0.f : __expf(M - Mf);
      acc *= a;
      den = wsum * a + __expf(z - Mf);
      M = Mf;
    }
  }
  float o = (M == -INFINITY) ? 0.f : acc / den;
  if (rope) {  // uniform: every lane takes part in the exchange
    const float partner = __shfl_xor(o, 1, kWave);
    if (d >= kRopeOff) o = (d & 1) ? o * cs.x - partner * cs.y : o * cs.x + partner * cs.y;
  }
  out[((int64_t)row * H + h) * kD + d] = o;
  if (d == 0 && lse_out) lse_out[(int64_t)row * H + h] = (M == -INFINITY) ? -INFINITY : M + __logf(den);
}

template <bool SPARSE, bool ROPE, bool PAGED, bool FUSED>
hipError_t launch_nhg(int H, dim3 grid, hipStream_t st, const uint16_t* q, const uint16_t* ckv, const int32_t* idx,
                      int k, const uint16_t* kv, const int64_t* kv_off, const int64_t* ent_off, const int64_t* q_pos,
                      int m, int n_win, int T, float scale_log2, int64_t max_entries, const AttnPlan& p, float* out,
                      float* lse, float* ws_o, float* ws_lse, float2* ws_rope, const AttnExtras& ex,
                      const AttnLayout& lay, int rows, const HcaJob& job, const TopkIn* topk) {
  const int kps = p.keys_per_split;
  const int tiles = kps / kKT;  // 1 or 2: gathered in one round; more: the prefetching loop
  // a fused launch carries the step's compression only for head counts of 16, 32, 64 or 128
  if (FUSED && H != 16 && H != 32 && H != 64 && H != 128) return hipErrorInvalidValue;
  // the rows' own top-k selection rides only in one-workgroup plans of the packed sparse gather
  if (topk && (p.nsub <= 1 || !SPARSE || PAGED || FUSED)) return hipErrorInvalidValue;
  const TopkIn tki = topk ? *topk : TopkIn{};
#define CSL_ATTN_LAUNCH_T(NHG, NSUB, MODE, TK)                                                                  \
  attn_kernel<NHG, NSUB, SPARSE, MODE, ROPE, PAGED, FUSED, TK><<<grid, NHG * NSUB * 64, 0, st>>>(             \
      q, ckv, idx, k, kv, kv_off, ent_off, q_pos, m, n_win, T, H, scale_log2, max_entries, kps, out, lse, ws_o, \
      ws_lse, ex.sink, ex.rope_theta1, ws_rope, lay, rows, job, tki)
#define CSL_ATTN_LAUNCH(NHG, NSUB, MODE) CSL_ATTN_LAUNCH_T(NHG, NSUB, MODE, false)
  if (p.nsub > 1) {  // a row's whole key list in one workgroup, its tiles multiplied at once
    if constexpr (FUSED) {
      return hipErrorInvalidValue;  // (its LDS holds no room for the job)
    } else {
#define CSL_ATTN_PAR(NHG, NSUB)                           \
  case NHG:                                              \
    if (p.nsub != NSUB) return hipErrorInvalidValue;       \
    if constexpr (SPARSE && !PAGED) {                    \
      if (topk)                                          \
        CSL_ATTN_LAUNCH_T(NHG, NSUB, 1, true);           \
      else                                               \
        CSL_ATTN_LAUNCH(NHG, NSUB, 1);                   \
    } else {                                             \
      CSL_ATTN_LAUNCH(NHG, NSUB, 1);                     \
    }                                                    \
    break;
      switch (H / 16) {
        CSL_ATTN_PAR(1, 4)
        CSL_ATTN_PAR(2, 4)
        CSL_ATTN_PAR(4, 4)
        CSL_ATTN_PAR(8, 2)
        default: return hipErrorInvalidValue;
      }
#undef CSL_ATTN_PAR
      return hipGetLastError();
    }
  }
#define CSL_ATTN_CASE(NHG)                 \
  case NHG:                                \
    if (tiles == 1)                        \
      CSL_ATTN_LAUNCH(NHG, 1, 1);          \
    else if (tiles == 2)                   \
      CSL_ATTN_LAUNCH(NHG, 1, 2);          \
    else                                   \
      CSL_ATTN_LAUNCH(NHG, 1, 0);          \
    break;
  if constexpr (FUSED) {
    switch (H / 16) {
      CSL_ATTN_CASE(1)
      CSL_ATTN_CASE(2)
      CSL_ATTN_CASE(4)
      CSL_ATTN_CASE(8)
      default: return hipErrorInvalidValue;
    }
  } else {
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
  }
#undef CSL_ATTN_CASE
#undef CSL_ATTN_LAUNCH
#undef CSL_ATTN_LAUNCH_T
  return hipGetLastError();
}

}  // namespace

// launch_nhg for the HCA step's fused launches (dense, with an HcaJob), compiled in its own unit
hipError_t launch_attention_fused(bool rope, bool paged, int H, dim3 grid, hipStream_t st, const uint16_t* q,
                                  const uint16_t* ckv, const uint16_t* kv, const int64_t* kv_off,
                                  const int64_t* ent_off, const int64_t* q_pos, int m, int n_win, int T,
                                  float scale_log2, int64_t max_entries, const AttnPlan& p, float* out, float* lse,
                                  float* ws_o, float* ws_lse, float2* ws_rope, const AttnExtras& ex,
                                  const AttnLayout& lay, int rows, const HcaJob& job);

}  // namespace csl
