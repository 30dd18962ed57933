// sparse_attn_decode / hca_attn_decode launches: the split plan, the workspace layout and the
// merge (the kernels are in attention_kernel.h).
#include "attention_kernel.h"

namespace csl {

// tiles multiplied at once by a decode workgroup of H heads: 4 (2 at 128 heads, whose workgroup
// already has 8 waves per tile) for head counts of 16, 32, 64 or 128, else 1
static int attn_nsub(int H) {
  switch (H) {
    case 16: case 32: case 64: return 4;
    case 128: return 2;
    default: return 1;
  }
}

AttnPlan attn_plan(int B, int T, int H, int64_t max_keys) {
  AttnPlan p;
  const int64_t rows = (int64_t)B * T;
  const int64_t tiles = max_keys > 0 ? (max_keys + kKT - 1) / kKT : 1;
  // a short key list (at most nsub tiles) in one workgroup that multiplies its tiles at once:
  // no partials and no merge. Longer lists use several workgroups: each matrix core then
  // multiplies fewer tiles than it would for a wave group of its own per tile
  p.nsub = 1;
  const int nsub = attn_nsub(H);
  if (rows < 512 && nsub > 1 && tiles > 1 && tiles <= nsub) {
    p.nsub = nsub;
    p.keys_per_split = nsub * kKT;
    p.nsplit = 1;
    return p;
  }
  // aim for about two workgroups per CU, with at least two tiles per split when the list has
  // them: a workgroup walking several tiles prefetches them, while every extra split adds a
  // partial (o, lse) to write and merge
  int64_t want = rows >= 512 ? 1 : (512 + rows - 1) / rows;
  if (want > (tiles + 1) / 2) want = (tiles + 1) / 2;
  if (want < 1) want = 1;
  const int64_t tps = (tiles + want - 1) / want;
  p.keys_per_split = (int)(tps * kKT);
  p.nsplit = (int)((tiles + tps - 1) / tps);
  return p;
}

size_t attn_workspace_bytes(int B, int T, int H, int64_t max_keys) {
  const AttnPlan p = attn_plan(B, T, H, max_keys);
  if (p.nsplit <= 1) return 0;
  // partials (o, lse) of every split, then one RoPE (cos, sin) table per row
  return (size_t)p.nsplit * B * T * H * (kD + 1) * sizeof(float) + (size_t)B * T * (kRope / 2) * sizeof(float2);
}

bool attention_carries_job(int B, int T, int H, int64_t max_keys, int64_t max_new) {
  // the job rides in plans of one tile per wave group (no parallel-tile groups), with at most
  // kHzMax new entries per sequence: a split pools those it finds rewritten into a side buffer
  // of that many rows before its own state is live
  const AttnPlan p = attn_plan(B, T, H, max_keys);
  return (H == 16 || H == 32 || H == 64 || H == 128) && max_new >= 1 && max_new <= kHzMax &&
         (int64_t)B * T + (int64_t)B * max_new <= 65535 && p.nsub == 1;
}

bool attention_selects_topk(int B, int T, int H, int k, int64_t max_keys, int64_t max_entries) {
  // one workgroup per query row holding the whole key list (the parallel-tile plan), whose
  // threads hold the row's scores (kSelItems each) and whose LDS holds its k selected slots
  const AttnPlan p = attn_plan(B, T, H, max_keys);
  if (p.nsub <= 1 || k < 1 || k > kSelMax) return false;
  const int64_t threads = (int64_t)(H / 16) * p.nsub * kWave;
  return max_entries >= 1 && max_entries <= kSelItems * threads;
}

hipError_t launch_attention(bool sparse, const void* q, const void* ckv, const int32_t* idx, int k, const void* kv,
                            const int64_t* kv_off, const int64_t* ent_off, const int64_t* q_pos, int m, int n_win,
                            int B, int T, int H, float scale, int64_t max_entries, int64_t max_keys, float* out,
                            float* lse, void* ws, const AttnExtras& ex, hipStream_t st, const PagedView* paged,
                            const HcaJob* job, const TopkIn* topk) {
  if (job && (sparse || !attention_carries_job(B, T, H, max_keys, job->max_new))) return hipErrorInvalidValue;
  if (topk && (!sparse || job || paged || !topk->scores || !topk->idx || topk->m < 1 ||
               !attention_selects_topk(B, T, H, k, max_keys, topk->max_entries)))
    return hipErrorInvalidValue;
  const AttnPlan p = attn_plan(B, T, H, max_keys);
  AttnLayout lay;
  if (paged) {
    lay.table = paged->table;
    lay.max_blocks = paged->max_blocks;
    lay.eb_shift = paged->eb_shift;
    lay.ring_rows = paged->ring_rows;
  }
  const int rows = B * T;
  // the workspace exists only with several splits (attn_workspace_bytes is 0 otherwise): one
  // split writes its output directly and never touches it
  float* ws_o = p.nsplit > 1 ? static_cast<float*>(ws) : nullptr;
  float* ws_lse = ws_o ? ws_o + (size_t)p.nsplit * rows * H * kD : nullptr;
  // the rows' RoPE tables follow the partials (8-byte aligned: the partials are whole rows
  // of 16 heads); only the merge reads them
  float2* ws_rope = ws_o ? reinterpret_cast<float2*>(ws_lse + (size_t)p.nsplit * rows * H) : nullptr;
  // with a job, the grid's first B * max_new rows are its workgroups
  const HcaJob none{};
  const HcaJob& hj = job ? *job : none;
  const int64_t grid_rows = rows + (job ? (int64_t)B * job->max_new : 0);
  dim3 grid((unsigned)p.nsplit, (unsigned)grid_rows);
  const float sl2 = scale * kLog2e;
  const uint16_t* q16 = static_cast<const uint16_t*>(q);
  const uint16_t* c16 = static_cast<const uint16_t*>(ckv);
  const uint16_t* k16 = static_cast<const uint16_t*>(kv);
#define CSL_ATTN_NHG(SP, RP, PG, FU)                                                                            \
  launch_nhg<SP, RP, PG, FU>(H, grid, st, q16, c16, idx, k, k16, kv_off, ent_off, q_pos, m, n_win, T, sl2,     \
                             max_entries, p, out, lse, ws_o, ws_lse, ws_rope, ex, lay, rows, hj, topk)
  const bool rope = ex.rope_dims > 0;
  hipError_t e;
  if (job)
    e = launch_attention_fused(rope, paged != nullptr, H, grid, st, q16, c16, k16, kv_off, ent_off, q_pos, m, n_win,
                               T, sl2, max_entries, p, out, lse, ws_o, ws_lse, ws_rope, ex, lay, rows, hj);
  else if (paged)
    e = sparse ? (rope ? CSL_ATTN_NHG(true, true, true, false) : CSL_ATTN_NHG(true, false, true, false))
               : (rope ? CSL_ATTN_NHG(false, true, true, false) : CSL_ATTN_NHG(false, false, true, false));
  else
    e = sparse ? (rope ? CSL_ATTN_NHG(true, true, false, false) : CSL_ATTN_NHG(true, false, false, false))
               : (rope ? CSL_ATTN_NHG(false, true, false, false) : CSL_ATTN_NHG(false, false, false, false));
#undef CSL_ATTN_NHG
  if (e != hipSuccess || p.nsplit <= 1) return e;
  const dim3 mgrid((unsigned)rows, (unsigned)((H * kD + 255) / 256));
#define CSL_MERGE(CH)                                                                                         \
  attn_merge_kernel<CH><<<mgrid, 256, 0, st>>>(ws_o, ws_lse, p.nsplit, rows, H, out, lse, ex.sink, \
                                               ex.rope_dims > 0, ws_rope)
  if (p.nsplit <= 8)
    CSL_MERGE(8);
  else if (p.nsplit <= 16)
    CSL_MERGE(16);
  else
    CSL_MERGE(32);
#undef CSL_MERGE
  return hipGetLastError();
}

}  // namespace csl
