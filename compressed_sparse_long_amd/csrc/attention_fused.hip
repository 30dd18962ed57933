// The HCA step's fused attention launches: dense attention whose spare workgroups pool the
// step's new entries (HcaJob), in a unit of its own so that it compiles beside attention.hip.
#include "attention_kernel.h"

namespace csl {

hipError_t launch_attention_fused(bool rope, bool paged, int H, dim3 grid, hipStream_t st, const uint16_t* q,
                                  const uint16_t* ckv, const uint16_t* kv, const int64_t* kv_off,
                                  const int64_t* ent_off, const int64_t* q_pos, int m, int n_win, int T,
                                  float scale_log2, int64_t max_entries, const AttnPlan& p, float* out, float* lse,
                                  float* ws_o, float* ws_lse, float2* ws_rope, const AttnExtras& ex,
                                  const AttnLayout& lay, int rows, const HcaJob& job) {
#define CSL_FUSED(RP, PG)                                                                                       \
  launch_nhg<false, RP, PG, true>(H, grid, st, q, ckv, nullptr, 0, kv, kv_off, ent_off, q_pos, m, n_win, T,    \
                                  scale_log2, max_entries, p, out, lse, ws_o, ws_lse, ws_rope, ex, lay, rows, job,   \
                                  nullptr)
  if (paged) return rope ? CSL_FUSED(true, true) : CSL_FUSED(false, true);
  return rope ? CSL_FUSED(true, false) : CSL_FUSED(false, false);
#undef CSL_FUSED
}

}  // namespace csl
