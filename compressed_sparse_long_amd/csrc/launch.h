// Internal launchers: one per kernel family. Host-side validation lives in api.cpp; these
// only pick template instances and grid shapes and enqueue work on the given stream.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace csl {

// Paged heterogeneous cache ([P2] "KV Cache Management"): compressed entries (and CSA
// indexer keys) in a pool of blocks of 2^eb_shift entries, block j of sequence b at pool
// block table[b * max_blocks + j]; raw rows in a per-sequence ring of ring_rows rows, raw
// row r of sequence b at ring row b * ring_rows + r mod ring_rows.
struct PagedView {
  const int32_t* table = nullptr;
  int max_blocks = 0;
  int eb_shift = 0;
  int ring_rows = 0;
  int64_t pool_rows = 0;
  int scale_shift = 0;  // fp8 indexer keys: the group scale of pool row r at k_scale[r >> scale_shift]
};

hipError_t launch_compress(const void* kv, const void* z, const int64_t* kv_off, const int64_t* ent_off,
                           const int64_t* first_entry, int B, int D, int m, int64_t max_new_entries,
                           void* out, bool out_bf16, hipStream_t stream, const PagedView* paged = nullptr);
// CSA's overlapped compression: entry i pools series-a rows [m*i, m*i + m) with series-b rows
// [m*(i-1), m*i) under one softmax per dimension (entry 0: series a alone)
hipError_t launch_compress_overlap(const void* kv_a, const void* z_a, const void* kv_b, const void* z_b,
                                   const int64_t* kv_off, const int64_t* ent_off, const int64_t* first_entry,
                                   int B, int D, int m, int64_t max_new_entries, void* out, bool out_bf16,
                                   hipStream_t stream, const PagedView* paged = nullptr);

// Newest-chunk compression (bf16 out, D = 128, m <= 8; one series or the overlapped pair) that
// the decode indexer can run in spare workgroups of its own launch.
struct CompressJob {
  const void* kv;
  const void* z;
  const int64_t* kv_off;
  const int64_t* first_entry;
  int64_t max_new;
  void* out;
  int m;
  const void* kv_b = nullptr;  // series b of the overlapped compression, or nullptr (one series)
  const void* z_b = nullptr;
};

// key_type: 0 bf16, 1 fp8 e4m3 (k_scale fp32 per scale_group entries), 2 MXFP4 (k_scale
// E8M0 bytes, two per key row)
hipError_t launch_indexer(const void* qI, const float* w, const void* kI, int key_type, const void* k_scale,
                          const int64_t* scale_off, int scale_group, const int64_t* ent_off,
                          const int64_t* q_pos, int m, int B, int T, int HI, int64_t max_entries,
                          float* scores, int64_t ld, void* topk_ws, int topk_k, hipStream_t stream,
                          const CompressJob* job = nullptr, const PagedView* paged = nullptr,
                          bool scores_on_demand = false);
// indexer fused with top-k (no scores written): ids of the k best visible entries per query
// row into idx [B, T, k], ascending, -1 padded; k <= indexer_topk_max_k(HI)
hipError_t launch_indexer_topk(const void* qI, const float* w, const void* kI, int key_type, const void* k_scale,
                               const int64_t* scale_off, int scale_group, const int64_t* ent_off,
                               const int64_t* q_pos, int m, int B, int T, int HI, int64_t max_entries, int k,
                               int32_t* idx, hipStream_t stream, const PagedView* paged = nullptr);
int indexer_topk_max_k(int HI);
// whether launch_indexer leaves top-k candidate lists in topk_ws for these shapes
bool indexer_prepares_topk(const void* topk_ws, int T, int64_t max_entries);
// whether launch_indexer can carry a CompressJob for these shapes (decode tiling, D = 128, m <= 8)
bool indexer_carries_compress(const void* topk_ws, int B, int T, int64_t max_entries, int D, int m);

bool topk_uses_row_kernel(int64_t max_entries);
int64_t topk_max_entries();
size_t topk_workspace_bytes(int B, int T, int64_t max_entries, int k);
int topk_max_k();
// The indexer inputs of a step whose indexer wrote no scores for rows with candidate lists
// (scores on demand): a row whose lists cannot prove its selection gets its scores recomputed,
// with the indexer's arithmetic, into its row of scores before the exact row pass. Packed
// layout, one query row per sequence.
struct RescoreIn {
  const void* qI;
  const float* w;
  const void* kI;
  int key_type;
  const void* k_scale;
  const int64_t* scale_off;
  int scale_group;
  int HI;
};
// whether the finishing kernel can recompute rows for these shapes (one chunk of 8 slots per thread)
bool topk_finish_can_rescore(int64_t max_entries, int k);
hipError_t launch_topk(const float* scores, int64_t ld, const int64_t* ent_off, const int64_t* q_pos, int m,
                       int B, int T, int k, int64_t max_entries, int32_t* idx, void* ws, bool prepared,
                       hipStream_t stream, const RescoreIn* rescore = nullptr);

struct AttnPlan {
  int nsplit;
  int keys_per_split;
  int nsub;  // tiles one workgroup multiplies at once (its waves in nsub groups)
};
// Per-query extras of the core attention: the attention sink (per-head logits added to the
// softmax denominator) and partial RoPE (the query's last rope_dims dims rotated at its
// position p, the output's at -p).
struct AttnExtras {
  const float* sink = nullptr;  // fp32 [H], natural-log logits, or nullptr
  int rope_dims = 0;            // 0 or a multiple of 32 up to 128
  double rope_theta1 = 1.0;     // base^(-2/rope_dims): pair j turns by p * rope_theta1^j
};
// The newest-chunk compression of an HCA step (bf16 entries, D = 128), run by spare
// workgroups of the step's attention launch: entries first_entry[b] .. + max_new of each
// sequence, pooled from kv / z (z nullable) into the cache. Attention workgroups whose key
// range holds such an entry pool it themselves instead of reading the cache.
struct HcaJob {
  const uint16_t* kv = nullptr;
  const uint16_t* z = nullptr;
  const int64_t* first_entry = nullptr;
  int64_t max_new = 0;
  uint16_t* ckv = nullptr;
};
// A CSA row's top-k selection made inside the sparse attention launch, where one workgroup
// per query row covers the row's whole key list: the indexer's scores [B*T, ld] and the
// selection's parameters; the selected ids are also written to the attention's idx buffer.
struct TopkIn {
  const float* scores = nullptr;
  int64_t ld = 0;
  int m = 1;                 // the indexer's compression ratio (visible entries floor(p / m))
  int64_t max_entries = 0;
  int32_t* idx = nullptr;    // [B*T, k]: the selection, also written here
};
AttnPlan attn_plan(int B, int T, int H, int64_t max_keys);
size_t attn_workspace_bytes(int B, int T, int H, int64_t max_keys);
hipError_t launch_attention(bool sparse, const void* q, const void* ckv, const int32_t* idx, int k, const void* kv,
                            const int64_t* kv_off, const int64_t* ent_off, const int64_t* q_pos, int m, int n_win,
                            int B, int T, int H, float scale, int64_t max_entries, int64_t max_keys, float* out,
                            float* lse, void* ws, const AttnExtras& ex, hipStream_t stream,
                            const PagedView* paged = nullptr, const HcaJob* job = nullptr,
                            const TopkIn* topk = nullptr);
// whether launch_attention can carry an HcaJob for these shapes
bool attention_carries_job(int B, int T, int H, int64_t max_keys, int64_t max_new);
// whether the sparse attention launch can make the rows' top-k selection itself (a TopkIn)
bool attention_selects_topk(int B, int T, int H, int k, int64_t max_keys, int64_t max_entries);

}  // namespace csl
