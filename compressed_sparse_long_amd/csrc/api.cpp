// C ABI of the library: host-side argument validation, thread-local error text, and the
// hand-off to the kernel launchers. Nothing here allocates device memory or synchronises.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>

#include "../../include/csl.h"
#include "launch.h"

namespace {

thread_local std::string g_last_error;

int fail(int status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}

int ok() {
  g_last_error.clear();
  return CSL_OK;
}

int hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(CSL_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

constexpr int kMaxGridY = 65535;

}  // namespace

extern "C" {

const char* csl_last_error(void) { return g_last_error.c_str(); }

int csl_version(void) { return 500; }

}  // extern "C"

namespace {

// Validation halves of the entry points: CSL_OK when the arguments are good (the launch may
// still have nothing to do), an error status (with the message set) otherwise.
int check_compress(const void* kv, const void* z, const int64_t* kv_off, const int64_t* ent_off, int B, int D, int m,
                   int64_t max_new_entries, const void* out, int out_dtype, const char* who = "compress_kv") {
  if (B < 0 || max_new_entries < 0) return fail(CSL_ERR_INVALID, "%s: negative B or max_new_entries", who);
  if (!kv || !kv_off || !ent_off || !out) return fail(CSL_ERR_INVALID, "%s: null pointer argument", who);
  if (m < 1 || m > 65536) return fail(CSL_ERR_INVALID, "%s: m must be in [1, 65536], got %d", who, m);
  if (D != 64 && D != 128 && D != 256 && D != 512)
    return fail(CSL_ERR_UNSUPPORTED, "%s: D must be 64, 128, 256 or 512, got %d", who, D);
  if (out_dtype != CSL_DTYPE_F32 && out_dtype != CSL_DTYPE_BF16)
    return fail(CSL_ERR_UNSUPPORTED, "%s: out_dtype must be F32 or BF16", who);
  if (B > kMaxGridY) return fail(CSL_ERR_UNSUPPORTED, "%s: B must be <= %d", who, kMaxGridY);
  if (!aligned(kv, 16) || (z && !aligned(z, 16)) || !aligned(out, 16))
    return fail(CSL_ERR_INVALID, "%s: kv, z and out must be 16-byte aligned", who);
  return CSL_OK;
}

// series b of the overlapped compression: kv_b given, its logits exactly when series a has them
int check_series_b(const void* kv_b, const void* z_a, const void* z_b, const char* who) {
  if (!kv_b) return fail(CSL_ERR_INVALID, "%s: null kv_b", who);
  if ((z_a == nullptr) != (z_b == nullptr))
    return fail(CSL_ERR_INVALID, "%s: z and z_b must both be given or both be NULL", who);
  if (!aligned(kv_b, 16) || (z_b && !aligned(z_b, 16)))
    return fail(CSL_ERR_INVALID, "%s: kv_b and z_b must be 16-byte aligned", who);
  return CSL_OK;
}

// The paged cache descriptor: a table of pool blocks (a power-of-two number of entries each)
// and a power-of-two ring of raw rows per sequence; fills the launchers' view.
int check_paged(const char* who, const csl_paged_cache* pc, int B, csl::PagedView& pv) {
  if (!pc->block_table) return fail(CSL_ERR_INVALID, "%s: paged cache without a block table", who);
  if (pc->max_blocks < 1 || pc->block_entries < 1 || (pc->block_entries & (pc->block_entries - 1)))
    return fail(CSL_ERR_INVALID, "%s: paged cache needs max_blocks >= 1 and a power-of-two block_entries", who);
  if (pc->ring_rows < 0 || (pc->ring_rows & (pc->ring_rows - 1)))
    return fail(CSL_ERR_INVALID, "%s: ring_rows must be 0 or a power of two", who);
  if (pc->pool_entries < 0 || pc->pool_entries > 0x7fffffff)
    return fail(CSL_ERR_INVALID, "%s: pool_entries must be in [0, 2^31)", who);
  if ((int64_t)B * pc->max_blocks > ((int64_t)1 << 40)) return fail(CSL_ERR_INVALID, "%s: block table too large", who);
  pv.table = pc->block_table;
  pv.max_blocks = pc->max_blocks;
  pv.eb_shift = __builtin_ctz((unsigned)pc->block_entries);
  pv.ring_rows = pc->ring_rows;
  pv.pool_rows = pc->pool_entries;
  return CSL_OK;
}

// fp8 indexer keys in the paged pool keep their group scales per block: the scale of pool row r
// is k_scale[r >> scale_shift], one scale per group of a block (groups smaller than a block) or
// one per block (a group spanning blocks, its scale repeated in each). Groups are powers of two,
// so a group never straddles a block boundary without covering the whole block.
int check_paged_scales(const char* who, int k_dtype, int scale_group, csl::PagedView& pv) {
  if (k_dtype != CSL_DTYPE_FP8_E4M3) return CSL_OK;
  if (scale_group < 1 || (scale_group & (scale_group - 1)))
    return fail(CSL_ERR_INVALID, "%s: fp8 keys in a paged cache need a power-of-two scale_group, got %d", who,
                scale_group);
  const int lg = __builtin_ctz((unsigned)scale_group);
  pv.scale_shift = lg < pv.eb_shift ? lg : pv.eb_shift;
  return CSL_OK;
}

// The per-sequence ring of raw rows must hold every raw row a call reads at once: the window
// of each of the T query rows (rows p - n_win + 1 .. p for p = q_pos + t, the newest rows of a
// context whose queries sit at its end: n_win + T - 1 rows) and the chunks being compressed
// (entries first_entry .. first_entry + max_new - 1, the newest ones: max_new chunks of m rows,
// one more for overlapped compression's series b, and up to m - 1 rows of uncompressed tail).
// Both are suffixes of the sequence, so the larger one covers their union. Nothing to check
// without a ring (raw rows packed as kv_off says).
int check_ring(const char* who, const csl_paged_cache* pc, int n_win, int T, int m, int64_t max_new, bool overlap) {
  if (!pc || pc->ring_rows == 0) return CSL_OK;
  int64_t need = 0;
  if (n_win > 0 && T > 0) need = (int64_t)n_win + T - 1;
  if (max_new > 0) {
    const int64_t comp = (max_new + (overlap ? 2 : 1)) * (int64_t)m - 1;
    need = comp > need ? comp : need;
  }
  if ((int64_t)pc->ring_rows < need)
    return fail(CSL_ERR_INVALID,
                "%s: ring_rows (%d) must hold every raw row the call reads: %lld (window n_win + T - 1, "
                "compressed chunks (max_new_entries + %d) * m - 1)",
                who, pc->ring_rows, (long long)need, overlap ? 2 : 1);
  return CSL_OK;
}

// the launcher's key type: 0 bf16, 1 fp8 e4m3, 2 MXFP4
int key_type(int k_dtype) {
  return k_dtype == CSL_DTYPE_FP8_E4M3 ? 1 : k_dtype == CSL_DTYPE_MXFP4 ? 2 : 0;
}

// topk_ws is cleared when the shapes need no candidate lists
int check_indexer(const void* q_idx, const float* w, const void* k_idx, int k_dtype, const void* k_scale,
                  const int64_t* scale_off, int scale_group, const int64_t* ent_off, const int64_t* q_pos, int m, int B,
                  int T, int HI, int CI, int64_t max_entries, const float* scores, int64_t ld, void*& topk_ws,
                  size_t topk_ws_bytes, int topk_k, const char* who = "indexer_scores", bool paged = false) {
  if (B < 0 || T < 0 || max_entries < 0) return fail(CSL_ERR_INVALID, "%s: negative size", who);
  if (!q_idx || !w || !k_idx || !ent_off || !q_pos || !scores)
    return fail(CSL_ERR_INVALID, "%s: null pointer argument", who);
  if (m < 1) return fail(CSL_ERR_INVALID, "%s: m must be >= 1", who);
  if (k_dtype != CSL_DTYPE_BF16 && k_dtype != CSL_DTYPE_FP8_E4M3 && k_dtype != CSL_DTYPE_MXFP4)
    return fail(CSL_ERR_UNSUPPORTED, "%s: k_dtype must be BF16, FP8_E4M3 or MXFP4", who);
  const bool fp8 = k_dtype == CSL_DTYPE_FP8_E4M3;
  const bool fp4 = k_dtype == CSL_DTYPE_MXFP4;
  // (in a paged cache the scales follow the pool rows and scale_off is not used)
  if (fp8 && (!k_scale || (!scale_off && !paged) || scale_group < 1))
    return fail(CSL_ERR_INVALID, "%s: fp8 keys need k_scale, scale_off and scale_group >= 1", who);
  if (fp4 && !k_scale) return fail(CSL_ERR_INVALID, "%s: MXFP4 keys need their E8M0 scales in k_scale", who);
  if (HI != 1 && HI != 2 && HI != 4 && HI != 8 && HI != 16)
    return fail(CSL_ERR_UNSUPPORTED, "%s: HI must be 1, 2, 4, 8 or 16, got %d", who, HI);
  if (CI != 64) return fail(CSL_ERR_UNSUPPORTED, "%s: CI must be 64, got %d", who, CI);
  if (ld < max_entries) return fail(CSL_ERR_INVALID, "%s: ld (%lld) < max_entries (%lld)", who,
                                    (long long)ld, (long long)max_entries);
  if (B > kMaxGridY) return fail(CSL_ERR_UNSUPPORTED, "%s: B must be <= %d", who, kMaxGridY);
  const int kalign = (fp8 || fp4) ? 8 : 16;
  if (!aligned(q_idx, 16) || !aligned(k_idx, kalign))
    return fail(CSL_ERR_INVALID, "%s: q_idx must be 16-byte and k_idx %d-byte aligned", who, kalign);
  if (topk_ws) {
    if (topk_k < 1 || topk_k > csl::topk_max_k())
      return fail(CSL_ERR_UNSUPPORTED, "%s: topk_k must be in [1, %d], got %d", who, csl::topk_max_k(), topk_k);
    const size_t need = csl_topk_workspace_bytes(B, T, max_entries, topk_k);
    if (topk_ws_bytes < need)
      return fail(CSL_ERR_WORKSPACE, "%s: top-k workspace of %zu bytes required, got %zu", who, need,
                  topk_ws_bytes);
    if (!aligned(topk_ws, 16)) return fail(CSL_ERR_INVALID, "%s: topk_ws must be 16-byte aligned", who);
    if (need == 0) topk_ws = nullptr;  // short rows: the selection needs no candidate lists
  }
  return CSL_OK;
}

int check_topk(const float* scores, int64_t ld, const int64_t* ent_off, const int64_t* q_pos, int m, int B, int T,
               int k, int64_t max_entries, const int32_t* idx, const void* ws, size_t ws_bytes) {
  if (B < 0 || T < 0 || max_entries < 0) return fail(CSL_ERR_INVALID, "topk_select: negative size");
  if (!scores || !ent_off || !q_pos || !idx) return fail(CSL_ERR_INVALID, "topk_select: null pointer argument");
  if (m < 1) return fail(CSL_ERR_INVALID, "topk_select: m must be >= 1");
  if (k < 1 || k > csl::topk_max_k())
    return fail(CSL_ERR_UNSUPPORTED, "topk_select: k must be in [1, %d], got %d", csl::topk_max_k(), k);
  if (max_entries > csl::topk_max_entries())
    return fail(CSL_ERR_UNSUPPORTED, "topk_select: max_entries must be <= %lld", (long long)csl::topk_max_entries());
  if (ld < max_entries) return fail(CSL_ERR_INVALID, "topk_select: ld < max_entries");
  if ((int64_t)B * T > 0x7fffffff) return fail(CSL_ERR_UNSUPPORTED, "topk_select: too many rows");
  if (B == 0 || T == 0) return CSL_OK;
  const size_t need = csl_topk_workspace_bytes(B, T, max_entries, k);
  if (need > 0) {
    if ((int64_t)B * T > kMaxGridY) return fail(CSL_ERR_UNSUPPORTED, "topk_select: long rows need B*T <= %d", kMaxGridY);
    if (!ws || ws_bytes < need)
      return fail(CSL_ERR_WORKSPACE, "topk_select: workspace of %zu bytes required, got %zu", need, ws ? ws_bytes : 0);
    if (!aligned(ws, 16)) return fail(CSL_ERR_INVALID, "topk_select: workspace must be 16-byte aligned");
  }
  return CSL_OK;
}

}  // namespace

extern "C" {

int csl_compress_kv(const void* kv, const void* z, const int64_t* kv_off, const int64_t* ent_off,
                    const int64_t* first_entry, int B, int D, int m, int64_t max_new_entries, void* out,
                    int out_dtype, const csl_paged_cache* paged, void* stream) {
  int st = check_compress(kv, z, kv_off, ent_off, B, D, m, max_new_entries, out, out_dtype);
  if (st != CSL_OK) return st;
  csl::PagedView pv;
  if (paged) {
    st = check_paged("compress_kv", paged, B, pv);
    if (st != CSL_OK) return st;
    st = check_ring("compress_kv", paged, 0, 0, m, max_new_entries, false);
    if (st != CSL_OK) return st;
  }
  if (B == 0 || max_new_entries == 0) return ok();
  return hip_status(csl::launch_compress(kv, z, kv_off, ent_off, first_entry, B, D, m, max_new_entries, out,
                                         out_dtype == CSL_DTYPE_BF16, as_stream(stream), paged ? &pv : nullptr),
                    "compress_kv launch");
}

int csl_compress_kv_overlap(const void* kv_a, const void* z_a, const void* kv_b, const void* z_b,
                            const int64_t* kv_off, const int64_t* ent_off, const int64_t* first_entry, int B, int D,
                            int m, int64_t max_new_entries, void* out, int out_dtype, const csl_paged_cache* paged,
                            void* stream) {
  int st = check_compress(kv_a, z_a, kv_off, ent_off, B, D, m, max_new_entries, out, out_dtype, "compress_kv_overlap");
  if (st != CSL_OK) return st;
  st = check_series_b(kv_b, z_a, z_b, "compress_kv_overlap");
  if (st != CSL_OK) return st;
  csl::PagedView pv;
  if (paged) {
    st = check_paged("compress_kv_overlap", paged, B, pv);
    if (st != CSL_OK) return st;
    st = check_ring("compress_kv_overlap", paged, 0, 0, m, max_new_entries, true);
    if (st != CSL_OK) return st;
  }
  if (B == 0 || max_new_entries == 0) return ok();
  return hip_status(csl::launch_compress_overlap(kv_a, z_a, kv_b, z_b, kv_off, ent_off, first_entry, B, D, m,
                                                 max_new_entries, out, out_dtype == CSL_DTYPE_BF16,
                                                 as_stream(stream), paged ? &pv : nullptr),
                    "compress_kv_overlap launch");
}

int csl_indexer_scores(const void* q_idx, const float* w, const void* k_idx, int k_dtype, const void* k_scale,
                       const int64_t* scale_off, int scale_group, const int64_t* ent_off, const int64_t* q_pos, int m,
                       int B, int T, int HI, int CI, int64_t max_entries, float* scores, int64_t ld, void* topk_ws,
                       size_t topk_ws_bytes, int topk_k, const csl_paged_cache* paged, void* stream) {
  int st = check_indexer(q_idx, w, k_idx, k_dtype, k_scale, scale_off, scale_group, ent_off, q_pos, m, B, T, HI,
                         CI, max_entries, scores, ld, topk_ws, topk_ws_bytes, topk_k, "indexer_scores",
                         paged != nullptr);
  if (st != CSL_OK) return st;
  csl::PagedView pv;
  if (paged) {
    st = check_paged("indexer_scores", paged, B, pv);
    if (st != CSL_OK) return st;
    st = check_paged_scales("indexer_scores", k_dtype, scale_group, pv);
    if (st != CSL_OK) return st;
  }
  if (B == 0 || T == 0 || max_entries == 0) return ok();
  return hip_status(csl::launch_indexer(q_idx, w, k_idx, key_type(k_dtype), k_scale, scale_off, scale_group,
                                        ent_off, q_pos, m, B, T, HI, max_entries, scores, ld, topk_ws, topk_k,
                                        as_stream(stream), nullptr, paged ? &pv : nullptr),
                    "indexer_scores launch");
}

int csl_indexer_topk_max_k(int HI) {
  return (HI == 1 || HI == 2 || HI == 4 || HI == 8 || HI == 16) ? csl::indexer_topk_max_k(HI) : 0;
}

int csl_indexer_topk(const void* q_idx, const float* w, const void* k_idx, int k_dtype, const void* k_scale,
                     const int64_t* scale_off, int scale_group, const int64_t* ent_off, const int64_t* q_pos, int m,
                     int B, int T, int HI, int CI, int64_t max_entries, int k, int32_t* idx,
                     const csl_paged_cache* paged, void* stream) {
  if (!idx) return fail(CSL_ERR_INVALID, "indexer_topk: null pointer argument");
  void* no_ws = nullptr;
  // the indexer's checks, with idx standing in for the score buffer it does not need
  int st = check_indexer(q_idx, w, k_idx, k_dtype, k_scale, scale_off, scale_group, ent_off, q_pos, m, B, T, HI, CI,
                         max_entries, reinterpret_cast<const float*>(idx), max_entries, no_ws, 0, 0,
                         "indexer_topk", paged != nullptr);
  if (st != CSL_OK) return st;
  const int kmax = csl_indexer_topk_max_k(HI);
  if (k < 1 || k > kmax) return fail(CSL_ERR_UNSUPPORTED, "indexer_topk: k must be in [1, %d], got %d", kmax, k);
  if (!aligned(idx, 4)) return fail(CSL_ERR_INVALID, "indexer_topk: idx must be 4-byte aligned");
  if (B > kMaxGridY) return fail(CSL_ERR_UNSUPPORTED, "indexer_topk: B must be <= %d", kMaxGridY);
  if (max_entries > 0x7fffffff) return fail(CSL_ERR_UNSUPPORTED, "indexer_topk: max_entries must be < 2^31");
  csl::PagedView pv;
  if (paged) {
    st = check_paged("indexer_topk", paged, B, pv);
    if (st != CSL_OK) return st;
    st = check_paged_scales("indexer_topk", k_dtype, scale_group, pv);
    if (st != CSL_OK) return st;
  }
  if (B == 0 || T == 0) return ok();
  return hip_status(csl::launch_indexer_topk(q_idx, w, k_idx, key_type(k_dtype), k_scale, scale_off, scale_group,
                                             ent_off, q_pos, m, B, T, HI, max_entries, k, idx, as_stream(stream),
                                             paged ? &pv : nullptr),
                    "indexer_topk launch");
}

size_t csl_topk_workspace_bytes(int B, int T, int64_t max_entries, int k) {
  if (B <= 0 || T <= 0 || max_entries <= 0 || k <= 0) return 0;
  return csl::topk_workspace_bytes(B, T, max_entries, k);
}

int csl_topk_select(const float* scores, int64_t ld, const int64_t* ent_off, const int64_t* q_pos, int m, int B,
                    int T, int k, int64_t max_entries, int32_t* idx, void* ws, size_t ws_bytes, int prepared,
                    void* stream) {
  const int st = check_topk(scores, ld, ent_off, q_pos, m, B, T, k, max_entries, idx, ws, ws_bytes);
  if (st != CSL_OK) return st;
  if (B == 0 || T == 0) return ok();
  const bool use_lists = prepared != 0 && csl::indexer_prepares_topk(ws, T, max_entries);
  return hip_status(csl::launch_topk(scores, ld, ent_off, q_pos, m, B, T, k, max_entries, idx, ws, use_lists,
                                     as_stream(stream)),
                    "topk_select launch");
}

size_t csl_attn_workspace_bytes(int B, int T, int H, int D, int64_t max_keys) {
  if (B <= 0 || T <= 0 || H <= 0 || D != 128 || max_keys < 0) return 0;
  return csl::attn_workspace_bytes(B, T, H, max_keys);
}

static int check_attn(const char* who, const void* q, const void* ckv, const void* kv, const int64_t* kv_off,
                      const int64_t* ent_off, const int64_t* q_pos, int n_win, int B, int T, int H, int D, float scale,
                      const float* out, void* ws, size_t ws_bytes, int64_t max_keys) {
  if (B < 0 || T < 0 || n_win < 0) return fail(CSL_ERR_INVALID, "%s: negative size", who);
  if (!q || !ckv || !kv || !kv_off || !ent_off || !q_pos || !out)
    return fail(CSL_ERR_INVALID, "%s: null pointer argument", who);
  if (D != 128) return fail(CSL_ERR_UNSUPPORTED, "%s: D must be 128, got %d", who, D);
  if (H < 16 || H > 128 || H % 16 != 0)
    return fail(CSL_ERR_UNSUPPORTED, "%s: H must be a multiple of 16 in [16, 128], got %d", who, H);
  if (!(std::isfinite(scale) && scale > 0.f)) return fail(CSL_ERR_INVALID, "%s: scale must be finite and > 0", who);
  if ((int64_t)B * T > kMaxGridY) return fail(CSL_ERR_UNSUPPORTED, "%s: B*T must be <= %d", who, kMaxGridY);
  if (!aligned(q, 16) || !aligned(ckv, 16) || !aligned(kv, 16) || !aligned(out, 16))
    return fail(CSL_ERR_INVALID, "%s: q, ckv, kv and out must be 16-byte aligned", who);
  if (B == 0 || T == 0) return -1;
  const size_t need = csl_attn_workspace_bytes(B, T, H, D, max_keys);
  if (need > 0 && (!ws || ws_bytes < need))
    return fail(CSL_ERR_WORKSPACE, "%s: workspace of %zu bytes required, got %zu", who, need, ws ? ws_bytes : 0);
  if (need > 0 && !aligned(ws, 16)) return fail(CSL_ERR_INVALID, "%s: workspace must be 16-byte aligned", who);
  return CSL_OK;
}

// attention extras: a valid RoPE width and base, an aligned sink; fills the launcher's form
static int check_extras(const char* who, const float* sink, int rope_dims, float rope_base, csl::AttnExtras& ex) {
  if (rope_dims < 0) return fail(CSL_ERR_INVALID, "%s: rope_dims must be >= 0", who);
  if (rope_dims != 0 && rope_dims != 64)
    return fail(CSL_ERR_UNSUPPORTED, "%s: rope_dims must be 0 or 64, got %d", who, rope_dims);
  if (rope_dims > 0 && !(std::isfinite(rope_base) && rope_base > 1.f))
    return fail(CSL_ERR_INVALID, "%s: rope_base must be finite and > 1", who);
  if (sink && !aligned(sink, 4)) return fail(CSL_ERR_INVALID, "%s: sink must be 4-byte aligned", who);
  ex.sink = sink;
  ex.rope_dims = rope_dims;
  ex.rope_theta1 = rope_dims > 0 ? std::pow((double)rope_base, -2.0 / rope_dims) : 1.0;
  return CSL_OK;
}

int csl_sparse_attn_decode(const void* q, const void* ckv, const int32_t* idx, int k, const void* kv,
                           const int64_t* kv_off, const int64_t* ent_off, const int64_t* q_pos, int n_win, int B, int T,
                           int H, int D, float scale, float* out, float* lse, void* ws, size_t ws_bytes,
                           const csl_attn_extras* extras, const csl_paged_cache* paged, void* stream) {
  csl::AttnExtras ex;
  if (extras) {
    const int se = check_extras("sparse_attn_decode", extras->sink, extras->rope_dims, extras->rope_base, ex);
    if (se != CSL_OK) return se;
  }
  if (k < 0) return fail(CSL_ERR_INVALID, "sparse_attn_decode: k must be >= 0");
  if (k > 0 && !idx) return fail(CSL_ERR_INVALID, "sparse_attn_decode: idx is NULL");
  const int64_t max_keys = (int64_t)k + n_win;
  int st = check_attn("sparse_attn_decode", q, ckv, kv, kv_off, ent_off, q_pos, n_win, B, T, H, D, scale, out, ws,
                      ws_bytes, max_keys);
  if (st == -1) return ok();
  if (st != CSL_OK) return st;
  csl::PagedView pv;
  if (paged) {
    st = check_paged("sparse_attn_decode", paged, B, pv);
    if (st != CSL_OK) return st;
    st = check_ring("sparse_attn_decode", paged, n_win, T, 1, 0, false);
    if (st != CSL_OK) return st;
  }
  return hip_status(csl::launch_attention(true, q, ckv, idx, k, kv, kv_off, ent_off, q_pos, 1, n_win, B, T, H, scale,
                                          (int64_t)1 << 62, max_keys, out, lse, ws, ex, as_stream(stream),
                                          paged ? &pv : nullptr),
                    "sparse_attn_decode launch");
}

int csl_hca_attn_decode(const void* q, const void* ckv, const void* kv, const int64_t* kv_off, const int64_t* ent_off,
                        const int64_t* q_pos, int m, int n_win, int B, int T, int H, int D, float scale,
                        int64_t max_entries, float* out, float* lse, void* ws, size_t ws_bytes,
                        const csl_attn_extras* extras, const csl_paged_cache* paged, void* stream) {
  csl::AttnExtras ex;
  if (extras) {
    const int se = check_extras("hca_attn_decode", extras->sink, extras->rope_dims, extras->rope_base, ex);
    if (se != CSL_OK) return se;
  }
  if (m < 1) return fail(CSL_ERR_INVALID, "hca_attn_decode: m must be >= 1");
  if (max_entries < 0) return fail(CSL_ERR_INVALID, "hca_attn_decode: max_entries must be >= 0");
  const int64_t max_keys = max_entries + n_win;
  int st = check_attn("hca_attn_decode", q, ckv, kv, kv_off, ent_off, q_pos, n_win, B, T, H, D, scale, out, ws,
                      ws_bytes, max_keys);
  if (st == -1) return ok();
  if (st != CSL_OK) return st;
  csl::PagedView pv;
  if (paged) {
    st = check_paged("hca_attn_decode", paged, B, pv);
    if (st != CSL_OK) return st;
    st = check_ring("hca_attn_decode", paged, n_win, T, m, 0, false);
    if (st != CSL_OK) return st;
  }
  return hip_status(csl::launch_attention(false, q, ckv, nullptr, 0, kv, kv_off, ent_off, q_pos, m, n_win, B, T, H,
                                          scale, max_entries, max_keys, out, lse, ws, ex, as_stream(stream),
                                          paged ? &pv : nullptr),
                    "hca_attn_decode launch");
}

int csl_hca_decode_step(const csl_hca_step* s, void* stream) {
  if (!s) return fail(CSL_ERR_INVALID, "hca_decode_step: null step");
  int st = check_compress(s->kv, s->z, s->kv_off, s->ent_off, s->B, 128, s->m, s->max_new_entries, s->ckv,
                          CSL_DTYPE_BF16, "hca_decode_step");
  if (st != CSL_OK) return st;
  csl::AttnExtras ex;
  st = check_extras("hca_decode_step", s->sink, s->rope_dims, s->rope_base, ex);
  if (st != CSL_OK) return st;
  if (s->max_entries < 0) return fail(CSL_ERR_INVALID, "hca_decode_step: max_entries must be >= 0");
  const int64_t max_keys = s->max_entries + s->n_win;
  st = check_attn("hca_decode_step", s->q, s->ckv, s->kv, s->kv_off, s->ent_off, s->q_pos, s->n_win, s->B, s->T, s->H,
                  128, s->scale, s->out, s->attn_ws, s->attn_ws_bytes, max_keys);
  if (st != CSL_OK && st != -1) return st;
  csl::PagedView pv;
  const csl::PagedView* pvp = nullptr;
  if (s->paged) {
    st = check_paged("hca_decode_step", s->paged, s->B, pv);
    if (st != CSL_OK) return st;
    st = check_ring("hca_decode_step", s->paged, s->n_win, s->T, s->m, s->max_new_entries, false);
    if (st != CSL_OK) return st;
    pvp = &pv;
  }
  const hipStream_t hs = as_stream(stream);
  const bool compress = s->B > 0 && s->max_new_entries > 0;
  const bool attend = s->B > 0 && s->T > 0;
  if (!attend) {  // no query rows: the compression alone
    if (!compress) return ok();
    return hip_status(csl::launch_compress(s->kv, s->z, s->kv_off, s->ent_off, s->first_entry, s->B, 128, s->m,
                                           s->max_new_entries, s->ckv, true, hs, pvp),
                      "hca_decode_step launch");
  }
  if (compress && csl::attention_carries_job(s->B, s->T, s->H, max_keys, s->max_new_entries)) {
    // the compression rides in spare workgroups of the attention launch
    csl::HcaJob job;
    job.kv = static_cast<const uint16_t*>(s->kv);
    job.z = static_cast<const uint16_t*>(s->z);
    job.first_entry = s->first_entry;
    job.max_new = s->max_new_entries;
    job.ckv = static_cast<uint16_t*>(s->ckv);
    return hip_status(csl::launch_attention(false, s->q, s->ckv, nullptr, 0, s->kv, s->kv_off, s->ent_off, s->q_pos,
                                            s->m, s->n_win, s->B, s->T, s->H, s->scale, s->max_entries, max_keys,
                                            s->out, s->lse, s->attn_ws, ex, hs, pvp, &job),
                      "hca_decode_step launch");
  }
  hipError_t e = hipSuccess;
  if (compress)
    e = csl::launch_compress(s->kv, s->z, s->kv_off, s->ent_off, s->first_entry, s->B, 128, s->m, s->max_new_entries,
                             s->ckv, true, hs, pvp);
  if (e != hipSuccess) return hip_status(e, "hca_decode_step launch");
  return hip_status(csl::launch_attention(false, s->q, s->ckv, nullptr, 0, s->kv, s->kv_off, s->ent_off, s->q_pos,
                                          s->m, s->n_win, s->B, s->T, s->H, s->scale, s->max_entries, max_keys, s->out,
                                          s->lse, s->attn_ws, ex, hs, pvp),
                    "hca_decode_step launch");
}

int csl_csa_decode_step(const csl_csa_step* s, void* stream) {
  if (!s) return fail(CSL_ERR_INVALID, "csa_decode_step: null argument");
  // every part is validated before anything is enqueued
  int st = check_compress(s->kv, s->z, s->kv_off, s->ent_off, s->B, s->D, s->m, s->max_new_entries, s->ckv,
                          CSL_DTYPE_BF16, "csa_decode_step");
  if (st != CSL_OK) return st;
  const bool overlap = s->kv_b != nullptr || s->z_b != nullptr;
  if (overlap) {
    st = check_series_b(s->kv_b, s->z, s->z_b, "csa_decode_step");
    if (st != CSL_OK) return st;
  }
  csl::AttnExtras ex;
  st = check_extras("csa_decode_step", s->sink, s->rope_dims, s->rope_base, ex);
  if (st != CSL_OK) return st;
  csl::PagedView pv;
  const csl::PagedView* pvp = nullptr;
  if (s->paged) {
    st = check_paged("csa_decode_step", s->paged, s->B, pv);
    if (st != CSL_OK) return st;
    st = check_paged_scales("csa_decode_step", s->k_dtype, s->scale_group, pv);
    if (st != CSL_OK) return st;
    st = check_ring("csa_decode_step", s->paged, s->n_win, s->T, s->m, s->max_new_entries, overlap);
    if (st != CSL_OK) return st;
    pvp = &pv;
  }
  // no score buffer: the indexer fused with top-k (csl_indexer_topk) makes the selection
  const bool scoreless = s->scores == nullptr;
  void* topk_ws = scoreless ? nullptr : s->topk_ws;
  if (scoreless) {
    if (!s->idx) return fail(CSL_ERR_INVALID, "csa_decode_step: null pointer argument");
    void* no_ws = nullptr;
    st = check_indexer(s->q_idx, s->w, s->k_idx, s->k_dtype, s->k_scale, s->scale_off, s->scale_group, s->ent_off,
                       s->q_pos, s->m, s->B, s->T, s->HI, s->CI, s->max_entries, reinterpret_cast<const float*>(s->idx),
                       s->max_entries, no_ws, 0, 0, "csa_decode_step", s->paged != nullptr);
    if (st != CSL_OK) return st;
    const int kmax = csl_indexer_topk_max_k(s->HI);
    if (s->k < 1 || s->k > kmax)
      return fail(CSL_ERR_UNSUPPORTED, "csa_decode_step: without scores k must be in [1, %d], got %d", kmax, s->k);
    if (s->max_entries > 0x7fffffff)
      return fail(CSL_ERR_UNSUPPORTED, "csa_decode_step: max_entries must be < 2^31");
  } else {
    st = check_indexer(s->q_idx, s->w, s->k_idx, s->k_dtype, s->k_scale, s->scale_off, s->scale_group, s->ent_off,
                       s->q_pos, s->m, s->B, s->T, s->HI, s->CI, s->max_entries, s->scores, s->ld, topk_ws,
                       s->topk_ws_bytes, s->k, "csa_decode_step", s->paged != nullptr);
    if (st != CSL_OK) return st;
    st = check_topk(s->scores, s->ld, s->ent_off, s->q_pos, s->m, s->B, s->T, s->k, s->max_entries, s->idx,
                    s->topk_ws, s->topk_ws_bytes);
    if (st != CSL_OK) return st;
  }
  const int64_t max_keys = (int64_t)s->k + s->n_win;
  st = check_attn("csa_decode_step", s->q, s->ckv, s->kv, s->kv_off, s->ent_off, s->q_pos, s->n_win, s->B, s->T, s->H,
                  s->D, s->scale, s->out, s->attn_ws, s->attn_ws_bytes, max_keys);
  if (st == -1) return ok();  // B or T is 0
  if (st != CSL_OK) return st;

  const hipStream_t hs = as_stream(stream);
  const int kt = key_type(s->k_dtype);
  const bool compress = s->max_new_entries > 0;
  const bool index = s->max_entries > 0;
  // rows whose whole key list one attention workgroup holds: that workgroup makes the row's
  // top-k selection itself (the same ids, also written to idx) instead of a top-k launch
  const bool select_in_attn = !scoreless && !pvp && index &&
                              csl::attention_selects_topk(s->B, s->T, s->H, s->k, max_keys, s->max_entries);
  const csl::TopkIn tk{s->scores, s->ld, s->m, s->max_entries, s->idx};
  // scores on demand: rows selected from candidate lists keep no scores; the finishing step
  // recomputes a row's scores where its lists cannot prove the selection
  const bool on_demand = s->scores_on_demand != 0 && !scoreless && !select_in_attn && !pvp && index &&
                         csl::indexer_prepares_topk(topk_ws, s->T, s->max_entries) &&
                         csl::topk_finish_can_rescore(s->max_entries, s->k);
  const csl::RescoreIn rescore{s->q_idx, s->w, s->k_idx, kt, s->k_scale, s->scale_off, s->scale_group, s->HI};
  hipError_t e = hipSuccess;
  if (scoreless) {
    if (compress && overlap)
      e = csl::launch_compress_overlap(s->kv, s->z, s->kv_b, s->z_b, s->kv_off, s->ent_off, s->first_entry, s->B,
                                       s->D, s->m, s->max_new_entries, s->ckv, true, hs, pvp);
    else if (compress)
      e = csl::launch_compress(s->kv, s->z, s->kv_off, s->ent_off, s->first_entry, s->B, s->D, s->m,
                               s->max_new_entries, s->ckv, true, hs, pvp);
    if (e == hipSuccess)
      e = csl::launch_indexer_topk(s->q_idx, s->w, s->k_idx, kt, s->k_scale, s->scale_off, s->scale_group, s->ent_off,
                                   s->q_pos, s->m, s->B, s->T, s->HI, s->max_entries, s->k, s->idx, hs, pvp);
  } else if (compress && index && csl::indexer_carries_compress(topk_ws, s->B, s->T, s->max_entries, s->D, s->m)) {
    // the newest-chunk compression rides in spare workgroups of the indexer launch
    const csl::CompressJob job{s->kv, s->z, s->kv_off, s->first_entry, s->max_new_entries, s->ckv, s->m,
                               s->kv_b, s->z_b};
    e = csl::launch_indexer(s->q_idx, s->w, s->k_idx, kt, s->k_scale, s->scale_off, s->scale_group, s->ent_off,
                            s->q_pos, s->m, s->B, s->T, s->HI, s->max_entries, s->scores, s->ld, topk_ws, s->k, hs, &job,
                            pvp, on_demand);
  } else {
    if (compress && overlap)
      e = csl::launch_compress_overlap(s->kv, s->z, s->kv_b, s->z_b, s->kv_off, s->ent_off, s->first_entry, s->B,
                                       s->D, s->m, s->max_new_entries, s->ckv, true, hs, pvp);
    else if (compress)
      e = csl::launch_compress(s->kv, s->z, s->kv_off, s->ent_off, s->first_entry, s->B, s->D, s->m,
                               s->max_new_entries, s->ckv, true, hs, pvp);
    if (e == hipSuccess && index)
      e = csl::launch_indexer(s->q_idx, s->w, s->k_idx, kt, s->k_scale, s->scale_off, s->scale_group, s->ent_off,
                              s->q_pos, s->m, s->B, s->T, s->HI, s->max_entries, s->scores, s->ld, topk_ws, s->k, hs,
                              nullptr, pvp, on_demand);
  }
  if (e != hipSuccess) return hip_status(e, "csa_decode_step launch");
  if (!scoreless && !select_in_attn)
    e = csl::launch_topk(s->scores, s->ld, s->ent_off, s->q_pos, s->m, s->B, s->T, s->k, s->max_entries, s->idx,
                         s->topk_ws, csl::indexer_prepares_topk(topk_ws, s->T, s->max_entries), hs,
                         on_demand ? &rescore : nullptr);
  if (e != hipSuccess) return hip_status(e, "csa_decode_step launch");
  return hip_status(csl::launch_attention(true, s->q, s->ckv, s->idx, s->k, s->kv, s->kv_off, s->ent_off, s->q_pos, 1,
                                          s->n_win, s->B, s->T, s->H, s->scale, (int64_t)1 << 62, max_keys, s->out,
                                          s->lse, s->attn_ws, ex, hs, pvp, nullptr, select_in_attn ? &tk : nullptr),
                    "csa_decode_step launch");
}

}  // extern "C"

// ---------------------------------------------------------------------------------------------
// The step without allocation: its two workspaces (the top-k candidate lists and the attention
// split partials) come from one file-scope device array instead of the caller's buffers. Every
// GPU holds its own copy of the array; its address on each device is looked up once (with that
// device current) and kept. Calls on one device share the array, so calls that overlap in time
// on one device race.
namespace {

static __device__ __align__(256) unsigned char scratch[CSL_STATIC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// the scratch array's device address on the current device (looked up on first use)
int current_scratch(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "csa_decode_step_static: hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(CSL_ERR_UNSUPPORTED, "csa_decode_step_static: device %d beyond the %d supported", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e, "csa_decode_step_static: hipGetSymbolAddress(scratch)");
    if (!p) return fail(CSL_ERR_HIP, "csa_decode_step_static: no device address for the scratch array");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return CSL_OK;
}

}  // namespace

extern "C" int csl_csa_decode_step_static(const csl_csa_step* s, void* stream) {
  if (!s) return fail(CSL_ERR_INVALID, "csa_decode_step_static: null argument");
  // the workspaces this step needs, as csl_csa_decode_step sizes them: candidate lists only
  // with a score buffer, split partials for the attention
  const bool scored = s->scores != nullptr;
  const size_t need_topk =
      (scored && s->B > 0 && s->T > 0) ? csl_topk_workspace_bytes(s->B, s->T, s->max_entries, s->k) : 0;
  const size_t need_attn =
      (s->B > 0 && s->T > 0 && s->k >= 0 && s->n_win >= 0)
          ? csl_attn_workspace_bytes(s->B, s->T, s->H, s->D, (int64_t)s->k + s->n_win)
          : 0;
  const size_t off_attn = (need_topk + 255) & ~(size_t)255;
  if (off_attn + need_attn > (size_t)CSL_STATIC_SCRATCH_BYTES)
    return fail(CSL_ERR_WORKSPACE,
                "csa_decode_step_static: the step needs %zu bytes of workspace, beyond the %zu-byte static scratch",
                off_attn + need_attn, (size_t)CSL_STATIC_SCRATCH_BYTES);
  void* base = nullptr;
  const int st = current_scratch(&base);
  if (st != CSL_OK) return st;
  csl_csa_step t = *s;
  t.topk_ws = need_topk ? base : nullptr;
  t.topk_ws_bytes = need_topk;
  t.attn_ws = need_attn ? static_cast<unsigned char*>(base) + off_attn : nullptr;
  t.attn_ws_bytes = need_attn;
  return csl_csa_decode_step(&t, stream);
}
