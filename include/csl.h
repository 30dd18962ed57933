/*
 * csl.h -- C ABI of the MI355X (gfx950) hybrid compressed-attention library.
 *
 * One attention layer of the method described on these pages:
 *   [P1] "1M Context != Lossless Long Memory: What DeepSeek-V4 Reveals About the
 *        Engineering Tradeoffs" (wiki.gxlh.xyz/doc/1210)
 *   [P2] "DeepSeek-V4: Million-Token Context via Hybrid Compressed Attention"
 *        (zhongzhoutan-coder.github.io, DeepSeek-V4 training notes)
 *   [P3] "DeepSeek-V4 的暗线之一：分层记忆比输入框更关键" (blog.xieydd.top)
 *   [P5] "DeepSeek-V4 technical report" breakdown (deconstructedpapers.com)
 *
 * CSA (compressed sparse attention): compress_kv (m = 4) -> indexer_scores -> topk_select
 *   -> sparse_attn_decode.  HCA (heavily compressed attention): compress_kv (m = 128) ->
 *   hca_attn_decode.
 *
 * Conventions shared by every call
 *   - Every tensor argument is a caller-owned DEVICE pointer to contiguous row-major data.
 *     bf16 tensors are passed as raw 16-bit words. The library never allocates, frees,
 *     synchronises, or keeps a pointer after the call returns; work is enqueued on
 *     `stream` (a hipStream_t; NULL is the default stream). Buffers must stay alive until
 *     the stream has passed the work.
 *   - Ragged batches are packed: sequence b owns raw rows [kv_off[b], kv_off[b+1]) of the
 *     raw K=V array and compressed entries [ent_off[b], ent_off[b+1]) of the compressed
 *     array. kv_off / ent_off are DEVICE int64 arrays of B+1 non-decreasing values.
 *     Query row t of sequence b sits at absolute position p = q_pos[b] + t (q_pos is a
 *     DEVICE int64 array of B values).
 *   - Visibility: a query at position p sees compressed entries s < floor(p / m) of its
 *     sequence (never the block it falls in, [P1] section 6.1) and the raw window of the
 *     n_win newest rows j with j <= p and j < N_b ([P1] section 6; [P2] "KV Cache
 *     Management"). Decode uses p = N_b: all floor(N_b/m) entries plus rows
 *     [N_b - n_win, N_b).
 *   - Host scalars are validated before anything is enqueued; a bad value returns
 *     CSL_ERR_INVALID or CSL_ERR_UNSUPPORTED and enqueues nothing. Device-resident data
 *     (offsets, positions, selected ids, scales) are preconditions and are not checked,
 *     except that selected ids outside [0, E_b) are treated as padding.
 *   - Every call returns a csl_status. csl_last_error() returns a thread-local message
 *     describing the last failure on the calling thread.
 *   - The library holds no global state (except the per-device scratch array of
 *     csl_csa_decode_step_static); calls on different streams may run concurrently as long
 *     as they do not share output or workspace buffers.
 */
#ifndef CSL_H
#define CSL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  CSL_OK = 0,
  CSL_ERR_INVALID = 1,     /* null pointer, negative size, inconsistent arguments       */
  CSL_ERR_UNSUPPORTED = 2, /* a shape or dtype outside what the kernels implement        */
  CSL_ERR_WORKSPACE = 3,   /* workspace pointer missing or smaller than required         */
  CSL_ERR_HIP = 4          /* the HIP runtime reported an error at launch                */
} csl_status;

typedef enum {
  CSL_DTYPE_BF16 = 0,
  CSL_DTYPE_F32 = 1,
  CSL_DTYPE_FP8_E4M3 = 2, /* OCP E4M3FN: bias 7, no infinities, max 448, S.1111.111 = NaN */
  CSL_DTYPE_MXFP4 = 3     /* OCP MXFP4: E2M1 codes, two per byte, one E8M0 scale per 32 values */
} csl_dtype;

/*
 * Paged heterogeneous cache ([P2] "KV Cache Management"): the compressed entries live in a
 * classical cache of fixed-size blocks and the raw rows in a per-sequence state cache.
 * Every call below takes an optional `const csl_paged_cache* paged`; NULL keeps the packed
 * layout described above. With it:
 *   - compressed entry e of sequence b (ckv rows, CSA indexer keys and their MXFP4 scales)
 *     sits at pool row  block_table[b * max_blocks + e / block_entries] * block_entries
 *     + e % block_entries; the caller allocates the blocks (block_entries = lcm(m, m') / m
 *     covers lcm(m, m') raw tokens: 32 for CSA's m = 4 beside HCA's m' = 128, 1 for HCA);
 *   - fp8 indexer keys keep their group scales with the blocks: scale_group must be a power
 *     of two, scale_off is ignored (may be NULL), and the scale of the key at pool row r is
 *     k_scale[r >> min(log2(scale_group), log2(block_entries))] -- one scale per group of a
 *     block, or, when a group spans several blocks, one per block (the group's scale
 *     repeated in each of its blocks); k_scale holds pool_entries >> that shift scales;
 *   - with ring_rows > 0, raw row r of sequence b (kv, z, and for overlapped compression
 *     kv_b, z_b) sits at ring row b * ring_rows + r % ring_rows: the state cache keeps the
 *     newest ring_rows rows of each sequence, which must hold every raw row a call reads.
 *     The host checks ring_rows >= max(n_win + T - 1, (max_new_entries + 1) * m - 1), with
 *     (max_new_entries + 2) * m - 1 for overlapped compression (each term only where the
 *     call has a window or compresses), and returns CSL_ERR_INVALID otherwise. That covers
 *     the windows of T query rows at the end of the context and the newest entries'
 *     chunks; queries elsewhere in the context, or compressing from entry 0 (first_entry
 *     NULL), need a ring that holds those rows too (a precondition);
 *   - with ring_rows = 0 the raw rows stay packed as kv_off says (only the compressed
 *     entries are paged);
 *   - kv_off and ent_off still give each sequence's raw-row and entry counts (as prefix
 *     sums); they no longer place rows.
 * block_table entries of the blocks a sequence uses, and the ring's rows, are preconditions.
 */
typedef struct csl_paged_cache {
  const int32_t* block_table; /* device int32 [B, max_blocks] */
  int max_blocks;             /* >= 1 */
  int block_entries;          /* entries per block, a power of two */
  int64_t pool_entries;       /* rows of the entry pool, < 2^31 */
  int ring_rows;              /* 0 (raw rows packed as kv_off says) or a power of two */
} csl_paged_cache;

/* Message for the last failed call on this thread ("" if none). Never NULL. */
const char* csl_last_error(void);

/* Library version as MAJOR*10000 + MINOR*100 + PATCH (0.5.0: csl_csa_step gains
 * scores_on_demand at its end; 0.4.0: overlapped compression, attention sink and partial
 * RoPE, MXFP4 indexer keys, paged cache). */
int csl_version(void);

/*
 * compress_kv -- softmax-weighted chunk pooling ([P3] section 3, the compressed KV entry;
 * [P2] "Deep Dive", CSA step 2 and HCA "How it works"; [P1] section 4.1).
 *
 *   out[ent_off[b] + i, d] = sum_{r<m} w_r[d] * kv[kv_off[b] + m*i + r, d],
 *   w[:, d] = softmax over the m rows of z[kv_off[b] + m*i + r, d]   (uniform 1/m if z NULL)
 *
 * for every sequence b and entry i with first_entry[b] <= i < E_b, E_b = floor(N_b / m),
 * N_b = kv_off[b+1] - kv_off[b], and at most max_new_entries entries per sequence
 * (i < first_entry[b] + max_new_entries). first_entry NULL means 0 (bulk compression of a
 * whole prefix); first_entry[b] = E_b - 1 recompresses only the newest complete chunk, as
 * a decode step does. The trailing N_b mod m rows are not pooled.
 *
 *   kv, z   bf16 [rows, D] (z nullable)        D in {64, 128, 256, 512}; m in [1, 65536]
 *   out     [*, D] of out_dtype (CSL_DTYPE_F32 or CSL_DTYPE_BF16, bf16 rounded to nearest
 *           even); out rows other than the ones listed above are not written.
 * Arithmetic: fp32, exponentials in base 2 with a log2(e) prescale.
 */
int csl_compress_kv(const void* kv, const void* z, const int64_t* kv_off, const int64_t* ent_off,
                    const int64_t* first_entry, int B, int D, int m, int64_t max_new_entries,
                    void* out, int out_dtype, const csl_paged_cache* paged, void* stream);

/*
 * compress_kv_overlap -- CSA's overlapped (dual-series) compression ([P2] "Deep Dive", CSA
 * dual-series KV compression; [P1] section 4.3, overlap compression). Two series a and b of
 * raw rows, each with its own logits, share the packed layout of compress_kv. Entry i pools
 * the m series-a rows of its own block and the m series-b rows of the block before it under
 * one softmax per dimension:
 *
 *   out[ent_off[b] + i, d] = sum_{r<m} wa_r[d] * kv_a[R + m*i + r, d]
 *                          + sum_{r<m} wb_r[d] * kv_b[R + m*(i-1) + r, d]       (R = kv_off[b])
 *   (wa, wb)[:, d] = softmax over the 2m logits z_a[R + m*i + r, d], z_b[R + m*(i-1) + r, d]
 *
 * Entry 0 has no block before it: its softmax runs over its m series-a rows alone. With
 * z_a and z_b both NULL the weights are uniform over the rows pooled. Entries, first_entry,
 * max_new_entries, D, m, out and out_dtype are as for compress_kv; series b rows
 * [m*(E_b-1), N_b) are never read.
 *
 *   kv_a, kv_b   bf16 [rows, D], the same rows and offsets; 16-byte aligned
 *   z_a, z_b     bf16 [rows, D], both given or both NULL (else CSL_ERR_INVALID)
 * It reads twice the bytes of compress_kv for the same entries.
 */
int csl_compress_kv_overlap(const void* kv_a, const void* z_a, const void* kv_b, const void* z_b,
                            const int64_t* kv_off, const int64_t* ent_off, const int64_t* first_entry, int B, int D,
                            int m, int64_t max_new_entries, void* out, int out_dtype,
                            const csl_paged_cache* paged, void* stream);

/*
 * indexer_scores -- Lightning-indexer scores ([P5], the indexer score formula;
 * [P2] "Deep Dive", CSA Lightning Indexer; [P1] section 4.2):
 *
 *   scores[b, t, s] = sum_{j<HI} w[b, t, j] * max(0, sum_{c<CI} q_idx[b, t, j, c] * key(s, c))
 *
 * for s < n(b, t) = min(floor(p / m), E_b, max_entries), E_b = ent_off[b+1] - ent_off[b].
 * key(s, c) = k_idx[ent_off[b] + s, c] for bf16 keys; for fp8 keys it is
 * decode(k_idx[ent_off[b] + s, c]) * k_scale[scale_off[b] + s / scale_group]; for MXFP4
 * keys ([P1] section 4.2, FP4 indexer; [P2] "Where It Breaks", the FP4 QK indexer) it is
 * e2m1(code c of row ent_off[b] + s) * 2^(E - 127), E the row's E8M0 byte for block c / 32.
 * No 1/sqrt(CI) factor is applied. scores[b, t, s] for s >= n(b, t) is not written.
 *
 *   q_idx   bf16 [B, T, HI, CI]     HI in {1, 2, 4, 8, 16}; CI == 64
 *   w       fp32 [B, T, HI]
 *   k_idx   [E_tot, CI] of k_dtype (CSL_DTYPE_BF16 or CSL_DTYPE_FP8_E4M3), or for
 *           CSL_DTYPE_MXFP4 uint8 [E_tot, CI/2]: byte j holds code 2j in its low nibble and
 *           code 2j+1 in its high nibble (8-byte aligned)
 *   k_scale fp8: fp32 scales with scale_off int64 [B+1], scale_group >= 1 entries per
 *           scale, scales positive (in a paged cache: per pool block, see csl_paged_cache). MXFP4: uint8 E8M0 [E_tot, CI/32], one per block of 32
 *           dims of a row, exponent bytes in [0, 254] (255, NaN, is a precondition
 *           violation); scale_off and scale_group are ignored. bf16: ignored (may be NULL).
 *   scores  fp32 [B, T, ld], ld >= max_entries
 *   topk_ws (nullable) with topk_ws_bytes >= csl_topk_workspace_bytes(B, T, max_entries,
 *           topk_k): when given with T == 1 and rows longer than 34816 entries, the kernel
 *           also leaves per-row top-k candidate lists in it (each 512-entry slice lists at
 *           most 16..64 entries, all of its entries above a slice-local cut), for the
 *           csl_topk_select call that follows with prepared = 1 and the same k and
 *           max_entries (rows of at most 2^20 entries); for other shapes it is not touched.
 * Arithmetic: bf16 MFMA products with fp32 accumulation; fp8 codes are widened to bf16
 * exactly before the product and the group scale multiplies the fp32 dot; MXFP4 codes are
 * widened and scaled to bf16 exactly (every such value is a bf16) before the product.
 */
int csl_indexer_scores(const void* q_idx, const float* w, const void* k_idx, int k_dtype,
                       const void* k_scale, const int64_t* scale_off, int scale_group,
                       const int64_t* ent_off, const int64_t* q_pos, int m, int B, int T, int HI,
                       int CI, int64_t max_entries, float* scores, int64_t ld, void* topk_ws,
                       size_t topk_ws_bytes, int topk_k, const csl_paged_cache* paged, void* stream);

/*
 * topk_select -- top-k compressed entries per query row ([P2] "Deep Dive", CSA top-k
 * selection; [P2] "Putting It Together"; [P1] section 4.1).
 *
 * For each row (b, t) with n = min(floor(p / m), E_b, max_entries) scores:
 *   idx[b, t, :] = the ids of the min(k, n) largest scores[b, t, 0:n], ordered by
 *   (score descending, id ascending) for the choice -- so the lower id wins a tie --
 *   then written in ASCENDING id order, padded with -1 up to k.
 * -0.0 and +0.0 compare equal. NaN scores are outside the contract.
 *
 *   scores fp32 [B, T, ld]; idx int32 [B, T, k]; 1 <= k <= 4096; max_entries <= 2^20.
 *   ws: device workspace of at least csl_topk_workspace_bytes(B, T, max_entries, k)
 *   bytes (may be NULL when that is 0); its contents on entry do not matter.
 *   prepared: 1 when the csl_indexer_scores call that wrote these scores was given this
 *   workspace, k and max_entries (its candidate lists are then used instead of a pass over
 *   the scores); 0 otherwise. The result is the same either way; if the lists cannot prove
 *   the selection exact (rows whose best entries crowd into a few 512-entry slices, or rows
 *   with more than 5 expected winners per 64 entries), the whole row is searched.
 * Integer work only: scores are compared through an order-preserving 32-bit key.
 */
size_t csl_topk_workspace_bytes(int B, int T, int64_t max_entries, int k);
int csl_topk_select(const float* scores, int64_t ld, const int64_t* ent_off, const int64_t* q_pos,
                    int m, int B, int T, int k, int64_t max_entries, int32_t* idx, void* ws,
                    size_t ws_bytes, int prepared, void* stream);

/*
 * indexer_topk -- the indexer fused with the top-k selection, the scores never written
 * ([P2] "Deep Dive", CSA Lightning Indexer and top-k selection; [P5] the indexer score
 * formula; [P1] section 4.2).
 *
 *   idx[b, t, :] = topk_select(indexer_scores(...))[b, t, :]
 *
 * The scores come from the arithmetic of indexer_scores' prefill tiling (taken when
 * B*T >= 64 and T >= 16, without candidate lists), so for such shapes the result equals
 * the two calls bit for bit; for others the scores differ from indexer_scores' only in the
 * fp32 rounding of the head sum's order. The choice is (score descending, id ascending)
 * and the output ascending ids, -1 padded, as for topk_select. Arguments are those of
 * indexer_scores (keys, scales, offsets, paged cache) and topk_select (k, idx), without the
 * score buffer and workspace.
 *
 *   k     1 <= k <= csl_indexer_topk_max_k(HI) (1952 for HI = 2 .. 16, 672 for HI = 1)
 *   idx   int32 [B, T, k]
 * One workgroup scores 8 query rows (16 at HI = 1) against all of their visible entries
 * and keeps each row's candidates in on-chip memory (two workgroups per compute unit up to
 * k = 672, one beyond), so the call suits batches of many query rows (prefill); a single
 * decode row is better served by indexer_scores with candidate lists and topk_select. No
 * workspace; nothing but idx is written.
 */
int csl_indexer_topk_max_k(int HI);
int csl_indexer_topk(const void* q_idx, const float* w, const void* k_idx, int k_dtype, const void* k_scale,
                     const int64_t* scale_off, int scale_group, const int64_t* ent_off, const int64_t* q_pos,
                     int m, int B, int T, int HI, int CI, int64_t max_entries, int k, int32_t* idx,
                     const csl_paged_cache* paged, void* stream);

/*
 * sparse_attn_decode -- CSA core attention ([P2] "Deep Dive", CSA core attention with
 * shared-KV MQA and the sliding-window branch; [P2] "Putting It Together"; [P5] the
 * attention formula):
 *
 *   X(b, t) = { ckv[ent_off[b] + idx[b,t,v]] : 0 <= idx[b,t,v] < E_b } followed by the raw
 *             window rows kv[kv_off[b] + j], j in [max(0, hi - n_win + 1), hi],
 *             hi = min(p, N_b - 1)
 *   out[b, t, h] = sum_{x in X} softmax_x(scale * q[b,t,h] . x) x   (K = V, one softmax)
 *   lse[b, t, h] = log sum_{x in X} exp(scale * q[b,t,h] . x)        (natural log)
 * An empty X gives out = 0 and lse = -inf. No de-duplication between the two lanes.
 *
 *   q bf16 [B, T, H, D]; ckv bf16 [E_tot, D]; idx int32 [B, T, k]; kv bf16 [N_tot, D]
 *   out fp32 [B, T, H, D]; lse fp32 [B, T, H] (nullable)
 *   D == 128; H a multiple of 16, <= 128; k >= 0; n_win >= 0; scale finite and > 0
 *   (CSL_ERR_INVALID otherwise).
 *   ws: at least csl_attn_workspace_bytes(B, T, H, D, k + n_win) bytes (contents free).
 * extras (nullable; NULL means none of them) adds per-query parts of the core attention:
 *   sink       device fp32 [H] or NULL: head h's sink logit z'_h ([P1] section 7). exp(z'_h)
 *              joins the softmax denominator with no value, so the weights sum to less
 *              than one: out = sum_x exp(l_x - lse) x, lse = log(exp(z'_h) + sum_x exp(l_x)).
 *              An empty X then gives out = 0 and lse = z'_h.
 *   rope_dims  0 or 64 ([P1] section 8, partial RoPE on the last 64 dims): the last R = 64
 *              dims of q are rotated at the query position p before the scores, and the
 *              same dims of out at -p after normalisation (the inverse rotation on the
 *              output side). Pair j = (dims D - R + 2j, D - R + 2j + 1) turns by the angle
 *              pos * rope_base^(-2j/R), counter-clockwise. Key rows (ckv, kv) are used as
 *              stored: rotating them at their own positions is up to their writer. Other
 *              widths return CSL_ERR_UNSUPPORTED.
 *   rope_base  > 1 and finite when rope_dims > 0 (the original RoPE uses 10000).
 * Arithmetic: bf16 MFMA operands with fp32 accumulation; each probability enters the value
 * product as two bf16 terms (hi + bf16(p - hi)), so it carries ~2^-16 relative error, and so
 * does each rotated query dim; fp32 online softmax in base 2; log-sum-exp merge of split
 * partials. RoPE angles are formed and reduced to one turn in double precision; their sine
 * and cosine come from the hardware instructions (absolute error about 1e-6).
 */
typedef struct csl_attn_extras {
  const float* sink; /* device fp32 [H], or NULL */
  int rope_dims;     /* 0 or 64 */
  float rope_base;   /* > 1 when rope_dims > 0 */
} csl_attn_extras;

size_t csl_attn_workspace_bytes(int B, int T, int H, int D, int64_t max_keys);
int csl_sparse_attn_decode(const void* q, const void* ckv, const int32_t* idx, int k,
                           const void* kv, const int64_t* kv_off, const int64_t* ent_off,
                           const int64_t* q_pos, int n_win, int B, int T, int H, int D, float scale,
                           float* out, float* lse, void* ws, size_t ws_bytes,
                           const csl_attn_extras* extras, const csl_paged_cache* paged, void* stream);

/*
 * hca_attn_decode -- HCA dense attention ([P1] section 5.1; [P2] "Heavily Compressed
 * Attention"): as sparse_attn_decode, with the compressed part of X being every visible
 * entry s < min(floor(p / m), E_b, max_entries) instead of a selected list.
 *   ws: at least csl_attn_workspace_bytes(B, T, H, D, max_entries + n_win) bytes.
 *   extras: as for sparse_attn_decode.
 */
int csl_hca_attn_decode(const void* q, const void* ckv, const void* kv, const int64_t* kv_off,
                        const int64_t* ent_off, const int64_t* q_pos, int m, int n_win, int B,
                        int T, int H, int D, float scale, int64_t max_entries, float* out,
                        float* lse, void* ws, size_t ws_bytes, const csl_attn_extras* extras,
                        const csl_paged_cache* paged, void* stream);

/*
 * csa_decode_step -- one whole CSA step of one layer ([P2] "Putting It Together"; [P1]
 * section 4.1): exactly
 *     csl_compress_kv(kv, z, kv_off, ent_off, first_entry, B, D, m, max_new_entries, ckv, BF16)
 *     csl_indexer_scores(q_idx, w, k_idx, ..., scores, ld, topk_ws, topk_ws_bytes, k)
 *     csl_topk_select(scores, ..., k, idx, topk_ws, topk_ws_bytes, prepared = 1)
 *     csl_sparse_attn_decode(q, ckv, idx, k, kv, ..., n_win, ..., out, lse, attn_ws)
 * in that order on one stream, with the same outputs (ckv rows, scores, idx, out, lse) up to
 * the rounding order of the pooled sums where the compression runs inside the indexer launch
 * (one bf16 unit in a compressed entry). The calls' own argument rules apply to the fields
 * below, and everything is validated before anything is enqueued. Where the shapes allow
 * (D == 128, m <= 8, the decode tiling of the indexer), the compression runs in spare
 * workgroups of the indexer launch instead of a launch of its own; it never reads what the
 * indexer writes, and the attention runs after both. Where one attention workgroup per query
 * row holds the row's whole key list (k + n_win spanning 2 to 4 tiles of 64 keys at H = 16,
 * 32 or 64, 2 tiles at H = 128, fewer than 512 query rows, k <= 256, max_entries <=
 * 1024 * H / 16 and <= 4096, unpaged), that workgroup selects the row's top-k from the scores
 * itself, with csl_topk_select's rule, and writes the same ids to idx: the top-k launch is
 * then left out.
 * With kv_b (and z_b when z is given) set, the compression is csl_compress_kv_overlap
 * of the series pair (kv, z) and (kv_b, z_b) instead, carried the same way; kv_b and z_b
 * both NULL keeps single-series compression. With scores NULL the indexer and top-k calls
 * are replaced by csl_indexer_topk (no score matrix; topk_ws, topk_ws_bytes and ld are
 * ignored; k <= csl_indexer_topk_max_k(HI)), for batches of many query rows.
 */
typedef struct csl_csa_step {
  /* raw K = V cache and the compression this step adds to ckv */
  const void* kv;             /* bf16 [N_tot, D] */
  const void* z;              /* bf16 [N_tot, D] compression logits, or NULL (uniform) */
  const int64_t* kv_off;      /* device [B+1] */
  const int64_t* ent_off;     /* device [B+1] */
  const int64_t* first_entry; /* device [B] or NULL (0): first entry compressed */
  int64_t max_new_entries;    /* entries compressed per sequence, >= 0 */
  void* ckv;                  /* bf16 [E_tot, D] compressed cache: written, then attended */
  /* indexer */
  const void* q_idx;          /* bf16 [B, T, HI, CI] */
  const float* w;             /* fp32 [B, T, HI] */
  const void* k_idx;          /* [E_tot, CI] of k_dtype */
  int k_dtype;
  const void* k_scale;        /* as for csl_indexer_scores */
  const int64_t* scale_off;
  int scale_group;
  int HI;
  int CI;
  float* scores;              /* fp32 [B, T, ld], or NULL: indexer fused with top-k */
  int64_t ld;
  void* topk_ws;              /* csl_topk_workspace_bytes(B, T, max_entries, k) bytes */
  size_t topk_ws_bytes;
  /* selection */
  int k;
  int32_t* idx;               /* int32 [B, T, k] */
  /* attention */
  const void* q;              /* bf16 [B, T, H, D] */
  int H;
  int D;
  int n_win;
  float scale;
  float* out;                 /* fp32 [B, T, H, D] */
  float* lse;                 /* fp32 [B, T, H] or NULL */
  void* attn_ws;              /* csl_attn_workspace_bytes(B, T, H, D, k + n_win) bytes */
  size_t attn_ws_bytes;
  /* geometry */
  const int64_t* q_pos;       /* device [B] */
  int m;
  int B;
  int T;
  int64_t max_entries;
  /* overlapped compression (NULL, NULL: one series) */
  const void* kv_b;           /* bf16 [N_tot, D] series b, or NULL */
  const void* z_b;            /* bf16 [N_tot, D] its logits: given exactly when z is */
  /* attention extras, as csl_attn_extras (sink NULL and rope_dims 0: none) */
  const float* sink;          /* device fp32 [H], or NULL */
  int rope_dims;
  float rope_base;
  /* paged cache (NULL: packed) */
  const csl_paged_cache* paged;
  /* 0: scores are written for every visible entry, as csl_indexer_scores does. Nonzero
   * (scores on demand): rows whose selection runs on candidate lists keep no scores (their
   * rows of `scores` are not written), which saves the score stores' share of the indexer's
   * HBM traffic; the selected ids, out and lse are the same. A row whose lists cannot prove
   * its selection (its winners crowd into a few 512-entry slices) has its row of `scores`
   * rebuilt inside the top-k launch before the exact row pass: the slices that could hide a
   * winner recomputed whole with the indexer's arithmetic and bits, the listed entries of the
   * others at their scores, elsewhere the NaN with every bit set (a row with fewer listed
   * entries than k is recomputed whole, streaming its keys through one workgroup). For single
   * query rows (T == 1) on candidate lists (max_entries > 34,816 and the finishing workgroup's
   * slots at most 8,192), packed layout; ignored otherwise. scores must still be given. */
  int scores_on_demand;
} csl_csa_step;

int csl_csa_decode_step(const csl_csa_step* s, void* stream);

/*
 * hca_decode_step -- one whole HCA step of one layer ([P1] section 5.1; [P2] "Heavily
 * Compressed Attention", HCA "How it works"): exactly
 *     csl_compress_kv(kv, z, kv_off, ent_off, first_entry, B, 128, m, max_new_entries, ckv, BF16)
 *     csl_hca_attn_decode(q, ckv, kv, kv_off, ent_off, q_pos, m, n_win, B, T, H, 128, ...)
 * in that order on one stream, with the same outputs up to the rounding order of the pooled
 * sums (one bf16 unit in a compressed entry, and what follows from it in out and lse). For H
 * in {16, 32, 64, 128}, 1 <= max_new_entries <= 4 and B * (T + max_new_entries) <= 65535
 * (and rows of more than 64 keys at fewer than 512 query rows, whose attention plan does not
 * multiply a row's few tiles at once) both run in one launch: spare workgroups pool the new
 * entries into the cache while the others attend, and an attention workgroup whose key range
 * holds an entry being rewritten pools that entry itself from the raw rows instead of
 * reading the cache. In a decode step no query sees the entry its own
 * token completes (a query sees only entries before its own block), so the compression then
 * costs the attention nothing. Other head counts run the two calls one after the other. All
 * fields follow the two calls' argument rules (D = 128, bf16 cache) and are validated before
 * anything is enqueued.
 */
typedef struct csl_hca_step {
  const void* kv;             /* bf16 [N_tot, 128] raw K = V rows */
  const void* z;              /* bf16 [N_tot, 128] compression logits, or NULL (uniform) */
  const int64_t* kv_off;      /* device [B+1] */
  const int64_t* ent_off;     /* device [B+1] */
  const int64_t* first_entry; /* device [B] or NULL (0): first entry compressed */
  int64_t max_new_entries;    /* entries compressed per sequence, >= 0 */
  void* ckv;                  /* bf16 [E_tot, 128] compressed cache: written, then attended */
  const void* q;              /* bf16 [B, T, H, 128] */
  int H;
  int n_win;
  float scale;
  float* out;                 /* fp32 [B, T, H, 128] */
  float* lse;                 /* fp32 [B, T, H] or NULL */
  void* attn_ws;              /* csl_attn_workspace_bytes(B, T, H, 128, max_entries + n_win) bytes */
  size_t attn_ws_bytes;
  const int64_t* q_pos;       /* device [B] */
  int m;
  int B;
  int T;
  int64_t max_entries;
  const float* sink;          /* attention extras as csl_attn_extras: sink NULL, rope_dims 0: none */
  int rope_dims;
  float rope_base;
  const csl_paged_cache* paged; /* NULL: packed */
} csl_hca_step;

int csl_hca_decode_step(const csl_hca_step* s, void* stream);

/*
 * csa_decode_step_static -- csl_csa_decode_step for callers that cannot allocate device
 * memory (code under stream or graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same step, outputs and argument rules, but s->topk_ws, s->topk_ws_bytes,
 * s->attn_ws and s->attn_ws_bytes are ignored. Both workspaces are taken instead from a
 * device array of CSL_STATIC_SCRATCH_BYTES inside the library, one copy per GPU, held until
 * the process ends; its address on a device is looked up on the first call made with that
 * device current. The call allocates and frees nothing.
 *   - A step whose workspaces (csl_topk_workspace_bytes with a score buffer, 256-byte
 *     aligned, plus csl_attn_workspace_bytes for k + n_win keys) exceed
 *     CSL_STATIC_SCRATCH_BYTES returns CSL_ERR_WORKSPACE and enqueues nothing.
 *   - Every call on one device uses that device's one array: calls whose work overlaps in
 *     time on one device (other streams, other threads) race and give undefined results.
 *     Serialise them, or use csl_csa_decode_step with buffers of your own.
 *   - The array keeps what the last call left in it; no call relies on its contents.
 */
#define CSL_STATIC_SCRATCH_BYTES (16u << 20)
int csl_csa_decode_step_static(const csl_csa_step* s, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* CSL_H */
