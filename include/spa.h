/*
 * spa.h — C ABI of the MI355X (gfx950) sparse paged attention library.
 *
 * The operation (RL-Kernel PR "Roadmap item 24: joint compressed/window
 * attention with sink", section "Reuse and arithmetic"; ATOM PR "test: add
 * block-level DeepSeek-V4 attention test", sections "What the reference
 * proves" and "Validation"): for every query token t of sequence b and every
 * query head h (KV head g = h / (Hq / Hkv)), the KV set is
 *
 *   compressed rows  the ids listed for the query (a top-k "CSA" layer), or
 *                    every complete group (an all-groups "HCA" layer), where
 *                    group c of ratio r is complete at t when r*(c+1) <= t+1;
 *                    none when ratio = 0 (a dense layer);
 *   window rows      raw positions max(0, t-W+1) .. t,
 *
 * in this canonical order ([compressed in list order || window ascending]).
 * Each logical position p (or compressed id c) is translated through its
 * sequence's page table: row = page_table[b][p / P] * P + p % P, in 64-bit
 * arithmetic (RL-Kernel "Fixed paged CK attention on ROCm").  Then
 *
 *   s_j = scale * <q_h, k_j>
 *   O   = sum_j exp(s_j) v_j / (sum_j exp(s_j) + exp(sink_h))
 *   LSE = ln(sum_j exp(s_j) + exp(sink_h))
 *
 * The sink logit is per head, is not scaled, and has no value row.  O is
 * written as bf16 (round to nearest even), LSE as fp32 natural log.
 *
 * Conventions for every call:
 *  - All data pointers are DEVICE pointers owned by the caller.  The library
 *    allocates nothing, keeps no global state except a thread-local error
 *    string, never synchronises, and enqueues its kernels on `stream` (a
 *    hipStream_t; NULL = the null stream).  Calls may be captured in a HIP
 *    graph.
 *  - Host-side validation runs before any HIP call and returns a distinct
 *    negative status per fault class (RL-Kernel joint attention PR, review of
 *    the guard matrix: one distinct error per fault).  attn_last_error()
 *    returns a message naming the offending argument.  Nothing is retried and
 *    there is no fallback path.
 *  - Per-element metadata (sequence ids, positions, compressed ids, page ids,
 *    list counts) is checked on the device.  A violating entry is masked
 *    (never dereferenced) and, when err_flag is not NULL, a bit is OR-ed into
 *    *err_flag: 1 = query sequence/position, 2 = compressed id outside the
 *    complete groups, 4 = page id outside the pool or page-table column out of
 *    range, 8 = list count outside [0, topk].  Page ids in page-table
 *    columns past the last page a query needs are never used to address a
 *    cache (RL-Kernel "Fixed paged CK attention on ROCm": the ids of unused
 *    columns must not reach the loads); the decode kernel may read such
 *    columns of a row no longer than 2048 entries (both tables together) in
 *    one wide load, within the row.
 *  - Inputs are read-only.  After SPA_ERR_LAUNCH the outputs and the
 *    workspace are undefined.
 */
#ifndef SPA_H_
#define SPA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum spa_status {
  SPA_OK = 0,
  SPA_ERR_NULL = -1,        /* a required pointer is NULL                          */
  SPA_ERR_SHAPE = -2,       /* a count or dimension is out of range / inconsistent */
  SPA_ERR_DTYPE = -3,       /* unknown dtype code, or raw KV not bf16              */
  SPA_ERR_UNSUPPORTED = -4, /* valid request this library does not implement
                               (head_dim other than 64/128/512, ...)              */
  SPA_ERR_ALIGN = -5,       /* a pointer lacks the alignment its call requires     */
  SPA_ERR_WORKSPACE = -6,   /* workspace NULL or smaller than attn_workspace_size  */
  SPA_ERR_SPLITS = -7,      /* num_splits outside [1, SPA_MAX_SPLITS]              */
  SPA_ERR_LAUNCH = -8,      /* HIP reported an error when launching                */
  SPA_ERR_MODE = -9         /* decode/prefill query arguments do not match the call */
} spa_status;

typedef enum spa_dtype {
  SPA_BF16 = 0,
  SPA_FP8_E4M3_OCP = 1,     /* OCP e4m3: bias 7, no inf, 0x7F/0xFF NaN, max 448 */
  SPA_FP8_E4M3_FNUZ = 2     /* FNUZ e4m3 (the gfx942 format, named beside OCP in
                               the RL-Kernel joint attention PR, "Reuse and
                               arithmetic"): bias 8, no inf, no -0, 0x80 NaN,
                               max 240.  Compressed pages only, wherever
                               e4m3 pages are taken (the forward at every
                               head_dim); SPA_ERR_UNSUPPORTED in the
                               backward, as for OCP                        */
} spa_dtype;

#define SPA_MAX_SPLITS 64

typedef struct spa_fwd_args {
  int32_t num_seqs;       /* B                                                   */
  int32_t num_queries;    /* Nq; decode: must equal B                            */
  int32_t num_q_heads;    /* Hq, a multiple of num_kv_heads                      */
  int32_t num_kv_heads;   /* Hkv                                                 */
  int32_t head_dim;       /* D in {64, 128, 512}.  512 is the shared latent
                              cache of the DeepSeek-V4 layout (RL-Kernel PR
                              "Roadmap item 24", review of the joint-attention
                              contract and the packed-page gather: one bf16
                              `_kv` buffer is K and V, heads 512 wide): it
                              needs v_raw == k_raw, v_cmp == k_cmp, with e4m3
                              compressed pages also v_cmp_scale ==
                              k_cmp_scale (one scale per latent row), and
                              heads_per_block = queries_per_block = 0
                              (SPA_ERR_UNSUPPORTED otherwise)                */
  int32_t page_size;      /* P >= 1 tokens (rows) per page, same for both caches */
  int32_t window;         /* W >= 0 raw tokens ending at the query token         */
  int32_t ratio;          /* r >= 0 tokens per compressed group; 0 = no groups   */
  int32_t topk;           /* list capacity (row stride of cmp_idx); 0 = every
                             complete group, no list                              */
  float scale;            /* > 0, multiplies q.k; not applied to the sink        */
  int32_t raw_dtype;      /* spa_dtype: must be SPA_BF16                         */
  int32_t cmp_dtype;      /* spa_dtype: SPA_BF16, SPA_FP8_E4M3_OCP or _FNUZ      */
  int32_t num_splits;     /* 1 = one pass; >1 = split-KV partials + LSE merge    */
  int32_t heads_per_block; /* query heads one job computes, sharing each KV
                              tile: 32 or 64, or 0 = chosen by the library: a
                              decode with head_dim 128 whose slice rows fit
                              (ceil(topk / num_splits), rounded up to 32 for
                              e4m3 pages, + ceil(window / num_splits) <=
                              1280, topk read as cmp_pt_stride * page_size
                              for an all-groups layer) takes 128 heads per
                              job when queries_per_block is 0 too, otherwise
                              64 when the KV group has more than 32 heads; a
                              tuning knob, the result does not depend on it */
  int32_t queries_per_block; /* queries one job serves, a tuning knob (the
                              result does not depend on it): 1 = one query per
                              job; 2 = query pairs (prefill only: two queries
                              stream the union of their KV sets through shared
                              tiles; needs bf16 caches, head_dim 128,
                              num_splits 1, topk > 0 or ratio 0, and
                              2 * (topk + window) <= 1280, else
                              SPA_ERR_UNSUPPORTED); 0 = library choice (pairs
                              for a prefill that fits them unless
                              heads_per_block is 32, else one query)        */

  const void *q;          /* bf16 [Nq, Hq, D]                                    */
  const void *k_raw;      /* bf16 [raw_pages, P, Hkv, D]                         */
  const void *v_raw;      /* bf16 [raw_pages, P, Hkv, D] (may alias k_raw)       */
  const void *k_cmp;      /* bf16 or e4m3 [cmp_pages, P, Hkv, D]; NULL if r = 0  */
  const void *v_cmp;      /* same layout as k_cmp (may alias it)                 */
  const float *k_cmp_scale; /* f32 [cmp_pages, P, Hkv]: FP8 only, else NULL     */
  const float *v_cmp_scale; /* f32 [cmp_pages, P, Hkv]: FP8 only, else NULL     */
  int64_t raw_pages;      /* pages in the raw pool (bound for page ids)          */
  int64_t cmp_pages;      /* pages in the compressed pool                        */
  const int32_t *raw_pt;  /* [B, raw_pt_stride] page ids                         */
  const int32_t *cmp_pt;  /* [B, cmp_pt_stride]; NULL if r = 0                   */
  int32_t raw_pt_stride;
  int32_t cmp_pt_stride;
  const int32_t *seq_lens;  /* [B] tokens in each sequence's raw cache           */
  const int32_t *query_seq; /* prefill [Nq] sequence of each query; decode NULL  */
  const int32_t *query_pos; /* prefill [Nq] position of each query; decode NULL
                               (decode query b sits at position seq_lens[b]-1)    */
  const int32_t *cmp_idx;   /* [Nq, topk] logical compressed ids (list order),
                               when topk > 0                                      */
  const int32_t *cmp_cnt;   /* [Nq] entries used in each list, when topk > 0     */
  const float *sink;        /* f32 [Hq] sink logits, or NULL (= -inf, no sink)   */

  void *o;                  /* out: bf16 [Nq, Hq, D]                             */
  float *lse;               /* out: f32 [Nq, Hq], natural log, sink included;
                               may be NULL                                        */
  int32_t *err_flag;        /* device i32 or NULL, see the conventions above     */
  void *workspace;          /* num_splits > 1: attn_workspace_size() bytes of
                               scratch for the split partials (no initial
                               contents needed), 16-byte aligned; one call at
                               a time                                        */
  size_t workspace_bytes;
} spa_fwd_args;

/* Bytes of workspace the call needs: 0 when num_splits == 1, otherwise the
   sink-free split partials f32 O [S, Nq, Hq, D] and f32 LSE [S, Nq, Hq]
   (the LSE at a 256-byte boundary; no initial contents needed): the buffer
   between a KV-split decode and its reduce in the decode trace of the ATOM PR
   "test: add block-level DeepSeek-V4 attention test", section "What this
   test actually drives".  Returns 0 for a NULL or inconsistent argument
   block. */
size_t attn_workspace_size(const spa_fwd_args *args);

/* Decode: one query per sequence at position seq_lens[b] - 1
   (query_seq = query_pos = NULL, num_queries = num_seqs).  With num_splits
   S > 1 every query's canonical KV list is cut into S slices, each slice
   yields a sink-free partial (O_s, LSE_s) in the workspace, and a second
   kernel on the same stream combines the partials plus the sink exactly as
   attn_merge_lse does (in slice order, so the result is deterministic). */
spa_status attn_fwd_decode(const spa_fwd_args *args, void *stream);

/* Decode that allocates nothing and needs no workspace, for callers that
   cannot allocate device memory (code under HIP graph capture, tight serving
   loops, harnesses that forbid allocation): the same operation and kernels
   as attn_fwd_decode, with the split partials in a scratch array of
   attn_noalloc_scratch_bytes() bytes (32 MiB) that the library holds per GPU
   until the process ends.  args->workspace and workspace_bytes are ignored.
   A call whose partials need more (4 * S * Nq * Hq * (D + 1) bytes, plus
   alignment) returns SPA_ERR_WORKSPACE before any HIP call.  Every call on a
   GPU shares that GPU's array (its contents are the last call's), so calls
   that overlap on one GPU (other streams, other host threads) race; they
   must be ordered by the caller. */
spa_status attn_fwd_decode_noalloc(const spa_fwd_args *args, void *stream);
size_t attn_noalloc_scratch_bytes(void);

/* Prefill / chunked prefill / multi-token decode: query i sits at
   (query_seq[i], query_pos[i]); every KV row it needs, its own and those of
   tokens of the same chunk included, is already in the paged caches. */
spa_status attn_fwd_prefill(const spa_fwd_args *args, void *stream);

/* Exact merge of sink-free partials (RL-Kernel PR "[WS2] CP-aware Attention
   contract", Behavior: deterministic (out, lse) reduction; tessera "Block
   AttnRes" PR: softmax_merge).  For every row r (r = query * Hq + head):
     LSE[r] = ln(sum_s exp(lse_parts[s][r]) + exp(sink[r % num_q_heads]))
     O[r]   = sum_s exp(lse_parts[s][r] - LSE[r]) * o_parts[s][r]
   An empty part has LSE = -inf and weight 0.  If every term is -inf the row
   gets O = 0, LSE = -inf.  o_parts f32 [num_parts, rows, head_dim],
   lse_parts f32 [num_parts, rows] (device); sink f32 [num_q_heads] or NULL;
   o_out bf16 [rows, head_dim]; lse_out f32 [rows] or NULL.
   head_dim in {64, 128, 512}; 1 <= num_parts <= SPA_MAX_SPLITS; o_parts 16-byte
   and o_out 8-byte aligned (else SPA_ERR_ALIGN). */
spa_status attn_merge_lse(const float *o_parts, const float *lse_parts, int32_t num_parts,
                          int64_t rows, int32_t head_dim, int32_t num_q_heads,
                          const float *sink, void *o_out, float *lse_out, void *stream);

/* Gather metadata, computed on the device by the same translation code the
   attention kernels use (the paged offsets that the ATOM PR "test: add
   block-level DeepSeek-V4 attention test" packs from the selected ids before
   the attention, sections "What this test actually drives" and "Why it
   drives the real metadata builder"): for each query, rows_out[i, :] holds the physical
   row index (within its pool) of every KV entry in canonical order — the
   n_sel compressed rows, then the win_len window rows — padded with -1 up to
   cap; counts_out[i] = {win_lo, win_len, n_c, n_sel}.  A masked (invalid)
   entry is reported as -2.  `decode` (nonzero) selects the decode query
   convention of attn_fwd_decode (query i of sequence i at seq_lens[i] - 1;
   query_seq and query_pos must be NULL); zero, that of attn_fwd_prefill.
   rows_out int64 [Nq, cap], counts_out int32 [Nq, 4] (device).  Entries past
   cap are not written; cap >= window + max list length suffices. */
spa_status attn_build_gather(const spa_fwd_args *args, int32_t decode, int32_t cap,
                             int64_t *rows_out, int32_t *counts_out, void *stream);

/* Top-k selection of compressed groups from per-token scores: the step
   before the attention core, whose selected ids become the query's list
   (cmp_idx / cmp_cnt).  ATOM PR "test: add block-level DeepSeek-V4
   attention test", sections "What this test actually drives" (the indexer
   scores, a radix top-k select, then the top-k -> paged offsets pack, which
   attn_build_gather exports) and "Validation" (the top-k truncates only once
   the complete groups outnumber it).  The scores themselves come from the
   caller; the pages do not define the indexer's scoring.
   For row i: the min(k, n_i) highest of scores[i * ld .. i * ld + n_i - 1],
   n_i = n_valid[i] clamped to [0, ld], in descending score order, ties by
   ascending id, -0.0 below +0.0, a NaN score below every number.
   scores f32 [num_rows, ld] (device, row stride ld); n_valid i32 [num_rows];
   ids_out i32 [num_rows, k]: ids in that order, -1 past the count;
   cnt_out i32 [num_rows]: min(k, n_i).  1 <= k <= SPA_MAX_TOPK
   (SPA_ERR_UNSUPPORTED otherwise), ld >= 1, num_rows >= 0 (SPA_ERR_SHAPE);
   NULL pointers give SPA_ERR_NULL. */
#define SPA_MAX_TOPK 2048
spa_status attn_topk_select(const float *scores, int64_t ld, const int32_t *n_valid, int32_t num_rows,
                            int32_t k, int32_t *ids_out, int32_t *cnt_out, void *stream);

/* The same selection as attn_topk_select, with the ids of each row written
   in ascending id order instead of by score (the same arguments, limits and
   errors).  The attention core takes a query's list as a set (its result
   depends on the order only through rounding), and ascending ids visit the
   compressed cache's pages in address order; this order also needs no sort
   of the selection. */
spa_status attn_topk_select_ids(const float *scores, int64_t ld, const int32_t *n_valid, int32_t num_rows,
                                int32_t k, int32_t *ids_out, int32_t *cnt_out, void *stream);

/* Backward pass: gradients of q, of both KV caches and of the sink, from
   the forward's saved O and LSE.  RL-Kernel PR "Roadmap item 24: joint
   compressed/window attention with sink": section "Reuse and arithmetic"
   keeps the fp32 LSE for the backward pass that follows the forward; the
   pages give no formulas, so these are the derivative of the forward's
   definition.  For one query head with KV rows j, s_j = scale <q, k_j>,
   p_j = exp(s_j - LSE), dp_j = <dO, v_j>, Delta = <dO, O> and
   ds_j = p_j (dp_j - Delta):
     dq = scale sum_j ds_j k_j           (written)
     dk_j += scale ds_j q, dv_j += p_j dO (accumulated into the row's cache slot)
     d_sink[h] += -sum_i exp(sink_h - LSE_ih) Delta_ih
   `args` describes the forward call exactly as it was made (decode when
   query_seq and query_pos are NULL, else prefill); args->o (bf16) and
   args->lse are that call's outputs and are read here; num_splits and
   heads_per_block are ignored.  queries_per_block: 0 lets the library
   choose; 1 takes one query per workgroup; 2 takes prefill query pairs,
   which stream the union of two neighbouring queries' KV sets so that a row
   both read is added once (a prefill call with a top-k list or no
   compressed part and 2 * (topk + window) <= 1280; SPA_ERR_UNSUPPORTED
   otherwise).  The library's choice is pairs wherever they fit.  Supported: bf16
   caches, head_dim 128 (SPA_ERR_UNSUPPORTED otherwise).
   grads->d_o bf16 [Nq, Hq, D], 16-byte aligned; grads->dq f32 [Nq, Hq, D];
   dk_raw/dv_raw f32 with the raw cache's layout [raw_pages, page_size,
   Hkv, D]; dk_cmp/dv_cmp f32 with the compressed cache's layout (required
   when ratio > 0); d_sink f32 [Hq] or NULL (no sink gradient; must be NULL
   when args->sink is).  The accumulated buffers are zeroed by the caller
   before the first call; dk/dv are added with float atomics, so their
   rounding order, and their last bits, vary from run to run.
   Workspace (args->workspace, 16-byte aligned, SPA_ERR_ALIGN otherwise):
   attn_bwd_workspace_size(args) bytes let a prefill call take the
   KV-block path, in which dk and dv are summed per block of 32 cache rows
   over every query that reads them and added once per block and slice of
   32 queries; the size then covers per-head LSE and Delta arrays and, for
   a top-k layer, a bitmap of each query's listed groups.  A smaller
   workspace (or a decode call) keeps the fused kernel, whose workgroups add
   dk and dv per query or query pair; it needs num_queries * num_q_heads * 4
   bytes with d_sink and none without (SPA_ERR_WORKSPACE when d_sink is
   set and the workspace is smaller).  Invalid metadata is flagged and
   masked as in the forward. */
typedef struct spa_bwd_grads {
  const void *d_o;
  float *dq;
  float *dk_raw, *dv_raw;
  float *dk_cmp, *dv_cmp;
  float *d_sink;
} spa_bwd_grads;

size_t attn_bwd_workspace_size(const spa_fwd_args *args);
spa_status attn_bwd(const spa_fwd_args *args, const spa_bwd_grads *grads, void *stream);

/* Message for the last non-OK status returned on this thread ("" if none):
   the reason behind the distinct status of each fault class (RL-Kernel joint
   attention PR, review of the guard matrix). */
const char *attn_last_error(void);

/* Library ABI version (this header: 1). */
int32_t attn_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SPA_H_ */
