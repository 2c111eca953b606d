// Internal interface between the C-ABI host code (spa_api.cpp) and the HIP
// kernels.  Not installed; the public interface is include/spa.h.
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

namespace spa {

// Device error bits (mirrors the err_flag convention of include/spa.h).
enum : int32_t { kErrQuery = 1, kErrCmpId = 2, kErrPage = 4, kErrCount = 8 };

// Everything a kernel needs, passed by value as a kernel argument.
struct Params {
  const uint16_t *q;                  // bf16 [Nq, Hq, D]
  const uint8_t *k_raw, *v_raw;       // bf16 rows
  const uint8_t *k_cmp, *v_cmp;       // bf16 or e4m3 rows
  const float *k_cmp_scale, *v_cmp_scale;
  int64_t raw_pages, cmp_pages;
  const int32_t *raw_pt, *cmp_pt;
  const int32_t *seq_lens, *query_seq, *query_pos;
  const int32_t *cmp_idx, *cmp_cnt;
  const float *sink;
  uint16_t *o;
  float *lse;
  float *part_o, *part_lse;           // split partials (num_splits > 1)
  int32_t *err_flag;
  int32_t raw_pt_stride, cmp_pt_stride;
  int32_t num_seqs, num_queries, hq, hkv, head_dim, page_size, window, ratio, topk, num_splits;
  int32_t group;                      // Hq / Hkv
  int32_t heads_per_block;            // query heads per job: 32 or 64
  int32_t head_groups;                // ceil(group / heads_per_block)
  // Jobs: (query i, KV head g, split s, head block hb).  A unit is one
  // (i, g) pair: u = i * Hkv + g, holding jobs_per_unit = num_splits *
  // head_groups jobs, r = s * head_groups + hb.  One launch covers the units
  // [unit_begin, unit_end).
  int32_t jobs_per_unit;
  int32_t unit_begin, unit_end;
  int32_t page_shift;                 // log2(page_size) when a power of two, else -1
  int32_t cmp_fp8;                    // e4m3 compressed pages
  int32_t cmp_fnuz;                   // ... in the FNUZ variant (decode slices only)
  float scale_log2;                   // scale * log2(e)
  int32_t num_cus;                    // compute units of the device (prefill pairs' item order)
};

hipError_t launch_attention(const Params &p, hipStream_t stream);

// Compute units of the current device (cached per device; 0 if unknown).
int32_t device_cu_count();

// Prefill with query pairs sharing KV tiles (spa_pair.hip): bf16 caches,
// D 128, one slice, a top-k list (or no compressed part) and at most
// kPairRowsMax rows in the union of a pair's KV sets, which holds whenever
// 2 * (topk + window) <= kPairRowsMax.
constexpr int kPairRowsMax = 1280;
constexpr int kMaxSplits = 64;      // SPA_MAX_SPLITS
constexpr int kPairStages = 3;      // LDS stages of the tile pipeline (prefill pairs)
bool prefill_pairs_eligible(const Params &p);
hipError_t launch_prefill_pairs(const Params &p, hipStream_t stream);
// Decode (spa_decode.hip): D 128, bf16 or e4m3 compressed pages, one
// workgroup per (query, KV head, 128-head block, KV slice), a slice's rows
// (compressed ones rounded up to whole tiles for e4m3) within
// kDecodeRowsMax.  With several slices it writes sink-free partials (plain
// row order) for the LSE merge.
constexpr int kDecodeRowsMax = 1280;
bool decode_eligible(const Params &p);
hipError_t launch_decode(const Params &p, hipStream_t stream);
// Decode in one KV pass per query (spa_decode_rows.hip): D 128, one slice,
// bf16 or e4m3 compressed pages; one workgroup per (query, KV head, block of
// 32 query heads) whose waves split the rows, their states combined in LDS.
// halves (bf16 pages): two workgroups per such block, each forming half of
// O's dimensions from all of K and its half of V.
bool decode_rows_eligible(const Params &p);
hipError_t launch_decode_rows(const Params &p, bool halves, hipStream_t stream);
// 512-wide heads over a shared latent cache (spa_latent.hip): bf16, k_raw ==
// v_raw and k_cmp == v_cmp; one workgroup per (query, KV head, 64-head block,
// KV slice); with several slices it writes sink-free partials (plain order).
hipError_t launch_latent(const Params &p, hipStream_t stream);
// unit_rows > 0: rows come in units of unit_rows consecutive rows (the query
// heads of one (query, KV head) pair), unit u's partials written on XCD
// u mod 8; the merge then reads each unit on that XCD.  0: plain order.
hipError_t launch_merge(const float *o_parts, const float *lse_parts, int32_t num_parts,
                        int64_t rows, int32_t head_dim, int32_t num_q_heads, const float *sink,
                        uint16_t *o_out, float *lse_out, int32_t unit_rows, hipStream_t stream);
hipError_t launch_gather(const Params &p, int32_t cap, int64_t *rows_out, int32_t *counts_out,
                         hipStream_t stream);
// Top-k selection from per-token scores (spa_topk.hip); 1 <= k <= kTopkMax.
constexpr int kTopkMax = 2048;
hipError_t launch_topk(const float *scores, int64_t ld, const int32_t *n_valid, int32_t rows, int32_t k,
                       int32_t *ids_out, int32_t *cnt_out, bool by_id, hipStream_t stream);

// Backward (spa_backward.hip): bf16 caches, D 128.  dq is written; the
// gradient caches and dsink are accumulated into.
struct BwdParams {
  const uint16_t *d_o, *o;            // bf16 [Nq, Hq, D]
  const float *lse;                   // [Nq, Hq], natural log
  float *dq;                          // [Nq, Hq, D]
  float *dk_raw, *dv_raw, *dk_cmp, *dv_cmp;   // the caches' layouts
  float *dsink_part;                  // [Nq, Hq] scratch, or null (no sink gradient)
  float *dsink;                       // [Hq], or null
  float scale;
  float *lse2_ws, *delta_ws;          // [Nq, Hkv, gp] LSE log2(e) and Delta per head, or null
  int32_t gp;                         // heads per KV head padded to 32
};

// Work plan of the KV-block pass (dK and dV summed per block of 32 rows of
// one sequence's raw or compressed rows, four blocks per workgroup, over
// slices of the queries).  Carved from the caller's workspace by
// backward_kv_workspace.
struct BwdKvPlan {
  int32_t nb_raw, nb_cmp;             // blocks per sequence
  int32_t ng_raw, ng_cmp;             // groups of four blocks per sequence
  int32_t nch;                        // query slices
  uint32_t *bitmap;                   // [Nq, nb_cmp] listed groups (top-k layers)
  int32_t *n_extra;                   // repeated listings: count
  int2 *extra;                        // and (query, group) entries
  int32_t cap_extra;
};
bool backward_eligible(const Params &p);
// the KV-block path: a prefill call (D 128, bf16 caches) whose compressed
// blocks per sequence fit the plan's bitmap
bool backward_kv_eligible(const Params &p);
// Workspace bytes of the KV-block path (the sink partials included); with
// base non-null, also carves `pl` and the LSE / Delta arrays of `b` from it.
size_t backward_kv_workspace(const Params &p, void *base, BwdKvPlan *pl, BwdParams *b);
// query pairs (four waves, the union of two KV sets): a prefill call with a
// top-k list or no compressed part and 2 * (topk + window) <= kPairRowsMax
bool backward_pairs_eligible(const Params &p);
hipError_t launch_backward(const Params &p, const BwdParams &b, bool pairs, const BwdKvPlan *kv, hipStream_t stream);

}  // namespace spa
