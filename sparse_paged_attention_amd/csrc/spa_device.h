// Device-side KV-set metadata and page-table translation.
//
// One definition serves the attention kernel and the gather-metadata export,
// so the exported rows are exactly the rows the attention reads.
//
// KV set of a query at position t of sequence b (ATOM PR "test: add
// block-level DeepSeek-V4 attention test", sections "What the reference
// proves" and "Validation"; RL-Kernel PR "Roadmap item 24", section
// "Contracts and lifetime"):
//   window       raw positions max(0, t-W+1) .. t
//   n_c          floor((t+1)/r) complete ratio-r groups (0 when r = 0)
//   compressed   the first cmp_cnt ids of the query's list (top-k layer), or
//                ids 0 .. n_c-1 (all-groups layer)
// Canonical entry order: compressed entries 0 .. n_sel-1, then the window.
// Page translation (RL-Kernel "Fixed paged CK attention on ROCm"): 64-bit
// row = page_table[b][p / P] * P + p % P.
//
// The translation is split in two steps (logical id, then physical row) so
// that a caller can issue every list load of a batch of entries before any
// page-table load.
#pragma once

#include "spa_internal.h"

namespace spa {

struct QueryKV {
  int32_t b, t, win_lo, win_len, n_c, n_sel;
};

__device__ __forceinline__ void flag_error(const Params &p, int32_t bits) {
  if (p.err_flag) atomicOr(p.err_flag, bits);
}

// KV-set counts of a query at position t of sequence b (b in range), with
// len = seq_lens[b] and cnt its list count (top-k layers).  `report` raises
// the error bits; without it the counts are also computed for t >= len
// (a caller that does not know len yet passes INT32_MAX).
__device__ __forceinline__ QueryKV query_kv_of(const Params &p, int32_t b, int32_t t, int32_t len,
                                               int32_t cnt, bool report) {
  QueryKV kv{0, 0, 0, 0, 0, 0};
  if (t < 0 || t >= len) {
    if (report) flag_error(p, kErrQuery);
    return kv;
  }
  kv.b = b;
  kv.t = t;
  kv.win_lo = p.window > 0 ? max(0, t - p.window + 1) : t + 1;
  kv.win_len = t - kv.win_lo + 1;
  kv.n_c = p.ratio > 0 ? (t + 1) / p.ratio : 0;
  if (p.ratio > 0 && p.topk > 0) {
    int32_t c = cnt;
    if (c < 0 || c > p.topk) {
      if (report) flag_error(p, kErrCount);
      c = c < 0 ? 0 : p.topk;
    }
    kv.n_sel = c;
  } else {
    kv.n_sel = p.ratio > 0 ? kv.n_c : 0;
  }
  return kv;
}

__device__ __forceinline__ QueryKV query_kv(const Params &p, int32_t i) {
  const int32_t b = p.query_seq ? p.query_seq[i] : i;
  if (b < 0 || b >= p.num_seqs) {
    flag_error(p, kErrQuery);
    return QueryKV{0, 0, 0, 0, 0, 0};
  }
  const int32_t len = p.seq_lens[b];
  const int32_t t = p.query_pos ? p.query_pos[i] : len - 1;
  return query_kv_of(p, b, t, len, (p.ratio > 0 && p.topk > 0) ? p.cmp_cnt[i] : 0, true);
}

// A listed compressed id is usable only if it names a complete group.
__device__ __forceinline__ int32_t check_cmp_id(const Params &p, const QueryKV &kv, int32_t c) {
  if (c < 0 || c >= kv.n_c) {
    flag_error(p, kErrCmpId);
    return -1;
  }
  return c;
}

// Step 1: logical id of canonical entry e (a compressed id when e < n_sel,
// else a raw position); -1 when the listed id is not a complete group.
__device__ __forceinline__ int32_t entry_logical(const Params &p, const QueryKV &kv, int32_t i,
                                                 int32_t e) {
  if (e < kv.n_sel) return check_cmp_id(p, kv, p.topk > 0 ? p.cmp_idx[(int64_t)i * p.topk + e] : e);
  return kv.win_lo + (e - kv.n_sel);
}

// Step 2: physical row (within its pool) of logical id `x` of the given kind,
// or -1 when the page-table column or the page id is out of range.
__device__ __forceinline__ int64_t logical_row(const Params &p, const QueryKV &kv, bool cmp, int32_t x) {
  if (x < 0) return -1;
  const int32_t P = p.page_size;
  const int32_t col = x / P;
  const int32_t stride = cmp ? p.cmp_pt_stride : p.raw_pt_stride;
  if (col >= stride) {
    flag_error(p, kErrPage);
    return -1;
  }
  const int32_t page = (cmp ? p.cmp_pt : p.raw_pt)[(int64_t)kv.b * stride + col];
  if (page < 0 || (int64_t)page >= (cmp ? p.cmp_pages : p.raw_pages)) {
    flag_error(p, kErrPage);
    return -1;
  }
  return (int64_t)page * P + (x - col * P);
}

__device__ __forceinline__ int64_t entry_row(const Params &p, const QueryKV &kv, int32_t i, int32_t e) {
  return logical_row(p, kv, e < kv.n_sel, entry_logical(p, kv, i, e));
}

}  // namespace spa
