// C-ABI entry points of libspa: host-side validation, workspace sizing and
// kernel launches.  See include/spa.h for the contract of every call.
//
// Validation follows the guard-matrix discussion in the RL-Kernel joint
// attention PR (review of test_joint_attention_rocm.py): every fault class
// returns its own status code before any HIP call, and the message names the
// argument.  There are no retries and no fallback path.

#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <mutex>
#include <string>

#include "spa.h"
#include "spa_internal.h"

namespace {

thread_local std::string g_last_error;

spa_status fail(spa_status code, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

spa_status ok() {
  g_last_error.clear();
  return SPA_OK;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Shape/dtype/pointer checks shared by the attention calls and the gather
// export.  `need_outputs` is false for the gather export.
spa_status validate(const spa_fwd_args *a, bool decode, bool need_outputs) {
  if (a == nullptr) return fail(SPA_ERR_NULL, "args is NULL");
  if (a->num_seqs < 1) return fail(SPA_ERR_SHAPE, "num_seqs must be >= 1 (got %d)", a->num_seqs);
  if (a->num_queries < 0) return fail(SPA_ERR_SHAPE, "num_queries must be >= 0 (got %d)", a->num_queries);
  if (a->num_q_heads < 1 || a->num_kv_heads < 1)
    return fail(SPA_ERR_SHAPE, "num_q_heads (%d) and num_kv_heads (%d) must be >= 1", a->num_q_heads,
                a->num_kv_heads);
  if (a->num_q_heads % a->num_kv_heads != 0)
    return fail(SPA_ERR_SHAPE, "num_q_heads (%d) must be a multiple of num_kv_heads (%d)", a->num_q_heads,
                a->num_kv_heads);
  if (a->page_size < 1) return fail(SPA_ERR_SHAPE, "page_size must be >= 1 (got %d)", a->page_size);
  if (a->window < 0) return fail(SPA_ERR_SHAPE, "window must be >= 0 (got %d)", a->window);
  if (a->ratio < 0) return fail(SPA_ERR_SHAPE, "ratio must be >= 0 (got %d)", a->ratio);
  if (a->topk < 0) return fail(SPA_ERR_SHAPE, "topk must be >= 0 (got %d)", a->topk);
  if (a->topk > 0 && a->ratio == 0) return fail(SPA_ERR_SHAPE, "topk > 0 needs ratio > 0");
  if (a->raw_pt_stride < 1) return fail(SPA_ERR_SHAPE, "raw_pt_stride must be >= 1");
  if (a->raw_pages < 1) return fail(SPA_ERR_SHAPE, "raw_pages must be >= 1");
  if (a->ratio > 0 && (a->cmp_pt_stride < 1 || a->cmp_pages < 1))
    return fail(SPA_ERR_SHAPE, "ratio > 0 needs cmp_pt_stride >= 1 and cmp_pages >= 1");
  if (a->head_dim != 64 && a->head_dim != 128 && a->head_dim != 512)
    return fail(SPA_ERR_UNSUPPORTED, "head_dim %d not supported (64, 128 or 512)", a->head_dim);
  if (a->head_dim == 512) {
    // the 512-wide path is the shared latent cache: one row is K and V
    if (a->k_raw != a->v_raw || (a->ratio > 0 && a->k_cmp != a->v_cmp))
      return fail(SPA_ERR_UNSUPPORTED, "head_dim 512 needs a shared latent cache (k_raw == v_raw, k_cmp == v_cmp)");
    if (a->ratio > 0 && a->cmp_dtype != SPA_BF16 && a->k_cmp_scale != a->v_cmp_scale)
      return fail(SPA_ERR_UNSUPPORTED, "head_dim 512 with e4m3 pages needs one shared scale array "
                  "(k_cmp_scale == v_cmp_scale)");
    if (a->heads_per_block != 0 || a->queries_per_block != 0)
      return fail(SPA_ERR_UNSUPPORTED, "head_dim 512 takes heads_per_block 0 and queries_per_block 0");
  }
  if (a->raw_dtype != SPA_BF16) return fail(SPA_ERR_DTYPE, "raw_dtype must be SPA_BF16 (got %d)", a->raw_dtype);
  if (a->cmp_dtype != SPA_BF16 && a->cmp_dtype != SPA_FP8_E4M3_OCP && a->cmp_dtype != SPA_FP8_E4M3_FNUZ)
    return fail(SPA_ERR_DTYPE, "cmp_dtype %d unknown", a->cmp_dtype);
  if (a->num_splits < 1 || a->num_splits > SPA_MAX_SPLITS)
    return fail(SPA_ERR_SPLITS, "num_splits %d outside [1, %d]", a->num_splits, SPA_MAX_SPLITS);
  if (a->heads_per_block != 0 && a->heads_per_block != 32 && a->heads_per_block != 64)
    return fail(SPA_ERR_UNSUPPORTED, "heads_per_block %d not supported (0, 32 or 64)", a->heads_per_block);
  if (a->queries_per_block < 0 || a->queries_per_block > 2)
    return fail(SPA_ERR_UNSUPPORTED, "queries_per_block %d not supported (0, 1 or 2)", a->queries_per_block);
  if (a->queries_per_block == 2 && decode)
    return fail(SPA_ERR_UNSUPPORTED, "queries_per_block 2 is a prefill layout");
  {
    const int64_t group = a->num_q_heads / a->num_kv_heads;
    const int64_t jobs = (int64_t)a->num_queries * a->num_kv_heads * a->num_splits * ((group + 31) / 32);
    if (jobs + 8 > 0x7FFFFFFFLL) return fail(SPA_ERR_SHAPE, "the job count exceeds the launch grid");
  }

  if (a->q == nullptr) return fail(SPA_ERR_NULL, "q is NULL");
  if (a->k_raw == nullptr || a->v_raw == nullptr) return fail(SPA_ERR_NULL, "k_raw/v_raw is NULL");
  if (a->raw_pt == nullptr) return fail(SPA_ERR_NULL, "raw_pt is NULL");
  if (a->seq_lens == nullptr) return fail(SPA_ERR_NULL, "seq_lens is NULL");
  if (a->ratio > 0) {
    if (a->k_cmp == nullptr || a->v_cmp == nullptr) return fail(SPA_ERR_NULL, "k_cmp/v_cmp is NULL");
    if (a->cmp_pt == nullptr) return fail(SPA_ERR_NULL, "cmp_pt is NULL");
    if (a->cmp_dtype != SPA_BF16 && (a->k_cmp_scale == nullptr || a->v_cmp_scale == nullptr))
      return fail(SPA_ERR_NULL, "FP8 compressed KV needs k_cmp_scale and v_cmp_scale");
  }
  if (a->topk > 0 && (a->cmp_idx == nullptr || a->cmp_cnt == nullptr))
    return fail(SPA_ERR_NULL, "topk > 0 needs cmp_idx and cmp_cnt");
  if (need_outputs && a->o == nullptr) return fail(SPA_ERR_NULL, "o is NULL");

  if (decode) {
    if (a->query_seq != nullptr || a->query_pos != nullptr)
      return fail(SPA_ERR_MODE, "decode takes no query_seq/query_pos (queries sit at seq_lens-1)");
    if (a->num_queries != a->num_seqs)
      return fail(SPA_ERR_MODE, "decode needs num_queries == num_seqs (%d vs %d)", a->num_queries, a->num_seqs);
  } else {
    if (a->query_seq == nullptr || a->query_pos == nullptr)
      return fail(SPA_ERR_MODE, "prefill needs query_seq and query_pos");
  }

  if (!aligned16(a->q) || !aligned16(a->k_raw) || !aligned16(a->v_raw))
    return fail(SPA_ERR_ALIGN, "q, k_raw and v_raw must be 16-byte aligned");
  if (a->ratio > 0 && (!aligned16(a->k_cmp) || !aligned16(a->v_cmp)))
    return fail(SPA_ERR_ALIGN, "k_cmp and v_cmp must be 16-byte aligned");
  if (need_outputs && !aligned16(a->o)) return fail(SPA_ERR_ALIGN, "o must be 16-byte aligned");
  return SPA_OK;
}

size_t round256(size_t x) { return (x + 255) / 256 * 256; }

// Workspace layout (num_splits > 1): partial O | partial LSE.
struct WorkspaceLayout {
  size_t part_o, part_lse, total;
};

WorkspaceLayout workspace_layout(const spa_fwd_args *a) {
  WorkspaceLayout w{0, 0, 0};
  if (a->num_splits <= 1) return w;
  const size_t rows = (size_t)a->num_queries * (size_t)a->num_q_heads;
  w.part_o = 0;
  w.part_lse = round256(rows * (size_t)a->head_dim * sizeof(float) * (size_t)a->num_splits);
  w.total = w.part_lse + rows * sizeof(float) * (size_t)a->num_splits;
  return w;
}

size_t workspace_bytes_for(const spa_fwd_args *a) { return workspace_layout(a).total; }

// Query heads per job: 64 (two compute waves sharing each KV tile) unless
// the KV group has at most 32 heads, or the caller's choice.
int32_t pick_heads_per_block(const spa_fwd_args *a) {
  if (a->heads_per_block > 0) return a->heads_per_block;
  const int64_t group = a->num_q_heads / a->num_kv_heads;
  return group > 32 ? 64 : 32;
}

spa::Params make_params(const spa_fwd_args *a, bool decode) {
  spa::Params p{};
  p.q = static_cast<const uint16_t *>(a->q);
  p.k_raw = static_cast<const uint8_t *>(a->k_raw);
  p.v_raw = static_cast<const uint8_t *>(a->v_raw);
  p.k_cmp = static_cast<const uint8_t *>(a->k_cmp);
  p.v_cmp = static_cast<const uint8_t *>(a->v_cmp);
  p.k_cmp_scale = a->k_cmp_scale;
  p.v_cmp_scale = a->v_cmp_scale;
  p.raw_pages = a->raw_pages;
  p.cmp_pages = a->ratio > 0 ? a->cmp_pages : 0;
  p.raw_pt = a->raw_pt;
  p.cmp_pt = a->cmp_pt;
  p.seq_lens = a->seq_lens;
  p.query_seq = a->query_seq;
  p.query_pos = a->query_pos;
  p.cmp_idx = a->cmp_idx;
  p.cmp_cnt = a->cmp_cnt;
  p.sink = a->sink;
  p.o = static_cast<uint16_t *>(a->o);
  p.lse = a->lse;
  p.err_flag = a->err_flag;
  p.raw_pt_stride = a->raw_pt_stride;
  p.cmp_pt_stride = a->ratio > 0 ? a->cmp_pt_stride : 1;
  p.num_seqs = a->num_seqs;
  p.num_queries = a->num_queries;
  p.hq = a->num_q_heads;
  p.hkv = a->num_kv_heads;
  p.head_dim = a->head_dim;
  p.page_size = a->page_size;
  p.window = a->window;
  p.ratio = a->ratio;
  p.topk = a->ratio > 0 ? a->topk : 0;
  p.num_splits = a->num_splits;
  p.group = a->num_q_heads / a->num_kv_heads;
  p.heads_per_block = pick_heads_per_block(a);
  p.head_groups = (p.group + p.heads_per_block - 1) / p.heads_per_block;
  p.jobs_per_unit = p.num_splits * p.head_groups;
  p.unit_begin = 0;
  p.unit_end = 0;   // set per launch
  p.page_shift = -1;
  for (int32_t sh = 0; sh < 31; ++sh)
    if ((int32_t(1) << sh) == a->page_size) p.page_shift = sh;
  p.cmp_fp8 = (a->ratio > 0 && (a->cmp_dtype == SPA_FP8_E4M3_OCP || a->cmp_dtype == SPA_FP8_E4M3_FNUZ)) ? 1 : 0;
  p.cmp_fnuz = (a->ratio > 0 && a->cmp_dtype == SPA_FP8_E4M3_FNUZ) ? 1 : 0;
  p.scale_log2 = a->scale * 1.4426950408889634f;
  return p;
}

// `scratch` (the no-allocation entry point): the split partials go there
// instead of into args->workspace, which is then ignored.
spa_status run_forward(const spa_fwd_args *a, bool decode, void *stream, void *scratch = nullptr) {
  spa_status st = validate(a, decode, true);
  if (st != SPA_OK) return st;
  if (!std::isfinite(a->scale) || !(a->scale > 0.f)) return fail(SPA_ERR_SHAPE, "scale must be finite and > 0");
  spa::Params p = make_params(a, decode);
  const size_t need = workspace_bytes_for(a);
  if (need > 0) {
    void *ws = scratch != nullptr ? scratch : a->workspace;
    if (scratch == nullptr) {
      if (a->workspace == nullptr) return fail(SPA_ERR_WORKSPACE, "num_splits > 1 needs a workspace");
      if (a->workspace_bytes < need)
        return fail(SPA_ERR_WORKSPACE, "workspace of %zu bytes, need %zu", a->workspace_bytes, need);
      if (!aligned16(a->workspace)) return fail(SPA_ERR_ALIGN, "workspace must be 16-byte aligned");
    }
    const WorkspaceLayout w = workspace_layout(a);
    char *base = static_cast<char *>(ws);
    p.part_o = reinterpret_cast<float *>(base + w.part_o);
    p.part_lse = reinterpret_cast<float *>(base + w.part_lse);
  }
  if (a->num_queries == 0) return ok();
  hipStream_t s = static_cast<hipStream_t>(stream);
  // Prefill: query pairs share each KV tile when the call fits that kernel
  // (the library's choice unless the caller asks for 32-head jobs or one
  // query per job); the result does not depend on the choice.
  const bool pairs_ok = !decode && a->head_dim != 512 && spa::prefill_pairs_eligible(p);
  if (a->queries_per_block == 2 && !pairs_ok)
    return fail(SPA_ERR_UNSUPPORTED,
                "queries_per_block 2 needs bf16 caches, head_dim 128, one split, a top-k list or no "
                "compressed part, and 2 * (topk + window) <= %d", spa::kPairRowsMax);
  const bool pairs = pairs_ok && (a->queries_per_block == 2 ||
                                  (a->queries_per_block == 0 && a->heads_per_block != 32));
  // Decode: one workgroup per (query, KV head, 128-head block, slice), when
  // the call fits it and the caller leaves both block sizes to the library.
  const bool dec = decode && a->heads_per_block == 0 && a->queries_per_block == 0 && spa::decode_eligible(p);
  // one slice: the waves of a workgroup split the query's rows (no partials),
  // while its workgroups (one per query, KV head and 32 heads) fit on the
  // chip at once; a larger batch keeps the 128-head workgroups
  const int64_t rows_wgs = (int64_t)a->num_queries * a->num_kv_heads * ((p.group + 31) / 32);
  const bool dec_rows = dec && a->num_splits == 1 && spa::decode_rows_eligible(p) &&
                        rows_wgs <= spa::device_cu_count();
  // the workgroups fit twice over: each takes half of O's dimensions (all
  // of K, half of each V row)
  const bool dec_halves = dec_rows && 2 * rows_wgs <= spa::device_cu_count();
  const bool latent = a->head_dim == 512;
  hipError_t e = latent  ? spa::launch_latent(p, s)
                 : pairs ? spa::launch_prefill_pairs(p, s)
                 : dec_rows ? spa::launch_decode_rows(p, dec_halves, s)
                 : dec   ? spa::launch_decode(p, s)
                         : spa::launch_attention(p, s);
  if (e != hipSuccess) return fail(SPA_ERR_LAUNCH, "attention launch failed: %s", hipGetErrorString(e));
  if (a->num_splits > 1) {
    // the job-stream kernel writes each (query, KV head) unit's partials on
    // one XCD and the merge reads them there; the decode and latent kernels
    // in row order
    e = spa::launch_merge(p.part_o, p.part_lse, a->num_splits, (int64_t)a->num_queries * a->num_q_heads,
                          a->head_dim, a->num_q_heads, a->sink, p.o, a->lse, (dec || latent) ? 0 : p.group, s);
    if (e != hipSuccess) return fail(SPA_ERR_LAUNCH, "merge launch failed: %s", hipGetErrorString(e));
  }
  return ok();
}

// ---- the no-allocation decode entry point: its split partials live in a
// file-scope device array (one per GPU, zero-initialised by the loader, kept
// until the process ends).  In host code `scratch` is a host-side stand-in,
// not a device address: the device address is taken once per device with
// hipGetSymbolAddress (that device current) and used wherever the array's
// memory is needed.
constexpr size_t kScratchBytes = size_t(32) << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<void *> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mutex;

// Device address of the current device's scratch array, or nullptr (with
// the reason recorded) if it cannot be had.
void *scratch_on_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  void *ptr = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (ptr != nullptr) return ptr;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  ptr = g_scratch_ptr[dev].load(std::memory_order_relaxed);
  if (ptr == nullptr) {
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) return nullptr;
    g_scratch_ptr[dev].store(ptr, std::memory_order_release);
  }
  return ptr;
}

}  // namespace

namespace spa {
int32_t device_cu_count() {
  static std::atomic<int32_t> cache[kMaxDevices];
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 0;
  int32_t n = cache[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    n = v;
    cache[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}
}  // namespace spa

extern "C" {

size_t attn_workspace_size(const spa_fwd_args *args) {
  if (args == nullptr || args->num_splits < 1 || args->num_queries < 0 || args->num_q_heads < 1 ||
      args->num_kv_heads < 1)
    return 0;
  if (args->head_dim != 64 && args->head_dim != 128 && args->head_dim != 512) return 0;
  return workspace_bytes_for(args);
}

spa_status attn_fwd_decode(const spa_fwd_args *args, void *stream) { return run_forward(args, true, stream); }

spa_status attn_fwd_prefill(const spa_fwd_args *args, void *stream) { return run_forward(args, false, stream); }

size_t attn_noalloc_scratch_bytes(void) { return kScratchBytes; }

spa_status attn_fwd_decode_noalloc(const spa_fwd_args *args, void *stream) {
  if (args == nullptr) return fail(SPA_ERR_NULL, "args is NULL");
  spa_status st = validate(args, true, true);
  if (st != SPA_OK) return st;
  const size_t need = workspace_bytes_for(args);
  if (need > kScratchBytes)
    return fail(SPA_ERR_WORKSPACE, "the split partials need %zu bytes; the no-allocation scratch holds %zu "
                "(fewer splits or queries per call)", need, kScratchBytes);
  void *ptr = nullptr;
  if (need > 0) {
    ptr = scratch_on_current_device();
    if (ptr == nullptr) return fail(SPA_ERR_LAUNCH, "no device address for the no-allocation scratch on this device");
  }
  return run_forward(args, true, stream, ptr);
}

spa_status attn_merge_lse(const float *o_parts, const float *lse_parts, int32_t num_parts, int64_t rows,
                          int32_t head_dim, int32_t num_q_heads, const float *sink, void *o_out,
                          float *lse_out, void *stream) {
  if (o_parts == nullptr || lse_parts == nullptr || o_out == nullptr)
    return fail(SPA_ERR_NULL, "o_parts, lse_parts and o_out must not be NULL");
  if (num_parts < 1 || num_parts > SPA_MAX_SPLITS)
    return fail(SPA_ERR_SPLITS, "num_parts %d outside [1, %d]", num_parts, SPA_MAX_SPLITS);
  if (rows < 0) return fail(SPA_ERR_SHAPE, "rows must be >= 0");
  if (num_q_heads < 1) return fail(SPA_ERR_SHAPE, "num_q_heads must be >= 1");
  if (head_dim != 64 && head_dim != 128 && head_dim != 512)
    return fail(SPA_ERR_UNSUPPORTED, "head_dim %d not supported (64, 128 or 512)", head_dim);
  if ((rows + 7) / 8 > 0x7FFFFFFFLL) return fail(SPA_ERR_SHAPE, "rows exceed the launch grid");
  if (!aligned16(o_parts)) return fail(SPA_ERR_ALIGN, "o_parts must be 16-byte aligned");
  if ((reinterpret_cast<uintptr_t>(o_out) & 7u) != 0) return fail(SPA_ERR_ALIGN, "o_out must be 8-byte aligned");
  hipError_t e = spa::launch_merge(o_parts, lse_parts, num_parts, rows, head_dim, num_q_heads, sink,
                                   static_cast<uint16_t *>(o_out), lse_out, 0, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(SPA_ERR_LAUNCH, "merge launch failed: %s", hipGetErrorString(e));
  return ok();
}

spa_status attn_build_gather(const spa_fwd_args *args, int32_t decode, int32_t cap, int64_t *rows_out,
                             int32_t *counts_out, void *stream) {
  spa_status st = validate(args, decode != 0, false);
  if (st != SPA_OK) return st;
  if (rows_out == nullptr || counts_out == nullptr) return fail(SPA_ERR_NULL, "rows_out/counts_out is NULL");
  if (cap < 0) return fail(SPA_ERR_SHAPE, "cap must be >= 0");
  if ((int64_t)(cap > 0 ? (cap + 255) / 256 : 1) * args->num_queries > 0x7FFFFFFFLL)
    return fail(SPA_ERR_SHAPE, "cap * num_queries exceeds the launch grid");
  spa::Params p = make_params(args, decode != 0);
  hipError_t e = spa::launch_gather(p, cap, rows_out, counts_out, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(SPA_ERR_LAUNCH, "gather launch failed: %s", hipGetErrorString(e));
  return ok();
}

namespace {
spa_status topk_select(const float *scores, int64_t ld, const int32_t *n_valid, int32_t num_rows, int32_t k,
                       int32_t *ids_out, int32_t *cnt_out, bool by_id, void *stream) {
  static_assert(SPA_MAX_TOPK == spa::kTopkMax, "header and kernel agree on the top-k limit");
  if (scores == nullptr || n_valid == nullptr || ids_out == nullptr || cnt_out == nullptr)
    return fail(SPA_ERR_NULL, "scores, n_valid, ids_out and cnt_out must not be NULL");
  if (num_rows < 0) return fail(SPA_ERR_SHAPE, "num_rows must be >= 0 (got %d)", num_rows);
  if (ld < 1) return fail(SPA_ERR_SHAPE, "ld must be >= 1 (got %lld)", (long long)ld);
  if (k < 1 || k > SPA_MAX_TOPK) return fail(SPA_ERR_UNSUPPORTED, "k %d outside [1, %d]", k, SPA_MAX_TOPK);
  hipError_t e = spa::launch_topk(scores, ld, n_valid, num_rows, k, ids_out, cnt_out, by_id,
                                  static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(SPA_ERR_LAUNCH, "top-k launch failed: %s", hipGetErrorString(e));
  return ok();
}
}  // namespace

spa_status attn_topk_select(const float *scores, int64_t ld, const int32_t *n_valid, int32_t num_rows,
                            int32_t k, int32_t *ids_out, int32_t *cnt_out, void *stream) {
  return topk_select(scores, ld, n_valid, num_rows, k, ids_out, cnt_out, false, stream);
}

spa_status attn_topk_select_ids(const float *scores, int64_t ld, const int32_t *n_valid, int32_t num_rows,
                                int32_t k, int32_t *ids_out, int32_t *cnt_out, void *stream) {
  return topk_select(scores, ld, n_valid, num_rows, k, ids_out, cnt_out, true, stream);
}

size_t attn_bwd_workspace_size(const spa_fwd_args *args) {
  if (args == nullptr || args->num_queries < 0 || args->num_q_heads < 1 || args->num_kv_heads < 1 ||
      args->num_q_heads % args->num_kv_heads != 0 || args->page_size < 1 || args->num_seqs < 0)
    return 0;
  const bool decode = args->query_seq == nullptr && args->query_pos == nullptr;
  const spa::Params p = make_params(args, decode);
  if (spa::backward_kv_eligible(p)) return spa::backward_kv_workspace(p, nullptr, nullptr, nullptr);
  return (size_t)args->num_queries * (size_t)args->num_q_heads * sizeof(float);
}

spa_status attn_bwd(const spa_fwd_args *args, const spa_bwd_grads *grads, void *stream) {
  if (args == nullptr || grads == nullptr) return fail(SPA_ERR_NULL, "args/grads is NULL");
  const bool decode = args->query_seq == nullptr && args->query_pos == nullptr;
  // the forward's split and head-block choices do not apply;
  // queries_per_block picks one query or a query pair per workgroup
  const int32_t qpb = args->queries_per_block;
  spa_fwd_args a = *args;
  a.num_splits = 1;
  a.heads_per_block = 0;
  a.queries_per_block = 0;
  spa_status st = validate(&a, decode, true);
  if (st != SPA_OK) return st;
  if (!std::isfinite(a.scale) || !(a.scale > 0.f)) return fail(SPA_ERR_SHAPE, "scale must be finite and > 0");
  if (a.head_dim != 128) return fail(SPA_ERR_UNSUPPORTED, "the backward takes head_dim 128 (got %d)", a.head_dim);
  if (a.ratio > 0 && a.cmp_dtype != SPA_BF16) return fail(SPA_ERR_UNSUPPORTED, "the backward takes bf16 caches");
  if (a.lse == nullptr) return fail(SPA_ERR_NULL, "lse (the forward's) is NULL");
  if (grads->d_o == nullptr || grads->dq == nullptr || grads->dk_raw == nullptr || grads->dv_raw == nullptr)
    return fail(SPA_ERR_NULL, "d_o, dq, dk_raw and dv_raw must not be NULL");
  if (a.ratio > 0 && (grads->dk_cmp == nullptr || grads->dv_cmp == nullptr))
    return fail(SPA_ERR_NULL, "ratio > 0 needs dk_cmp and dv_cmp");
  if (grads->d_sink != nullptr && a.sink == nullptr) return fail(SPA_ERR_NULL, "d_sink without a sink");
  if (!aligned16(grads->d_o) || !aligned16(grads->dq)) return fail(SPA_ERR_ALIGN, "d_o and dq must be 16-byte aligned");
  if (qpb < 0 || qpb > 2) return fail(SPA_ERR_UNSUPPORTED, "queries_per_block %d not supported (0, 1 or 2)", qpb);
  spa::Params p = make_params(&a, decode);
  const bool pairs_ok = !decode && spa::backward_pairs_eligible(p);
  if (qpb == 2 && !pairs_ok)
    return fail(SPA_ERR_UNSUPPORTED, "queries_per_block 2 needs a prefill call with a top-k list or no compressed part "
                "and 2 * (topk + window) <= %d", spa::kPairRowsMax);
  const bool pairs = pairs_ok && qpb != 1;
  spa::BwdParams b{};
  b.d_o = static_cast<const uint16_t *>(grads->d_o);
  b.o = static_cast<const uint16_t *>(a.o);
  b.lse = a.lse;
  b.dq = grads->dq;
  b.dk_raw = grads->dk_raw;
  b.dv_raw = grads->dv_raw;
  b.dk_cmp = a.ratio > 0 ? grads->dk_cmp : nullptr;
  b.dv_cmp = a.ratio > 0 ? grads->dv_cmp : nullptr;
  b.dsink = grads->d_sink;
  b.scale = a.scale;
  // the KV-block path when the workspace holds its plan, else the fused
  // kernel (float atomics per query or query pair), which needs a
  // workspace only for the sink gradient
  spa::BwdKvPlan plan{};
  const size_t need_kv = spa::backward_kv_eligible(p) ? spa::backward_kv_workspace(p, nullptr, nullptr, nullptr) : 0;
  const bool use_kv = need_kv > 0 && a.workspace != nullptr && a.workspace_bytes >= need_kv;
  const size_t need_sink = (size_t)a.num_queries * (size_t)a.num_q_heads * sizeof(float);
  if (a.workspace != nullptr && (use_kv || grads->d_sink != nullptr) && !aligned16(a.workspace))
    return fail(SPA_ERR_ALIGN, "workspace must be 16-byte aligned");
  if (use_kv) spa::backward_kv_workspace(p, a.workspace, &plan, &b);
  if (grads->d_sink != nullptr) {
    if (need_sink > 0 && (a.workspace == nullptr || a.workspace_bytes < need_sink))
      return fail(SPA_ERR_WORKSPACE, "the sink gradient needs a workspace of %zu bytes", need_sink);
    b.dsink_part = static_cast<float *>(a.workspace);
  }
  if (a.num_queries == 0) return ok();
  if ((int64_t)a.num_queries * a.num_kv_heads * ((a.num_q_heads / a.num_kv_heads + 63) / 64) > 0x7FFFFFFFLL)
    return fail(SPA_ERR_SHAPE, "the job count exceeds the launch grid");
  hipError_t e = spa::launch_backward(p, b, pairs, use_kv ? &plan : nullptr, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(SPA_ERR_LAUNCH, "backward launch failed: %s", hipGetErrorString(e));
  return ok();
}

const char *attn_last_error(void) { return g_last_error.c_str(); }

int32_t attn_abi_version(void) { return 1; }

}  // extern "C"
