// Drives every C-ABI entry point of libspa through its host-side paths
// (argument validation, workspace sizing, kernel selection) for the
// AddressSanitizer / UndefinedBehaviorSanitizer build of the host code.  The
// library objects are host-only (no device code) and the run hides every
// GPU, so no kernel launches: calls that pass validation end in
// SPA_ERR_LAUNCH.  Device pointers are fake, never dereferenced by the host.
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "spa.h"

namespace {

int failures = 0;

void expect(const char *what, int got, int want) {
  if (got != want) {
    std::fprintf(stderr, "%s: status %d, expected %d (%s)\n", what, got, want, attn_last_error());
    ++failures;
  }
}

void *fake(uintptr_t x) { return reinterpret_cast<void *>(x); }

spa_fwd_args good(bool decode) {
  spa_fwd_args a;
  std::memset(&a, 0, sizeof a);
  a.num_seqs = 3;
  a.num_queries = decode ? 3 : 7;
  a.num_q_heads = 128;
  a.num_kv_heads = 1;
  a.head_dim = 128;
  a.page_size = 64;
  a.window = 128;
  a.ratio = 4;
  a.topk = 512;
  a.scale = 0.0883883f;
  a.raw_dtype = SPA_BF16;
  a.cmp_dtype = SPA_BF16;
  a.num_splits = 1;
  a.q = fake(0x100000);
  a.k_raw = fake(0x200000);
  a.v_raw = fake(0x300000);
  a.k_cmp = fake(0x400000);
  a.v_cmp = fake(0x500000);
  a.raw_pages = 1000;
  a.cmp_pages = 100;
  a.raw_pt = static_cast<const int32_t *>(fake(0x600000));
  a.cmp_pt = static_cast<const int32_t *>(fake(0x700000));
  a.raw_pt_stride = 64;
  a.cmp_pt_stride = 16;
  a.seq_lens = static_cast<const int32_t *>(fake(0x800000));
  if (!decode) {
    a.query_seq = static_cast<const int32_t *>(fake(0x810000));
    a.query_pos = static_cast<const int32_t *>(fake(0x820000));
  }
  a.cmp_idx = static_cast<const int32_t *>(fake(0x900000));
  a.cmp_cnt = static_cast<const int32_t *>(fake(0xA00000));
  a.sink = static_cast<const float *>(fake(0xB00000));
  a.o = fake(0xC00000);
  a.lse = static_cast<float *>(fake(0xD00000));
  return a;
}

}  // namespace

int main() {
  // null and malformed argument blocks
  expect("decode NULL", attn_fwd_decode(nullptr, nullptr), SPA_ERR_NULL);
  expect("prefill NULL", attn_fwd_prefill(nullptr, nullptr), SPA_ERR_NULL);
  expect("noalloc NULL", attn_fwd_decode_noalloc(nullptr, nullptr), SPA_ERR_NULL);
  if (attn_workspace_size(nullptr) != 0) ++failures;
  for (int d = 0; d < 2; ++d) {
    const bool decode = d == 0;
    auto call = [&](const spa_fwd_args &a) { return decode ? attn_fwd_decode(&a, nullptr) : attn_fwd_prefill(&a, nullptr); };
    spa_fwd_args a = good(decode);
    a.num_seqs = 0;                  expect("num_seqs 0", call(a), SPA_ERR_SHAPE);
    a = good(decode); a.num_kv_heads = 0;   expect("kv heads 0", call(a), SPA_ERR_SHAPE);
    if (attn_workspace_size(&a) != 0) ++failures;
    a = good(decode); a.num_kv_heads = 2; a.num_q_heads = 129;  expect("heads not multiple", call(a), SPA_ERR_SHAPE);
    a = good(decode); a.head_dim = 96;      expect("head_dim 96", call(a), SPA_ERR_UNSUPPORTED);
    a = good(decode); a.cmp_dtype = 7;      expect("cmp dtype", call(a), SPA_ERR_DTYPE);
    a = good(decode); a.num_splits = 65;    expect("splits 65", call(a), SPA_ERR_SPLITS);
    a = good(decode); a.q = fake(0x100004); expect("q unaligned", call(a), SPA_ERR_ALIGN);
    a = good(decode); a.q = nullptr;        expect("q NULL", call(a), SPA_ERR_NULL);
    a = good(decode); a.scale = -1.f;       expect("scale", call(a), SPA_ERR_SHAPE);
    a = good(decode); a.num_splits = 4;     expect("no workspace", call(a), SPA_ERR_WORKSPACE);
    a.workspace = fake(0xE00000);
    a.workspace_bytes = attn_workspace_size(&a) - 1;
    expect("short workspace", call(a), SPA_ERR_WORKSPACE);
    // well-formed calls: validation passes, the launch finds no device
    for (int s : {1, 3, 4, 64}) {
      for (int fp8 : {0, 1, 2}) {
        for (int hpb : {0, 32, 64}) {
          a = good(decode);
          a.num_splits = s;
          a.cmp_dtype = fp8;
          a.heads_per_block = hpb;
          if (fp8) {
            a.k_cmp_scale = static_cast<const float *>(fake(0xF00000));
            a.v_cmp_scale = static_cast<const float *>(fake(0xF10000));
          }
          a.workspace = fake(0x1000000);
          a.workspace_bytes = attn_workspace_size(&a);
          const int st = call(a);
          if (st != SPA_ERR_LAUNCH && st != SPA_ERR_UNSUPPORTED) {
            std::fprintf(stderr, "valid call s=%d fp8=%d hpb=%d: status %d (%s)\n", s, fp8, hpb, st, attn_last_error());
            ++failures;
          }
          if (decode && hpb == 0) attn_fwd_decode_noalloc(&a, nullptr);
        }
      }
    }
    a = good(decode);
    a.head_dim = 512;
    a.v_raw = a.k_raw;
    a.v_cmp = a.k_cmp;
    a.num_q_heads = 64;
    expect("latent", call(a), SPA_ERR_LAUNCH);
    a = good(decode);
    if (!decode) {
      a.queries_per_block = 2;
      expect("pairs", call(a), SPA_ERR_LAUNCH);
    }
    int64_t rows[1];
    int32_t counts[4];
    a = good(decode);
    expect("gather", attn_build_gather(&a, decode, 700, rows, counts, nullptr), SPA_ERR_LAUNCH);
    expect("gather NULL", attn_build_gather(&a, decode, 700, nullptr, counts, nullptr), SPA_ERR_NULL);
    // backward
    spa_bwd_grads g;
    std::memset(&g, 0, sizeof g);
    expect("bwd NULL grads", attn_bwd(&a, nullptr, nullptr), SPA_ERR_NULL);
    g.d_o = fake(0x2000000);
    g.dq = static_cast<float *>(fake(0x2100000));
    g.dk_raw = static_cast<float *>(fake(0x2200000));
    g.dv_raw = static_cast<float *>(fake(0x2300000));
    g.dk_cmp = static_cast<float *>(fake(0x2400000));
    g.dv_cmp = static_cast<float *>(fake(0x2500000));
    g.d_sink = static_cast<float *>(fake(0x2600000));
    expect("bwd no workspace", attn_bwd(&a, &g, nullptr), SPA_ERR_WORKSPACE);
    a.workspace = fake(0x3000000);
    a.workspace_bytes = attn_bwd_workspace_size(&a);
    expect("bwd", attn_bwd(&a, &g, nullptr), SPA_ERR_LAUNCH);
  }
  // merge and top-k
  expect("merge NULL", attn_merge_lse(nullptr, nullptr, 4, 100, 128, 128, nullptr, nullptr, nullptr, nullptr),
         SPA_ERR_NULL);
  expect("merge", attn_merge_lse(static_cast<const float *>(fake(0x100000)), static_cast<const float *>(fake(0x200000)),
                                 4, 100, 128, 128, nullptr, fake(0x300000), nullptr, nullptr),
         SPA_ERR_LAUNCH);
  expect("merge parts", attn_merge_lse(static_cast<const float *>(fake(0x100000)),
                                       static_cast<const float *>(fake(0x200000)), 65, 100, 128, 128, nullptr,
                                       fake(0x300000), nullptr, nullptr),
         SPA_ERR_SPLITS);
  expect("topk k", attn_topk_select(static_cast<const float *>(fake(0x100000)), 1024,
                                    static_cast<const int32_t *>(fake(0x200000)), 32, 4096,
                                    static_cast<int32_t *>(fake(0x300000)), static_cast<int32_t *>(fake(0x400000)),
                                    nullptr),
         SPA_ERR_UNSUPPORTED);
  expect("topk", attn_topk_select(static_cast<const float *>(fake(0x100000)), 1024,
                                  static_cast<const int32_t *>(fake(0x200000)), 32, 512,
                                  static_cast<int32_t *>(fake(0x300000)), static_cast<int32_t *>(fake(0x400000)),
                                  nullptr),
         SPA_ERR_LAUNCH);
  expect("topk ids", attn_topk_select_ids(static_cast<const float *>(fake(0x100000)), 1024,
                                          static_cast<const int32_t *>(fake(0x200000)), 32, 512,
                                          static_cast<int32_t *>(fake(0x300000)),
                                          static_cast<int32_t *>(fake(0x400000)), nullptr),
         SPA_ERR_LAUNCH);
  if (attn_abi_version() != 1) ++failures;
  std::printf("host paths driven; %d unexpected statuses\n", failures);
  return failures == 0 ? 0 : 1;
}
