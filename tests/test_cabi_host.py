"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, the ctypes mirror of spa_fwd_args matches the C layout, and
host-side validation returns the documented status for each fault class
(validation runs before any HIP call)."""
import ctypes
import os
import re
import subprocess

import pytest

from sparse_paged_attention_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "spa.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.fail("libspa.so is not built (run __graft_entry__.build())")
    return _lib.load()


def _declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(attn_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol(lib):
    declared = _declared_functions()
    assert set(declared) == set(_lib.SYMBOLS)
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(line.split()[-1] for line in out.splitlines() if line.strip())
    for name in declared:
        assert name in exported, name
        assert hasattr(lib, name)


def test_struct_layout_matches_header(tmp_path):
    fields = [f[0] for f in _lib.SpaFwdArgs._fields_]
    src = tmp_path / "layout.c"
    body = "\n".join(f'  printf("{f} %zu\\n", offsetof(spa_fwd_args, {f}));' for f in fields)
    src.write_text('#include <stdio.h>\n#include <stddef.h>\n#include "spa.h"\nint main(void){\n'
                   + body + '\n  printf("SIZE %zu\\n", sizeof(spa_fwd_args));\n  return 0;\n}\n')
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c99", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split("\n")
    got = dict(line.split() for line in out if line)
    for f in fields:
        assert int(got[f]) == getattr(_lib.SpaFwdArgs, f).offset, f
    assert int(got["SIZE"]) == ctypes.sizeof(_lib.SpaFwdArgs)


def _good_args():
    """A well-formed decode argument block with fake (never dereferenced)
    16-byte aligned device addresses."""
    a = _lib.SpaFwdArgs()
    a.num_seqs = 2
    a.num_queries = 2
    a.num_q_heads = 8
    a.num_kv_heads = 1
    a.head_dim = 128
    a.page_size = 16
    a.window = 16
    a.ratio = 4
    a.topk = 8
    a.scale = 0.125
    a.raw_dtype = _lib.SPA_BF16
    a.cmp_dtype = _lib.SPA_BF16
    a.num_splits = 1
    base = 0x10000000
    for i, f in enumerate(["q", "k_raw", "v_raw", "k_cmp", "v_cmp", "raw_pt", "cmp_pt", "seq_lens",
                           "cmp_idx", "cmp_cnt", "sink", "o", "lse"]):
        setattr(a, f, base + 0x1000 * i)
    a.raw_pages = 4
    a.cmp_pages = 4
    a.raw_pt_stride = 2
    a.cmp_pt_stride = 2
    return a


FAULTS = [
    ("null_q", lambda a: setattr(a, "q", None), -1),
    ("null_raw_pt", lambda a: setattr(a, "raw_pt", None), -1),
    ("null_cmp_when_ratio", lambda a: setattr(a, "k_cmp", None), -1),
    ("null_list_when_topk", lambda a: setattr(a, "cmp_idx", None), -1),
    ("null_out", lambda a: setattr(a, "o", None), -1),
    ("fp8_without_scales", lambda a: setattr(a, "cmp_dtype", _lib.SPA_FP8_E4M3_OCP), -1),
    ("zero_seqs", lambda a: setattr(a, "num_seqs", 0), -2),
    ("heads_not_multiple", lambda a: setattr(a, "num_kv_heads", 3), -2),
    ("page_size_zero", lambda a: setattr(a, "page_size", 0), -2),
    ("negative_window", lambda a: setattr(a, "window", -1), -2),
    ("topk_without_ratio", lambda a: setattr(a, "ratio", 0), -2),
    ("raw_pages_zero", lambda a: setattr(a, "raw_pages", 0), -2),
    ("raw_dtype_fp8", lambda a: setattr(a, "raw_dtype", _lib.SPA_FP8_E4M3_OCP), -3),
    ("cmp_dtype_unknown", lambda a: setattr(a, "cmp_dtype", 7), -3),
    ("head_dim_96", lambda a: setattr(a, "head_dim", 96), -4),
    ("misaligned_q", lambda a: setattr(a, "q", a.q + 2), -5),
    ("misaligned_out", lambda a: setattr(a, "o", a.o + 8), -5),
    ("scale_zero", lambda a: setattr(a, "scale", 0.0), -2),
    ("heads_per_block_48", lambda a: setattr(a, "heads_per_block", 48), -4),
    ("queries_per_block_3", lambda a: setattr(a, "queries_per_block", 3), -4),
    ("queries_per_block_2", lambda a: setattr(a, "queries_per_block", 2), -4),
    ("heads_per_block_128", lambda a: (setattr(a, "num_q_heads", 128), setattr(a, "heads_per_block", 128)), -4),
    ("d512_separate_kv", lambda a: setattr(a, "head_dim", 512), -4),
    ("fnuz_without_scales", lambda a: setattr(a, "cmp_dtype", _lib.SPA_FP8_E4M3_FNUZ), -1),
    ("d512_fp8", lambda a: (setattr(a, "head_dim", 512), setattr(a, "v_raw", a.k_raw), setattr(a, "v_cmp", a.k_cmp),
                            setattr(a, "cmp_dtype", _lib.SPA_FP8_E4M3_OCP), setattr(a, "k_cmp_scale", 0x30000000),
                            setattr(a, "v_cmp_scale", 0x30001000)), -4),
    ("d512_heads_per_block", lambda a: (setattr(a, "head_dim", 512), setattr(a, "v_raw", a.k_raw),
                                        setattr(a, "v_cmp", a.k_cmp), setattr(a, "heads_per_block", 64)), -4),
    ("splits_zero", lambda a: setattr(a, "num_splits", 0), -7),
    ("splits_too_many", lambda a: setattr(a, "num_splits", 65), -7),
    ("decode_with_positions", lambda a: setattr(a, "query_pos", 0x20000000), -9),
    ("decode_count_mismatch", lambda a: setattr(a, "num_queries", 3), -9),
]


@pytest.mark.parametrize("name,mutate,code", FAULTS, ids=[f[0] for f in FAULTS])
def test_decode_validation(lib, name, mutate, code):
    a = _good_args()
    mutate(a)
    st = lib.attn_fwd_decode(ctypes.byref(a), None)
    assert st == code, (name, st, lib.attn_last_error())
    assert lib.attn_last_error().decode()


def test_null_args(lib):
    assert lib.attn_fwd_decode(None, None) == -1
    assert lib.attn_fwd_prefill(None, None) == -1
    assert lib.attn_workspace_size(None) == 0


def test_prefill_needs_positions(lib):
    a = _good_args()
    assert lib.attn_fwd_prefill(ctypes.byref(a), None) == -9


PAIR_FAULTS = [
    ("fp8_cache", lambda a: (setattr(a, "cmp_dtype", _lib.SPA_FP8_E4M3_OCP), setattr(a, "k_cmp_scale", 0x30000000),
                             setattr(a, "v_cmp_scale", 0x30001000))),
    ("head_dim_64", lambda a: setattr(a, "head_dim", 64)),
    ("rows_beyond_capacity", lambda a: setattr(a, "topk", 700)),
    ("all_groups_layer", lambda a: setattr(a, "topk", 0)),
]


@pytest.mark.parametrize("name,mutate", PAIR_FAULTS, ids=[f[0] for f in PAIR_FAULTS])
def test_prefill_pairs_rejected_when_ineligible(lib, name, mutate):
    """queries_per_block 2 asks for the pair kernel: a call it cannot serve
    is refused before any HIP call."""
    a = _good_args()
    a.query_seq = 0x20000000
    a.query_pos = 0x20001000
    a.queries_per_block = 2
    mutate(a)
    st = lib.attn_fwd_prefill(ctypes.byref(a), None)
    assert st == -4, (name, st, lib.attn_last_error())
    assert b"queries_per_block 2" in lib.attn_last_error()


def test_workspace_rules(lib):
    a = _good_args()
    a.num_splits = 4
    need = lib.attn_workspace_size(ctypes.byref(a))
    rows = a.num_queries * a.num_q_heads
    assert need >= rows * 128 * 4 * 4 + rows * 4 * 4
    assert lib.attn_fwd_decode(ctypes.byref(a), None) == -6       # missing
    a.workspace = 0x30000000
    a.workspace_bytes = need - 1
    assert lib.attn_fwd_decode(ctypes.byref(a), None) == -6       # too small
    a.num_splits = 1
    assert lib.attn_workspace_size(ctypes.byref(a)) == 0


def test_merge_validation(lib):
    good = dict(o=0x10000000, l=0x10010000, out=0x10020000)
    assert lib.attn_merge_lse(None, good["l"], 2, 10, 128, 4, None, good["out"], None, None) == -1
    assert lib.attn_merge_lse(good["o"], good["l"], 0, 10, 128, 4, None, good["out"], None, None) == -7
    assert lib.attn_merge_lse(good["o"], good["l"], 65, 10, 128, 4, None, good["out"], None, None) == -7
    assert lib.attn_merge_lse(good["o"], good["l"], 2, -1, 128, 4, None, good["out"], None, None) == -2
    assert lib.attn_merge_lse(good["o"], good["l"], 2, 10, 96, 4, None, good["out"], None, None) == -4
    # o_parts is read 16 bytes per lane, o_out written 8 bytes per lane
    assert lib.attn_merge_lse(good["o"] + 8, good["l"], 2, 10, 128, 4, None, good["out"], None, None) == -5
    assert lib.attn_merge_lse(good["o"], good["l"], 2, 10, 128, 4, None, good["out"] + 4, None, None) == -5


def test_gather_validation(lib):
    a = _good_args()
    assert lib.attn_build_gather(ctypes.byref(a), 1, 16, None, 0x10000000, None) == -1
    assert lib.attn_build_gather(ctypes.byref(a), 1, -1, 0x10000000, 0x10000000, None) == -2
    a.head_dim = 32
    assert lib.attn_build_gather(ctypes.byref(a), 1, 16, 0x10000000, 0x10000000, None) == -4


@pytest.mark.parametrize("name", ["attn_topk_select", "attn_topk_select_ids"])
def test_topk_validation(lib, name):
    """attn_topk_select and attn_topk_select_ids refuse bad arguments before
    any HIP call."""
    P = 0x10000000
    fn = getattr(lib, name)
    assert fn(None, 8, P, 1, 4, P, P, None) == -1
    assert fn(P, 8, P, 1, 4, None, P, None) == -1
    assert fn(P, 8, P, -1, 4, P, P, None) == -2
    assert fn(P, 0, P, 1, 4, P, P, None) == -2
    assert fn(P, 8, P, 1, 0, P, P, None) == -4
    assert fn(P, 8, P, 1, _lib.SPA_MAX_TOPK + 1, P, P, None) == -4
    assert b"k " in lib.attn_last_error()


def test_bwd_grads_layout_matches_header(tmp_path):
    fields = [f[0] for f in _lib.SpaBwdGrads._fields_]
    src = tmp_path / "bwd_layout.c"
    body = "\n".join(f'  printf("{f} %zu\\n", offsetof(spa_bwd_grads, {f}));' for f in fields)
    src.write_text('#include <stdio.h>\n#include <stddef.h>\n#include "spa.h"\nint main(void){\n'
                   + body + '\n  printf("SIZE %zu\\n", sizeof(spa_bwd_grads));\n  return 0;\n}\n')
    exe = tmp_path / "bwd_layout"
    subprocess.run(["gcc", "-std=c99", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split("\n")
    got = dict(line.split() for line in out if line)
    for f in fields:
        assert int(got[f]) == getattr(_lib.SpaBwdGrads, f).offset, f
    assert int(got["SIZE"]) == ctypes.sizeof(_lib.SpaBwdGrads)


def _good_grads():
    g = _lib.SpaBwdGrads()
    for i, f in enumerate(["d_o", "dq", "dk_raw", "dv_raw", "dk_cmp", "dv_cmp", "d_sink"]):
        setattr(g, f, 0x40000000 + 0x1000 * i)
    return g


BWD_FAULTS = [
    ("null_grads", None, None, -1),
    ("null_dq", None, lambda g: setattr(g, "dq", None), -1),
    ("null_dk_cmp_with_ratio", None, lambda g: setattr(g, "dk_cmp", None), -1),
    ("null_lse", lambda a: setattr(a, "lse", None), None, -1),
    ("null_o", lambda a: setattr(a, "o", None), None, -1),
    ("d_sink_without_sink", lambda a: setattr(a, "sink", None), None, -1),
    ("head_dim_64", lambda a: setattr(a, "head_dim", 64), None, -4),
    ("fp8_cache", lambda a: (setattr(a, "cmp_dtype", _lib.SPA_FP8_E4M3_OCP), setattr(a, "k_cmp_scale", 0x30000000),
                             setattr(a, "v_cmp_scale", 0x30001000)), None, -4),
    ("misaligned_d_o", None, lambda g: setattr(g, "d_o", g.d_o + 2), -5),
    ("no_workspace_for_dsink", None, None, -6),
    ("scale_negative", lambda a: setattr(a, "scale", -1.0), None, -2),
    ("positions_half_given", lambda a: setattr(a, "query_pos", 0x20000000), None, -9),
]


@pytest.mark.parametrize("name,mut_a,mut_g,code", BWD_FAULTS, ids=[f[0] for f in BWD_FAULTS])
def test_backward_validation(lib, name, mut_a, mut_g, code):
    """attn_bwd refuses bad arguments before any HIP call."""
    a = _good_args()
    g = _good_grads()
    if name != "no_workspace_for_dsink":
        a.workspace = 0x50000000
        a.workspace_bytes = lib.attn_bwd_workspace_size(ctypes.byref(a))
    if mut_a:
        mut_a(a)
    if mut_g:
        mut_g(g)
    st = lib.attn_bwd(ctypes.byref(a), None if name == "null_grads" else ctypes.byref(g), None)
    assert st == code, (name, st, lib.attn_last_error())
    assert lib.attn_last_error().decode()
    assert lib.attn_bwd_workspace_size(None) == 0


def test_noalloc_refuses_oversize_before_any_hip_call(lib):
    """The no-allocation decode entry point checks the size of its split
    partials against its fixed scratch array before touching the GPU."""
    assert lib.attn_noalloc_scratch_bytes() == 32 << 20
    a = _good_args()
    a.num_splits = 64
    a.num_q_heads = a.num_kv_heads * 4096
    a.workspace = None
    a.workspace_bytes = 0
    assert lib.attn_fwd_decode_noalloc(ctypes.byref(a), None) == -6
    assert b"no-allocation scratch" in lib.attn_last_error()
    assert lib.attn_fwd_decode_noalloc(None, None) == -1
