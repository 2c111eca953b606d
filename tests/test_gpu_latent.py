"""GPU parity of the 512-wide shared-latent path (K = V, one cache per pool)
with the FP64 oracle, at the forward's tolerance: decode with and without
KV slices (the LSE merge at D 512), prefill positions from 0 up, window-only
and all-groups layers, grouped query heads with a partial head group, and
the full decode_latent workload."""
import numpy as np
import pytest

from sparse_paged_attention_amd import synth

from gpu_helpers import check_against_oracle, need_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()


@pytest.mark.parametrize("splits", [1, 3, 8])
def test_latent_decode_splits(splits):
    p = synth.make_problem("lat_dec", "decode", [700, 1300, 4096, 130, 2], 64, 1, 512, 256, 128, 4, 96, seed=31,
                           shared_kv=True)
    check_against_oracle(p, splits, label=f"latent decode S={splits}")


def test_latent_prefill_ragged_positions():
    pos = [(0, t) for t in (0, 1, 3, 4, 31, 32, 127, 128, 129, 511, 512, 1000)] + [(1, 9), (1, 300)]
    p = synth.make_problem("lat_pre", "prefill", [1001, 301], 64, 1, 512, 256, 128, 4, 64, seed=32,
                           query_positions=pos, selection="score", shared_kv=True)
    check_against_oracle(p, 1, label="latent prefill")


@pytest.mark.parametrize("ratio,topk", [(0, 0), (128, 0)])
def test_latent_window_only_and_all_groups(ratio, topk):
    p = synth.make_problem("lat_layers", "decode", [5000, 900, 128], 64, 1, 512, 256, 128, ratio, topk, seed=33,
                           shared_kv=True)
    check_against_oracle(p, 2, label=f"latent ratio={ratio}")


def test_latent_grouped_heads_partial_group():
    """2 KV heads of 40 query heads: the second head group of each block
    holds 8 real heads."""
    p = synth.make_problem("lat_gqa", "decode", [1500, 2600], 80, 2, 512, 256, 128, 4, 128, seed=34,
                           shared_kv=True, with_sink=True)
    check_against_oracle(p, 4, label="latent gqa")


def test_latent_no_sink_and_empty_lists():
    p = synth.make_problem("lat_nosink", "decode", [3000, 2000], 64, 1, 512, 256, 128, 4, 64, seed=35,
                           shared_kv=True, with_sink=False)
    p.cmp_cnt[1] = 0
    check_against_oracle(p, 4, label="latent no sink, empty list")


def test_latent_full_workload():
    p = synth.make_workload("decode_latent")
    check_against_oracle(p, p.num_splits, label="decode_latent")


@pytest.mark.parametrize("fmt,splits", [("ocp", 1), ("ocp", 4), ("fnuz", 1), ("fnuz", 3)])
def test_latent_e4m3_pages(fmt, splits):
    """e4m3 compressed latent pages (one code row and one fp32 scale per
    token, shared by the key and value roles), OCP and FNUZ, decode with and
    without slices: a slice's compressed entries and window entries run as
    separate chunks of e4m3 and bf16 tiles."""
    p = synth.make_problem("lat_f8", "decode", [700, 1300, 4096, 130, 2, 2100], 64, 1, 512, 256, 128, 4, 200,
                           seed=36, shared_kv=True, cmp_fp8=True, fp8_format=fmt)
    assert p.k_cmp is p.v_cmp and p.k_cmp_scale is p.v_cmp_scale
    check_against_oracle(p, splits, label=f"latent e4m3 {fmt} S={splits}")


def test_latent_e4m3_prefill():
    pos = [(0, t) for t in (0, 3, 4, 127, 128, 600, 1000)] + [(1, 300)]
    p = synth.make_problem("lat_f8_pre", "prefill", [1001, 301], 64, 1, 512, 256, 128, 4, 64, seed=37,
                           query_positions=pos, selection="score", shared_kv=True, cmp_fp8=True)
    check_against_oracle(p, 1, label="latent e4m3 prefill")
