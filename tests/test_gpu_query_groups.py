"""GPU parity of the query-group path: a workgroup serves several consecutive
queries, streaming the union of their KV sets once (or one pass per query
when they do not share a sequence / window span / LDS-sized id range)."""
import numpy as np
import pytest

from sparse_paged_attention_amd import synth

from gpu_helpers import check_against_oracle, need_gpu, run_hip

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()


@pytest.mark.parametrize("qpb,hpb", [(1, 64), (2, 64), (4, 32), (2, 32), (1, 128)])
def test_prefill_csa_groups(qpb, hpb):
    check_against_oracle(synth.make_workload("prefill_csa"), num_splits=1, heads_per_block=hpb,
                         queries_per_block=qpb, label=f"prefill qpb{qpb} hpb{hpb}")


@pytest.mark.parametrize("qpb", [2, 4])
def test_tiny_groups(qpb):
    check_against_oracle(synth.make_workload("tiny"), queries_per_block=qpb, label=f"tiny qpb{qpb}")


def _prefill(name, seq_lens, positions, hq, hkv, d, page, window, ratio, topk, **kw):
    return synth.make_problem(name, "prefill", seq_lens, hq, hkv, d, page, window, ratio, topk, seed=31,
                              query_positions=positions, **kw)


@pytest.mark.parametrize("qpb", [2, 4])
def test_groups_fp8_union(qpb):
    p = _prefill("fp8u", [1500], [(0, t) for t in range(1000, 1037)], 64, 1, 128, 64, 128, 4, 200,
                 cmp_fp8=True, selection="score")
    check_against_oracle(p, queries_per_block=qpb, label=f"fp8 union qpb{qpb}")


def test_groups_all_groups_layer():
    p = _prefill("hca", [3000], [(0, t) for t in list(range(120, 140)) + list(range(2990, 3000))],
                 16, 1, 64, 128, 128, 128, 0)
    check_against_oracle(p, queries_per_block=4, label="hca groups")


def test_groups_window_only_layer():
    p = _prefill("dense", [300], [(0, t) for t in range(0, 300, 3)], 32, 2, 128, 16, 64, 0, 0)
    check_against_oracle(p, queries_per_block=4, label="dense groups")


def test_groups_ragged_fall_back_to_passes():
    """Groups that span sequences, jump beyond a window, or end early."""
    pos = [(0, 5), (1, 70), (0, 6), (2, 900), (2, 100), (2, 101), (2, 102), (1, 0), (0, 63)]
    p = _prefill("ragged", [64, 71, 1024], pos, 64, 1, 128, 16, 48, 4, 30)
    check_against_oracle(p, queries_per_block=4, label="ragged groups")
    check_against_oracle(p, queries_per_block=2, label="ragged groups 2")


def test_groups_union_beyond_lds_cap():
    """More compressed groups than the LDS union holds: per-query passes."""
    p = _prefill("long", [20000], [(0, t) for t in range(19990, 20000)], 16, 1, 64, 64, 32, 4, 64)
    check_against_oracle(p, queries_per_block=4, label="beyond cap")


def test_groups_match_single_query_path():
    p = synth.make_workload("prefill_csa")
    O1, L1, _ = run_hip(p, 1, queries_per_block=1)
    O4, L4, _ = run_hip(p, 1, queries_per_block=4)
    assert np.max(np.abs(O1 - O4)) < 2e-2 and np.max(np.abs(L1 - L4)) < 1e-3
