"""GPU parity of the persistent job streams: each workgroup runs a list of
jobs as one stream of Q and KV tiles, with the rows translated ahead of the
loads.  These cases vary what the stream has to carry: many jobs per
workgroup, jobs of very different lengths, empty and fully masked jobs,
split slices, partial head blocks, both head-block sizes, page sizes that
are not powers of two, and more jobs than one launch takes."""
import numpy as np
import pytest

from sparse_paged_attention_amd import synth

from gpu_helpers import announce, check_against_oracle, need_gpu, run_hip
import oracle
from oracle.compare import accept

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()


def _prefill(name, seq_lens, positions, hq, hkv, d, page, window, ratio, topk, **kw):
    return synth.make_problem(name, "prefill", seq_lens, hq, hkv, d, page, window, ratio, topk, seed=31,
                              query_positions=positions, **kw)


@pytest.mark.parametrize("hpb", [32, 64])
def test_prefill_csa_head_blocks(hpb):
    check_against_oracle(synth.make_workload("prefill_csa"), num_splits=1, heads_per_block=hpb,
                         label=f"prefill hpb{hpb}")


def test_prefill_fp8_stream():
    p = _prefill("fp8p", [1500], [(0, t) for t in range(1000, 1037)], 64, 1, 128, 64, 128, 4, 200,
                 cmp_fp8=True, selection="score")
    check_against_oracle(p, label="fp8 prefill")


def test_prefill_all_groups_layer():
    p = _prefill("hca", [3000], [(0, t) for t in list(range(120, 140)) + list(range(2990, 3000))],
                 16, 1, 64, 128, 128, 128, 0)
    check_against_oracle(p, label="hca prefill")


def test_prefill_window_only_layer():
    p = _prefill("dense", [300], [(0, t) for t in range(0, 300, 3)], 32, 2, 128, 16, 64, 0, 0)
    check_against_oracle(p, label="dense prefill")


def test_prefill_ragged_order():
    """Queries of several sequences in no particular order, including the
    first token of a sequence (one-row set) and jumps across windows."""
    pos = [(0, 5), (1, 70), (0, 6), (2, 900), (2, 100), (2, 101), (2, 102), (1, 0), (0, 63)]
    p = _prefill("ragged", [64, 71, 1024], pos, 64, 1, 128, 16, 48, 4, 30)
    check_against_oracle(p, label="ragged prefill")


def test_prefill_long_context():
    p = _prefill("long", [20000], [(0, t) for t in range(19990, 20000)], 16, 1, 64, 64, 32, 4, 64)
    check_against_oracle(p, label="long prefill")


@pytest.mark.parametrize("page", [24, 7])
def test_page_size_not_power_of_two(page):
    p = synth.make_problem("pg", "decode", [333, 1000, 64, 517], 8, 1, 64, page, 40, 4, 48, seed=32)
    check_against_oracle(p, num_splits=1, label=f"page {page}")
    check_against_oracle(p, num_splits=3, label=f"page {page} split")


def test_partial_head_block():
    """40 query heads per KV head: the second 32-head wave of a 64-head job
    has 8 real heads; the rest read zero Q rows and write nothing."""
    p = synth.make_problem("h40", "decode", [700, 129], 80, 2, 128, 64, 128, 4, 64, seed=33)
    check_against_oracle(p, num_splits=1, heads_per_block=64, label="40 heads / hpb 64")
    check_against_oracle(p, num_splits=2, heads_per_block=32, label="40 heads / hpb 32 / 2 splits")


def test_many_jobs_per_workgroup_with_splits():
    """More jobs than resident workgroups, each a split slice."""
    p = synth.make_workload("decode_csa", batch=600)
    announce("decode_csa batch 600, 2 splits, sampled")
    O, L, _ = run_hip(p, 2)
    qs = list(range(0, 600, 37)) + [599]
    Oref, Lref = oracle.attention(p, qs)
    rep = accept(O[qs], L[qs], Oref, Lref)
    assert rep.ok, rep


def test_more_jobs_than_one_launch():
    """80,000 jobs (20,000 tiny decode queries x 4 splits) exceed what one
    launch gives its workgroups; the library splits the launch by units.
    Sampled queries against the oracle, all checked finite."""
    rng = np.random.default_rng(5)
    lens = rng.integers(1, 80, size=20000)
    p = synth.make_problem("many", "decode", lens, 4, 1, 64, 16, 16, 4, 8, seed=34, spare_pages=0,
                           keep_logical=False)
    announce("20000 decode queries x 4 splits, sampled")
    O, L, _ = run_hip(p, 4)
    assert np.isfinite(O).all() and np.isfinite(L).all()
    qs = sorted(set(list(range(0, 20000, 997)) + [19999, 1, 2]))
    Oref, Lref = oracle.attention(p, qs)
    rep = accept(O[qs], L[qs], Oref, Lref)
    assert rep.ok, rep
