"""GPU parity of the prefill kernel that serves query pairs (two queries of a
sequence streaming the union of their KV sets through shared tiles).

The cases cover both ways a pair's rows are built: the union (same
sequence, touching windows: bitmaps of the selected groups, ranked and
translated through page-table slices in LDS; also an odd last query) and
the concatenation (pairs across sequences, far-apart positions, groups
beyond the bitmaps, a list that names a group twice), plus partial and
multiple head blocks, empty sets, duplicate queries, disjoint lists at the
row capacity, and the device-side checks.  Every case is compared with the FP64 oracle
and, where the one-query-per-job kernel also applies, with it too."""
import numpy as np
import pytest

import oracle
from oracle.compare import accept
from sparse_paged_attention_amd import synth

from gpu_helpers import announce, check_against_oracle, need_gpu, run_hip, torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()


def _prefill(name, seq_lens, positions, hq, hkv, page, window, ratio, topk, seed=41, **kw):
    return synth.make_problem(name, "prefill", seq_lens, hq, hkv, 128, page, window, ratio, topk, seed=seed,
                              query_positions=positions, **kw)


def _both(p, label):
    """The pair kernel and the one-query kernel, each against the oracle."""
    check_against_oracle(p, num_splits=1, queries_per_block=2, label=f"{label} pairs")
    check_against_oracle(p, num_splits=1, queries_per_block=1, label=f"{label} single")


def test_prefill_csa_both_kernels():
    p = synth.make_workload("prefill_csa")
    check_against_oracle(p, num_splits=1, queries_per_block=1, label="prefill_csa single")
    check_against_oracle(p, num_splits=1, queries_per_block=2, label="prefill_csa pairs")


def test_union_every_position():
    """Every position of one sequence, t = 0 upward: sets grow from one row;
    no group is complete at t < 3; top-k truncates once n_c > topk."""
    p = _prefill("every", [400], [(0, t) for t in range(400)], 64, 1, 16, 96, 4, 64, selection="score")
    _both(p, "every position")


def test_union_random_lists_at_capacity():
    """Neighbouring queries with independent random lists from 1024 groups:
    the union holds up to 2 * topk + W + 1 rows (1153 of the 1280 a pair
    can hold)."""
    pos = [(0, t) for t in range(4090, 4096)] + [(1, t) for t in range(5000, 5003)]
    p = _prefill("cap", [4096, 5003], pos, 64, 1, 64, 128, 4, 512)
    _both(p, "random lists at capacity")


def test_concat_pairs_across_sequences():
    """Queries alternate between sequences, so every pair is concatenated."""
    rng = np.random.default_rng(7)
    pos = []
    for k in range(40):
        s = k % 3
        pos.append((s, int(rng.integers(0, [300, 900, 2000][s]))))
    p = _prefill("xseq", [300, 900, 2000], pos, 64, 1, 32, 128, 4, 100)
    _both(p, "pairs across sequences")


def test_concat_far_apart_and_odd_count():
    """Same sequence, windows that do not touch, and an odd query count (the
    last pair has one query)."""
    pos = [(0, 10), (0, 900), (0, 1500), (0, 200), (0, 1999), (0, 1000), (0, 1130)]
    p = _prefill("far", [2000], pos, 64, 1, 16, 128, 4, 200, selection="score")
    _both(p, "far apart / odd")


def test_duplicate_queries():
    pos = [(0, 700), (0, 700), (0, 5), (0, 5), (0, 0)]
    p = _prefill("dup", [800], pos, 64, 1, 16, 64, 4, 50)
    _both(p, "duplicates")


def test_partial_and_multiple_head_blocks():
    """40 query heads per KV head over 2 KV heads (a partial 64-head block),
    and 160 heads per KV head (three blocks, the last partial)."""
    p = _prefill("h40", [600], [(0, t) for t in range(300, 331)], 80, 2, 16, 64, 4, 40, selection="score")
    _both(p, "40 heads x 2 kv")
    p = _prefill("h160", [600], [(0, t) for t in range(500, 517)], 160, 1, 16, 64, 4, 40, selection="score")
    _both(p, "160 heads")


def test_window_only_layer():
    p = _prefill("win", [300, 50], [(0, t) for t in range(0, 300, 7)] + [(1, 49), (1, 48)], 64, 1, 16, 100, 0, 0)
    _both(p, "window only")


def test_empty_sets_in_pairs():
    """W = 0: positions 0-2 have no complete group, so their sets are empty
    (O = 0, LSE = sink); they pair with non-empty neighbours."""
    for with_sink in (True, False):
        pos = [(0, 0), (0, 1), (0, 2), (0, 3), (0, 7), (0, 2)]
        p = _prefill("empty", [8], pos, 64, 1, 4, 0, 4, 2, with_sink=with_sink)
        _both(p, f"empty sets sink={with_sink}")


def test_groups_beyond_the_bitmaps():
    """n_c > 32768 groups: pairs fall back to concatenation."""
    pos = [(0, 131100), (0, 131101), (0, 140000), (0, 140001), (0, 140002)]
    p = _prefill("nc_big", [140003], pos, 64, 1, 256, 32, 4, 40, keep_logical=False)
    announce("n_c > 32768, 5 queries")
    check_against_oracle(p, num_splits=1, queries_per_block=2, label="beyond bitmaps pairs")


def test_corrupt_ids_and_pages_in_pairs():
    """A listed id that is no complete group, and a page id outside the pool:
    masked, never loaded, and flagged; the rest matches the oracle over the
    set without them."""
    p = _prefill("bad", [1000], [(0, t) for t in range(900, 908)], 64, 1, 16, 64, 4, 30)
    p.cmp_idx[2, 4] = 5000             # beyond the complete groups of query 2
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    announce("corrupt id, pairs")
    O, L, _ = run_hip(p, 1, err_flag=flag, queries_per_block=2)
    assert int(flag.item()) & 2
    ids = np.delete(p.cmp_idx[2, :p.cmp_cnt[2]], 4)
    p.cmp_idx[2, :] = -1
    p.cmp_idx[2, :len(ids)] = ids
    p.cmp_cnt[2] = len(ids)
    Oref, Lref = oracle.attention(p)
    rep = accept(O, L, Oref, Lref)
    assert rep.ok, rep

    q = _prefill("badpage", [1000], [(0, t) for t in range(900, 904)], 64, 1, 16, 64, 4, 30)
    q.raw_pt[0, 895 // 16] = 10_000_000   # the page of positions 880..895
    flag.zero_()
    O, L, _ = run_hip(q, 1, err_flag=flag, queries_per_block=2)
    assert int(flag.item()) & 4
    assert np.isfinite(O).all() and np.isfinite(L).all()


def test_pairs_deterministic():
    p = synth.make_workload("prefill_csa")
    announce("prefill_csa pairs twice")
    O1, L1, _ = run_hip(p, 1, queries_per_block=2)
    O2, L2, _ = run_hip(p, 1, queries_per_block=2)
    assert np.array_equal(O1, O2) and np.array_equal(L1, L2)


def test_group_listed_twice_counts_twice():
    """A list that names a group twice (outside the oracle's input contract,
    which takes distinct ids) attends to that row twice in the canonical
    order: the pair leaves the union, whose bitmap would merge the two, for
    the concatenation, and agrees with the one-query kernel."""
    p = _prefill("dup_ids", [1000], [(0, t) for t in range(900, 906)], 64, 1, 16, 64, 4, 30)
    p.cmp_idx[2, 5] = p.cmp_idx[2, 4]
    p.cmp_idx[3, 0] = p.cmp_idx[3, 7]
    announce("group listed twice: pairs vs one query per job")
    O2, L2, _ = run_hip(p, 1, queries_per_block=2)
    O1, L1, _ = run_hip(p, 1, queries_per_block=1)
    rep = accept(O2, L2, O1, L1)
    assert rep.ok, rep
    # and the duplicate matters: without it the result differs
    q = _prefill("dup_ids", [1000], [(0, t) for t in range(900, 906)], 64, 1, 16, 64, 4, 30)
    O0, _, _ = run_hip(q, 1, queries_per_block=2)
    assert not np.allclose(O0[2], O2[2], atol=1e-3)
