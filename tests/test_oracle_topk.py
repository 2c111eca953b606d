"""Pins of the top-k oracle (oracle/topk.py), independent of its numpy
ordering: a brute force over Python float comparisons, the closed cases,
and the invariants a top-k selection must satisfy."""
import math

import numpy as np
import pytest

from oracle.topk import order_key, topk_select


def _rank(x: float):
    """Sort key of one score for a descending order: NaN last, then by
    value, -0.0 after +0.0 (Python floats, no bit tricks)."""
    if math.isnan(x):
        return (1, 0.0, 0)
    return (0, -x, 0 if math.copysign(1.0, x) > 0 else 1)


def _brute(row, n, k):
    vals = [float(v) for v in row[:n]]
    order = sorted(range(n), key=lambda j: (_rank(vals[j]), j))
    return order[:min(k, n)]


def _special_row(rng, n):
    """Scores with ties, signed zeros, infinities, NaN and subnormals."""
    pool = np.array([0.0, -0.0, 1.0, -1.0, np.inf, -np.inf, np.nan, 1e-40, -1e-40, 3.5, 3.5, -2.25],
                    dtype=np.float32)
    row = rng.standard_normal(n).astype(np.float32)
    pick = rng.random(n) < 0.4
    row[pick] = rng.choice(pool, size=int(pick.sum()))
    return row


@pytest.mark.parametrize("seed", range(6))
def test_topk_matches_brute_force(seed):
    rng = np.random.default_rng(seed)
    rows, ld = 9, 60
    scores = np.stack([_special_row(rng, ld) for _ in range(rows)])
    n_valid = rng.integers(-2, ld + 5, size=rows)
    for k in (1, 7, 30, 64):
        ids, cnt = topk_select(scores, n_valid, k)
        for i in range(rows):
            n = min(max(int(n_valid[i]), 0), ld)
            want = _brute(scores[i], n, k)
            assert cnt[i] == len(want)
            assert list(ids[i, :cnt[i]]) == want, (seed, k, i)
            assert np.all(ids[i, cnt[i]:] == -1)


@pytest.mark.parametrize("seed", range(3))
def test_topk_by_id_matches_brute_force(seed):
    """The id-ordered list is the brute-force selection sorted by id."""
    rng = np.random.default_rng(100 + seed)
    rows, ld = 7, 50
    scores = np.stack([_special_row(rng, ld) for _ in range(rows)])
    n_valid = rng.integers(-2, ld + 5, size=rows)
    for k in (1, 9, 25, 64):
        ids, cnt = topk_select(scores, n_valid, k, by_id=True)
        for i in range(rows):
            n = min(max(int(n_valid[i]), 0), ld)
            want = sorted(_brute(scores[i], n, k))
            assert cnt[i] == len(want)
            assert list(ids[i, :cnt[i]]) == want, (seed, k, i)
            assert np.all(ids[i, cnt[i]:] == -1)


def test_order_key_is_monotone():
    vals = np.array([-np.inf, -3e38, -1.0, -1e-40, -0.0, 0.0, 1e-40, 1.0, 2.0, 3e38, np.inf], dtype=np.float32)
    keys = order_key(vals)
    assert np.all(np.diff(keys.astype(np.int64)) > 0)
    assert order_key(np.array([np.nan], dtype=np.float32))[0] < keys.min()


def test_all_selected_when_k_covers_the_row():
    rng = np.random.default_rng(1)
    scores = rng.standard_normal((3, 20)).astype(np.float32)
    ids, cnt = topk_select(scores, np.array([20, 5, 0]), 64)
    assert list(cnt) == [20, 5, 0]
    assert sorted(ids[0, :20]) == list(range(20))
    assert list(ids[0, :20]) == list(np.argsort(-scores[0], kind="stable"))
    assert sorted(ids[1, :5]) == list(range(5))
    assert np.all(ids[2] == -1)


def test_selection_invariants():
    """Every selected score ranks at or above every unselected one, ids are
    distinct and valid, and a tie at the cut keeps the lower ids."""
    rng = np.random.default_rng(7)
    scores = rng.integers(0, 6, size=(5, 200)).astype(np.float32)   # many ties
    n_valid = np.array([200, 150, 7, 199, 64])
    ids, cnt = topk_select(scores, n_valid, 50)
    for i in range(5):
        n = n_valid[i]
        sel = ids[i, :cnt[i]]
        assert len(set(sel.tolist())) == len(sel) and sel.min() >= 0 and sel.max() < n
        rest = np.setdiff1d(np.arange(n), sel)
        if len(rest):
            assert scores[i, sel].min() >= scores[i, rest].max()
            cut = scores[i, sel].min()
            tied_out = rest[scores[i, rest] == cut]
            tied_in = sel[scores[i, sel] == cut]
            if len(tied_out):
                assert tied_in.max() < tied_out.min()
