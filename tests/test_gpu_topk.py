"""GPU parity of the top-k selection (attn_topk_select, by score, and
attn_topk_select_ids, by id) with the oracle (oracle/topk.py): bit-exact ids
and counts.  Rows cover ties, signed zeros,
infinities, NaN and subnormals, counts below, at and above k and past the
row length, k from 1 to its maximum, and rows of 200,000 scores.  The last
test composes the path the pages describe: scores -> top-k -> attention."""
import numpy as np
import pytest

import oracle
from oracle.compare import accept
from oracle.topk import topk_select as oracle_topk
from sparse_paged_attention_amd import synth

from gpu_helpers import announce, need_gpu, run_hip, torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()


def _gpu_topk(scores, n_valid, k, by_id=False):
    from sparse_paged_attention_amd import api
    s = torch.from_numpy(np.ascontiguousarray(scores, dtype=np.float32)).cuda()
    ids, cnt = api.topk_select(s, torch.from_numpy(np.asarray(n_valid, dtype=np.int32)), k, by_id=by_id)
    torch.cuda.synchronize()
    return ids.cpu().numpy(), cnt.cpu().numpy()


def _check(scores, n_valid, k, label):
    """Both entry points: by score (attn_topk_select) and by id
    (attn_topk_select_ids)."""
    for by_id in (False, True):
        announce(f"topk {label}: rows={scores.shape[0]} ld={scores.shape[1]} k={k} by_id={by_id}")
        ids, cnt = _gpu_topk(scores, n_valid, k, by_id)
        rid, rcnt = oracle_topk(scores, n_valid, k, by_id=by_id)
        assert np.array_equal(cnt, rcnt), label
        bad = np.argwhere(ids != rid)
        assert bad.size == 0, f"{label} by_id={by_id}: first mismatch at {bad[:3].tolist()}"


@pytest.mark.parametrize("k", [1, 7, 64, 512])
def test_topk_normal_scores(k):
    rng = np.random.default_rng(k)
    scores = rng.standard_normal((300, 1024)).astype(np.float32)
    n_valid = rng.integers(0, 1100, size=300)
    _check(scores, n_valid, k, "normal")


def test_topk_ties_and_specials():
    rng = np.random.default_rng(5)
    scores = rng.integers(-3, 4, size=(200, 700)).astype(np.float32)   # heavy ties
    pool = np.array([0.0, -0.0, np.inf, -np.inf, np.nan, 1e-40, -1e-40], dtype=np.float32)
    pick = rng.random(scores.shape) < 0.15
    scores[pick] = rng.choice(pool, size=int(pick.sum()))
    n_valid = np.concatenate([[0, 1, 700, 800, -5], rng.integers(0, 701, size=195)])
    for k in (3, 100, 700, 2048):
        _check(scores, n_valid, k, f"ties/specials k={k}")


def test_topk_long_rows():
    rng = np.random.default_rng(9)
    scores = rng.standard_normal((8, 200_000)).astype(np.float32)
    scores[2, ::7] = 1.5                      # a large tie group at the cut
    n_valid = np.array([200_000, 150_001, 200_000, 2048, 2049, 12, 4096, 4097])   # keys in registers up to 4096
    _check(scores, n_valid, 2048, "long rows")
    _check(scores, n_valid, 512, "long rows k=512")


def test_topk_register_widths():
    """Row strides that keep 4 keys per thread (up to 1024) and 16 (up to
    4096), at and around those limits, with heavy ties so that the radix
    passes stop early and the cut falls inside a tie group."""
    rng = np.random.default_rng(13)
    for ld in (1023, 1024, 1025, 2500, 4096):
        scores = rng.standard_normal((40, ld)).astype(np.float32)
        scores[::2] = np.round(scores[::2] * 2)          # ties on the even rows
        n_valid = rng.integers(0, ld + 1, size=40)
        n_valid[:4] = [ld, ld - 1, 1, 0]
        for k in (1, 511, 2048):
            _check(scores, n_valid, k, f"ld={ld} k={k}")


@pytest.mark.parametrize("by_id", [False, True])
def test_topk_then_attention(by_id):
    """Scores over the complete groups of each prefill token -> top-k on the
    GPU (by score or by id) -> the lists of the attention call; the result
    matches the oracle over the oracle's own top-k lists (bit-identical to
    the GPU's)."""
    ratio, topk = 4, 96
    positions = [(0, t) for t in range(1200, 1232)]
    p = synth.make_problem("topk_attn", "prefill", [1300], 64, 1, 128, 16, 128, ratio, topk, seed=71,
                           query_positions=positions)
    rng = np.random.default_rng(71)
    n_c = np.array([(t + 1) // ratio for _, t in positions], dtype=np.int32)
    scores = rng.standard_normal((len(positions), int(n_c.max()))).astype(np.float32)
    ids, cnt = _gpu_topk(scores, n_c, topk, by_id)
    rid, rcnt = oracle_topk(scores, n_c, topk, by_id=by_id)
    assert np.array_equal(ids, rid) and np.array_equal(cnt, rcnt)
    p.cmp_idx[:, :] = ids
    p.cmp_cnt[:] = cnt
    O, L, _ = run_hip(p, 1)
    Oref, Lref = oracle.attention(p)
    rep = accept(O, L, Oref, Lref)
    assert rep.ok, rep


@pytest.mark.parametrize("rows", [64, 600])
def test_topk_both_sort_paths(rows):
    """A launch with at most as many rows as compute units orders each row's
    selection with one network over the workgroup, a larger launch with
    per-wave runs and searches: both on ties, signed zeros, infinities, NaN
    and subnormals, and on normal scores, with selections of up to 512."""
    rng = np.random.default_rng(rows)
    scores = rng.integers(-3, 4, size=(rows, 1024)).astype(np.float32)
    pool = np.array([0.0, -0.0, np.inf, -np.inf, np.nan, 1e-40, -1e-40], dtype=np.float32)
    pick = rng.random(scores.shape) < 0.15
    scores[pick] = rng.choice(pool, size=int(pick.sum()))
    half = rows // 2
    scores[half:] = rng.standard_normal((rows - half, 1024)).astype(np.float32)
    n_valid = rng.integers(0, 1100, size=rows)
    for k in (100, 512):
        _check(scores, n_valid, k, f"sort paths rows={rows} k={k}")


@pytest.mark.parametrize("shape", ["topk_decode", "topk_prefill"])
def test_topk_bench_shapes(shape):
    """The two shapes bench.py times, with its seed and launch: 32 rows of
    1024 groups, and 2560 prefill rows of floor((t+1)/4) groups, k 512."""
    rng = np.random.default_rng(7)
    if shape == "topk_decode":
        n_valid = np.full(32, 1024, dtype=np.int32)
    else:
        n_valid = np.array([(t + 1) // 4 for t in range(2560)], dtype=np.int32)
    scores = rng.standard_normal((len(n_valid), int(n_valid.max()))).astype(np.float32)
    _check(scores, n_valid, 512, shape)
