"""Pins of the FP64 oracle against things other than itself.

What pins what:
* KV-set rule: sizes printed on the pages (tests/golden/kv_set_sizes.txt),
  plus a brute-force enumeration of membership predicates.
* Attention math: reduction to textbook dense causal softmax attention, and
  an mpmath 50-digit brute force on tiny inputs over unpaged logical arrays.
* Order invariance: permuted index lists (within 1e-12), permuted physical
  page placement (bitwise).
* Merge: random partitions and random merge trees (atol 1e-12), as in the
  tessera Block AttnRes PR's merge-lemma test.
* Sink: closed forms for one KV entry and the two limits.
* Formats: the e4m3 table against an independent enumeration of the format's
  values and special codes; bf16 widening against known bit patterns.
* Comparator: a x1.05 perturbation must fail (ATOM DeepSeek-V4 block test PR,
  "Pass criterion").
"""
import math
import os

import mpmath
import numpy as np
import pytest

import oracle
from oracle import sparse_attention as A
from oracle.compare import accept
from sparse_paged_attention_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden_rows():
    rows = []
    with open(os.path.join(GOLDEN, "kv_set_sizes.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if not line:
                continue
            name, *vals = line.split()
            rows.append((name, [None if v == "-" else int(v) for v in vals]))
    return rows


@pytest.mark.parametrize("name,vals", _golden_rows(), ids=[r[0] for r in _golden_rows()])
def test_kv_set_sizes_printed(name, vals):
    ratio, window, topk, seqlen, pos, n_c, n_sel, win_len, total = vals
    p = synth.make_problem(name, "prefill", [seqlen], 2, 1, 8, 16, window, ratio, topk,
                           seed=11, query_positions=[(0, pos)], selection="random",
                           keep_logical=False, spare_pages=0)
    s = A.kv_set(p, 0)
    assert s.n_c == n_c
    assert s.n_sel == n_sel
    if win_len is not None:
        assert s.win_len == win_len
    if total is not None:
        assert s.size == total


def test_kv_set_rule_brute_enumeration():
    """Enumerate membership over every position: a raw position p is in the
    window of t iff t-W < p <= t; a group c is complete at t iff its last token
    r*c + r-1 is at or before t."""
    for ratio, W in [(4, 16), (128, 128), (0, 5), (1, 3), (4, 0)]:
        L = 300
        p = synth.make_problem("enum", "prefill", [L], 2, 1, 8, 16, W, ratio, 0,
                               seed=3, query_positions=[(0, t) for t in range(L)],
                               keep_logical=False)
        for t in range(L):
            s = A.kv_set(p, t)
            win = [q for q in range(L) if t - W < q <= t]
            groups = [c for c in range(L) if ratio > 0 and ratio * c + ratio - 1 <= t]
            assert list(s.win_pos) == win
            assert list(s.cmp_ids) == groups


# ------------------------------------------------------------ dense reduction

def _textbook_causal(q, k, v, scale):
    """Dense causal softmax attention with a full score matrix and a
    bottom-right causal mask; q [T, Hq, D], k/v [L, Hkv, D], queries are the
    last T positions."""
    T, Hq, D = q.shape
    L, Hkv, _ = k.shape
    grp = Hq // Hkv
    out = np.zeros((T, Hq, D))
    lse = np.zeros((T, Hq))
    qpos = np.arange(L - T, L)
    mask = np.arange(L)[None, :] <= qpos[:, None]            # [T, L]
    for h in range(Hq):
        g = h // grp
        S = scale * q[:, h, :] @ k[:, g, :].T
        S = np.where(mask, S, -np.inf)
        mx = S.max(axis=1, keepdims=True)
        E = np.exp(S - mx)
        Z = E.sum(axis=1, keepdims=True)
        out[:, h] = (E / Z) @ v[:, g, :]
        lse[:, h] = (mx + np.log(Z))[:, 0]
    return out, lse


def _bf(x):
    return oracle.bf16_to_f64(x)


@pytest.mark.parametrize("Hq,Hkv", [(4, 1), (4, 2), (6, 3)])
def test_dense_reduction_window_only(Hq, Hkv):
    L = 40
    p = synth.make_problem("dense", "prefill", [L], Hq, Hkv, 16, 8, L + 5, 0, 0, seed=5,
                           query_positions=[(0, t) for t in range(L)], with_sink=False)
    O, LSE = oracle.attention(p)
    Oref, Lref = _textbook_causal(_bf(p.q), _bf(p.k_raw_logical[0]), _bf(p.v_raw_logical[0]),
                                  float(p.scale))
    np.testing.assert_allclose(O, Oref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(LSE, Lref, rtol=0, atol=1e-12)


def test_dense_reduction_shared_latent_d512():
    """A 512-wide shared latent cache (one array is K and V) in 256-token
    pages: window-only attention over all positions is dense causal
    attention with v = k."""
    L = 300
    p = synth.make_problem("latent", "prefill", [L], 4, 1, 512, 256, L + 1, 0, 0, seed=7,
                           query_positions=[(0, t) for t in (0, 1, 100, 255, 256, 299)], with_sink=False,
                           shared_kv=True)
    assert p.v_raw is p.k_raw
    O, LSE = oracle.attention(p)
    k = _bf(p.k_raw_logical[0])
    Oref, Lref = _textbook_causal(_bf(p.q[[5]]), k, k, float(p.scale))   # t = 299: the last row
    np.testing.assert_allclose(O[5], Oref[0], rtol=0, atol=1e-12)
    np.testing.assert_allclose(LSE[5], Lref[0], rtol=0, atol=1e-12)
    for i, t in enumerate((0, 1, 100, 255, 256)):
        Oi, Li = _textbook_causal(_bf(p.q[[i]]), k[:t + 1], k[:t + 1], float(p.scale))
        np.testing.assert_allclose(O[i], Oi[0], rtol=0, atol=1e-12)
        np.testing.assert_allclose(LSE[i], Li[0], rtol=0, atol=1e-12)


def test_dense_reduction_ratio1_compressed_equals_raw():
    """r = 1, compressed cache holding the raw rows, every group selected,
    no window: again dense causal attention."""
    L = 33
    p = synth.make_problem("r1", "prefill", [L], 4, 1, 16, 8, 0, 1, 0, seed=6,
                           query_positions=[(0, t) for t in range(L)], with_sink=False)
    # copy the raw logical rows into the compressed pages
    P = p.page_size
    for c in range(L):
        pg = p.cmp_pt[0, c // P]
        p.k_cmp[pg, c % P] = p.k_raw_logical[0][c]
        p.v_cmp[pg, c % P] = p.v_raw_logical[0][c]
    O, LSE = oracle.attention(p)
    Oref, Lref = _textbook_causal(_bf(p.q), _bf(p.k_raw_logical[0]), _bf(p.v_raw_logical[0]),
                                  float(p.scale))
    np.testing.assert_allclose(O, Oref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(LSE, Lref, rtol=0, atol=1e-12)


# ------------------------------------------------------------ brute force

mpmath.mp.dps = 50


def _brute(p):
    """Membership predicates over unpaged logical arrays, sums of exp in
    50-digit arithmetic."""
    Nq, Hq, D = p.q.shape
    Hkv = p.num_kv_heads
    grp = Hq // Hkv
    scale = mpmath.mpf(float(np.float32(p.scale)))
    O = np.zeros((Nq, Hq, D))
    LSE = np.zeros((Nq, Hq))
    for i in range(Nq):
        b = i if p.mode == "decode" else int(p.query_seq[i])
        t = int(p.seq_lens[b]) - 1 if p.mode == "decode" else int(p.query_pos[i])
        members = []   # (k row f64[Hkv,D], v row)
        kr, vr = _bf(p.k_raw_logical[b]), _bf(p.v_raw_logical[b])
        if p.cmp_fp8:
            dec = oracle.e4m3fnuz_to_f64 if p.cmp_fp8_fnuz else oracle.e4m3_to_f64
            kc = dec(p.k_cmp_logical[b]) * p.k_cmp_scale_logical[b].astype(np.float64)[..., None]
            vc = dec(p.v_cmp_logical[b]) * p.v_cmp_scale_logical[b].astype(np.float64)[..., None]
        else:
            kc, vc = _bf(p.k_cmp_logical[b]), _bf(p.v_cmp_logical[b])
        for c in range(kc.shape[0]):
            complete = p.ratio > 0 and p.ratio * (c + 1) <= t + 1
            listed = (p.topk == 0) or (c in set(int(x) for x in p.cmp_idx[i, :p.cmp_cnt[i]]))
            if complete and listed:
                members.append((kc[c], vc[c]))
        for pos in range(int(p.seq_lens[b])):
            if t - p.window < pos <= t:
                members.append((kr[pos], vr[pos]))
        q = _bf(p.q[i])
        for h in range(Hq):
            g = h // grp
            ss = [scale * mpmath.fsum(mpmath.mpf(float(a)) * mpmath.mpf(float(bb))
                                      for a, bb in zip(q[h], k[g])) for k, _ in members]
            ex = [mpmath.exp(s) for s in ss]
            Z = mpmath.fsum(ex)
            if p.sink is not None:
                Z += mpmath.exp(mpmath.mpf(float(p.sink[h])))
            LSE[i, h] = float(mpmath.log(Z))
            for d in range(D):
                O[i, h, d] = float(mpmath.fsum(e * mpmath.mpf(float(v[g][d]))
                                               for e, (_, v) in zip(ex, members)) / Z)
    return O, LSE


def test_brute_force_tiny():
    p = synth.make_workload("tiny")
    sel = [0, 7, 15]
    p_small = _subset_queries(p, sel)
    O, L = oracle.attention(p_small)
    Ob, Lb = _brute(p_small)
    np.testing.assert_allclose(O, Ob, rtol=0, atol=1e-12)
    np.testing.assert_allclose(L, Lb, rtol=0, atol=1e-12)


@pytest.mark.parametrize("fp8,topk,ratio", [(True, 5, 4), (False, 0, 8), (True, 0, 2)])
def test_brute_force_variants(fp8, topk, ratio):
    L = 37
    p = synth.make_problem("bv", "prefill", [L], 4, 2, 8, 8, 6, ratio, topk, seed=9,
                           cmp_fp8=fp8, query_positions=[(0, t) for t in (0, 5, 20, 36)],
                           selection="random")
    O, LSE = oracle.attention(p)
    Ob, Lb = _brute(p)
    np.testing.assert_allclose(O, Ob, rtol=0, atol=1e-12)
    np.testing.assert_allclose(LSE, Lb, rtol=0, atol=1e-12)


def test_brute_force_fnuz_pages():
    L = 37
    p = synth.make_problem("bvf", "prefill", [L], 4, 2, 8, 8, 6, 4, 5, seed=19, cmp_fp8=True,
                           fp8_format="fnuz", query_positions=[(0, t) for t in (3, 20, 36)], selection="random")
    assert p.cmp_fp8_fnuz
    O, LSE = oracle.attention(p)
    Ob, Lb = _brute(p)
    np.testing.assert_allclose(O, Ob, rtol=0, atol=1e-12)
    np.testing.assert_allclose(LSE, Lb, rtol=0, atol=1e-12)


def _subset_queries(p, sel):
    import copy
    q = copy.copy(p)
    q.q = p.q[sel]
    q.query_seq = p.query_seq[sel]
    q.query_pos = p.query_pos[sel]
    q.cmp_idx = p.cmp_idx[sel]
    q.cmp_cnt = p.cmp_cnt[sel]
    return q


# ------------------------------------------------------------ invariances

def test_permuted_index_lists():
    p = synth.make_workload("tiny")
    O, L = oracle.attention(p)
    rng = np.random.default_rng(1)
    for i in range(p.num_queries):
        c = p.cmp_cnt[i]
        p.cmp_idx[i, :c] = p.cmp_idx[i, :c][rng.permutation(c)]
    O2, L2 = oracle.attention(p)
    np.testing.assert_allclose(O2, O, rtol=0, atol=1e-12)
    np.testing.assert_allclose(L2, L, rtol=0, atol=1e-12)


def _repage(p, seed):
    """Move every page of both pools to a new random slot; same logical data."""
    rng = np.random.default_rng(seed)
    for kk, vv, pt in (("k_raw", "v_raw", "raw_pt"), ("k_cmp", "v_cmp", "cmp_pt")):
        n = getattr(p, kk).shape[0]
        perm = rng.permutation(n)
        for name in (kk, vv):
            old = getattr(p, name)
            new = np.empty_like(old)
            new[perm] = old
            setattr(p, name, new)
        if kk == "k_cmp" and p.k_cmp_scale is not None:
            for name in ("k_cmp_scale", "v_cmp_scale"):
                old = getattr(p, name)
                new = np.empty_like(old)
                new[perm] = old
                setattr(p, name, new)
        tab = getattr(p, pt)
        valid = tab != synth.PT_PAD
        tab = tab.copy()
        tab[valid] = perm[tab[valid]]
        setattr(p, pt, tab)


@pytest.mark.parametrize("fp8", [False, True])
def test_permuted_pages_bitwise(fp8):
    p = synth.make_problem("pg", "decode", [100, 57, 230], 8, 2, 16, 16, 32, 4, 12, seed=4,
                           cmp_fp8=fp8)
    O, L = oracle.attention(p)
    _repage(p, 3)
    O2, L2 = oracle.attention(p)
    assert np.array_equal(O, O2) and np.array_equal(L, L2)


# ------------------------------------------------------------ merge

def _random_tree_merge(parts, rng):
    """Merge a list of sink-free partials pairwise in a random tree order."""
    parts = list(parts)
    while len(parts) > 1:
        i, j = sorted(rng.choice(len(parts), size=2, replace=False))
        merged = A.merge([parts[i], parts[j]], None)
        parts = [x for k, x in enumerate(parts) if k not in (i, j)] + [merged]
    return parts[0]


def test_merge_random_partitions():
    p = synth.make_problem("mg", "decode", [300, 1000, 77], 8, 2, 16, 16, 64, 4, 40, seed=8)
    rng = np.random.default_rng(0)
    scale = float(p.scale)
    sink = p.sink.astype(np.float64)
    for i in range(p.num_queries):
        s = A.kv_set(p, i)
        K, V = A.gather_rows(p, s)
        q = A.query_f64(p, i)
        ref = A.attend(q, K, V, scale, sink)
        for trial in range(6):
            nparts = int(rng.integers(1, 9))
            lab = rng.integers(0, nparts, size=len(K))
            parts = [A.attend_partial(q, K[lab == j], V[lab == j], scale) for j in range(nparts)]
            root = _random_tree_merge(parts, rng)
            O, L = A.merge([root], sink)
            np.testing.assert_allclose(O, ref[0], rtol=0, atol=1e-12)
            np.testing.assert_allclose(L, ref[1], rtol=0, atol=1e-12)
            # flat merge with sink folded once
            O2, L2 = A.merge(parts, sink)
            np.testing.assert_allclose(O2, ref[0], rtol=0, atol=1e-12)
            np.testing.assert_allclose(L2, ref[1], rtol=0, atol=1e-12)


def test_merge_contiguous_splits_and_empty():
    p = synth.make_workload("tiny")
    scale = float(p.scale)
    sink = p.sink.astype(np.float64)
    for i in range(p.num_queries):
        s = A.kv_set(p, i)
        K, V = A.gather_rows(p, s)
        q = A.query_f64(p, i)
        ref = A.attend(q, K, V, scale, sink)
        for S in (1, 2, 3, 4, 7, 40):
            parts = [A.attend_partial(q, K[a:b], V[a:b], scale) for a, b in A.partial_split(len(K), S)]
            O, L = A.merge(parts, sink)
            np.testing.assert_allclose(O, ref[0], rtol=0, atol=1e-12)
            np.testing.assert_allclose(L, ref[1], rtol=0, atol=1e-12)
    empty = A.attend_partial(np.ones((2, 4)), np.zeros((0, 1, 4)), np.zeros((0, 1, 4)), 1.0)
    assert np.all(empty[1] == -np.inf) and np.all(empty[0] == 0)


def test_lse_merge_arrays_flat_rows():
    """The flat-array merge (rows = query * Hq + head, sink of row r is
    sink[r % Hq]) over 3 contiguous partials of every query's KV set equals the
    sink-folded single pass, query by query and head by head."""
    p = synth.make_workload("tiny")
    scale = float(p.scale)
    Hq, D, S = p.num_q_heads, p.head_dim, 3
    o_parts = np.zeros((S, p.num_queries * Hq, D))
    lse_parts = np.zeros((S, p.num_queries * Hq))
    for i in range(p.num_queries):
        s = A.kv_set(p, i)
        K, V = A.gather_rows(p, s)
        q = A.query_f64(p, i)
        for j, (a, b) in enumerate(A.partial_split(len(K), S)):
            o, l = A.attend_partial(q, K[a:b], V[a:b], scale)
            o_parts[j, i * Hq:(i + 1) * Hq] = o
            lse_parts[j, i * Hq:(i + 1) * Hq] = l
    O, L = A.lse_merge_arrays(o_parts, lse_parts, p.sink, Hq)
    Oref, Lref = oracle.attention(p)
    np.testing.assert_allclose(O.reshape(Oref.shape), Oref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(L.reshape(Lref.shape), Lref, rtol=0, atol=1e-12)
    # a sink row mapping shifted by one head must not pass
    O2, _ = A.lse_merge_arrays(o_parts, lse_parts, np.roll(p.sink, 1), Hq)
    assert np.abs(O2.reshape(Oref.shape) - Oref).max() > 1e-6


def test_partial_split_covers():
    for n in range(0, 50):
        for S in range(1, 9):
            sl = A.partial_split(n, S)
            assert len(sl) == S
            assert sl[0][0] == 0 and sl[-1][1] == n
            assert all(sl[j][1] == sl[j + 1][0] for j in range(S - 1))


# ------------------------------------------------------------ sink closed forms

def test_sink_single_entry_closed_form():
    rng = np.random.default_rng(2)
    for _ in range(50):
        D = 8
        q = rng.standard_normal((3, D))
        K = rng.standard_normal((1, 1, D))
        V = rng.standard_normal((1, 1, D))
        sink = rng.standard_normal(3) * 3
        scale = 0.3
        O, L = A.attend(q, K, V, scale, sink)
        s = scale * q @ K[0, 0]
        sig = 1.0 / (1.0 + np.exp(-(s - sink)))
        np.testing.assert_allclose(O, sig[:, None] * V[0, 0][None, :], rtol=1e-13, atol=1e-14)
        np.testing.assert_allclose(L, np.logaddexp(s, sink), rtol=0, atol=1e-13)


def test_sink_limits():
    rng = np.random.default_rng(3)
    q = rng.standard_normal((4, 8))
    K = rng.standard_normal((5, 1, 8))
    V = rng.standard_normal((5, 1, 8))
    s = 0.5 * q @ K[:, 0].T
    w = np.exp(s - s.max(1, keepdims=True))
    plain = (w / w.sum(1, keepdims=True)) @ V[:, 0]
    O, L = A.attend(q, K, V, 0.5, None)
    np.testing.assert_allclose(O, plain, atol=1e-13)
    O, L = A.attend(q, K, V, 0.5, np.full(4, -1e4))
    np.testing.assert_allclose(O, plain, atol=1e-13)
    O, L = A.attend(q, K, V, 0.5, np.full(4, 1e4))
    assert np.all(np.abs(O) < 1e-300) and np.allclose(L, 1e4)
    # empty set: sink alone -> O = 0, LSE = sink;  no sink -> LSE = -inf
    Oe, Le = A.attend(q, K[:0], V[:0], 0.5, np.array([1.0, 2, 3, 4]))
    assert np.all(Oe == 0) and np.allclose(Le, [1, 2, 3, 4])
    Oe, Le = A.attend(q, K[:0], V[:0], 0.5, None)
    assert np.all(Oe == 0) and np.all(Le == -np.inf)


# ------------------------------------------------------------ formats

def test_e4m3fnuz_table_properties():
    """FNUZ e4m3 (bias 8): +-240 at 0x7F / 0xFF, the only NaN at 0x80, the
    smallest subnormal 2^-10 and smallest normal 2^-7, sign symmetry, a
    monotone positive half, and the cross-format identity FNUZ(c) = OCP(c)/2
    for every other code (the exponent bias is one larger)."""
    f = oracle.e4m3fnuz_table()
    o = oracle.e4m3_table()
    assert f[0x7F] == 240.0 and f[0xFF] == -240.0
    assert np.isnan(f[0x80]) and np.isnan(f).sum() == 1
    assert f[0x01] == 2.0 ** -10 and f[0x08] == 2.0 ** -7 and f[0x00] == 0.0
    assert np.all(np.diff(f[:0x80]) > 0)
    for c in range(1, 128):
        assert f[c | 0x80] == -f[c]
    for c in range(256):
        if c not in (0x7F, 0xFF, 0x80):
            assert f[c] == o[c] / 2, hex(c)


def test_e4m3fnuz_quantise_roundtrip_and_rounding():
    f = oracle.e4m3fnuz_table()
    codes = np.array([c for c in range(256) if c != 0x80], dtype=np.uint8)
    back = synth.quantize_e4m3_fnuz(f[codes])
    assert np.all(f[back] == f[codes])           # every finite value maps to its own value
    assert not np.any(back == 0x80)
    # midpoints between neighbours round to the even code; beyond 240 saturates
    pos = f[:0x80]
    mids = (pos[:-1] + pos[1:]) / 2
    got = synth.quantize_e4m3_fnuz(mids)
    want = np.where(np.arange(127) % 2 == 0, np.arange(127), np.arange(1, 128))
    assert np.array_equal(got, want.astype(np.uint8))
    assert synth.quantize_e4m3_fnuz(np.array([1e6, -1e6]))[0] == 0x7F
    assert synth.quantize_e4m3_fnuz(np.array([-1e6]))[0] == 0xFF
    assert synth.quantize_e4m3_fnuz(np.array([-0.0, -1e-9]))[0] == 0x00


def test_e4m3_table_enumeration():
    """The OCP e4m3 finite positives are m*2^-9 (m = 0..7, subnormal) and
    (8+m)*2^(e-10) for exponent fields e = 1..15, except e = 15, m = 7 (NaN);
    codes are ordered by magnitude, the sign bit mirrors them."""
    tab = oracle.e4m3_table()
    expected = [m * 2.0 ** -9 for m in range(8)]
    expected += [(8 + m) * 2.0 ** (e - 10) for e in range(1, 16) for m in range(8)][:-1]
    assert len(expected) == 127
    assert np.array_equal(tab[:127], np.array(expected))
    assert np.array_equal(tab[128:255], -np.array(expected))
    assert math.isnan(tab[127]) and math.isnan(tab[255])
    assert tab[0x7E] == 448.0 and tab[0x38] == 1.0 and tab[0x08] == 2.0 ** -6
    assert tab[0x01] == 2.0 ** -9 and tab[0xB8] == -1.0


def test_e4m3_quantise_roundtrip_and_rounding():
    tab = oracle.e4m3_table()
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF, 0x80)], dtype=np.uint8)
    assert np.array_equal(synth.quantize_e4m3(tab[codes]), codes)
    # saturation and ties-to-even between neighbours
    assert synth.quantize_e4m3(np.array([1e6]))[0] == 0x7E
    assert synth.quantize_e4m3(np.array([-500.0]))[0] == 0xFE
    fin = tab[:127]
    mids = (fin[:-1] + fin[1:]) / 2
    q = synth.quantize_e4m3(mids)
    lo = np.arange(126)
    even = np.where(lo % 2 == 0, lo, lo + 1)
    assert np.array_equal(q, even.astype(np.uint8))


def test_bf16_widening():
    bits = np.array([0x3F80, 0xC000, 0x0001, 0x7F7F, 0x8000], dtype=np.uint16)
    vals = oracle.bf16_to_f64(bits)
    assert vals[0] == 1.0 and vals[1] == -2.0 and vals[2] == 2.0 ** -133
    assert vals[3] == (2 - 2.0 ** -7) * 2.0 ** 127 and vals[4] == 0.0
    assert np.isinf(oracle.bf16_to_f64(np.array([0x7F80], dtype=np.uint16))[0])
    # generator rounding: ties to even
    x = np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, 1.0 + 2.0 ** -9], dtype=np.float32)
    assert list(synth.f32_to_bf16_bits(x)) == [0x3F80, 0x3F82, 0x3F80]


# ------------------------------------------------------------ comparator

def test_comparator_rejects_perturbation():
    p = synth.make_workload("tiny")
    O, L = oracle.attention(p)
    assert accept(O, L, O, L).ok
    assert not accept(O * 1.05, L, O, L).ok
    bad = O.copy()
    bad[0, 0, 0] = np.nan
    assert not accept(bad, L, O, L).ok
    assert not accept(O, L + 2e-3, O, L).ok
    assert accept(O, L + 5e-4, O, L).ok


# ------------------------------------------------------------ generator

@pytest.mark.parametrize("name", ["tiny", "decode_csa", "decode_hca", "mixed_fp8"])
def test_generator_invariants(name):
    p = synth.make_workload(name, batch=4 if name != "tiny" else None, keep_logical=True)
    for pt, pool in ((p.raw_pt, p.k_raw), (p.cmp_pt, p.k_cmp)):
        used = pt[pt != synth.PT_PAD]
        assert len(np.unique(used)) == len(used)            # pages never shared
        assert used.min() >= 0 and used.max() < pool.shape[0]
    for i in range(p.num_queries):
        s = A.kv_set(p, i)                                   # validates the list
        if p.topk:
            assert p.cmp_cnt[i] == min(p.topk, s.n_c)
            assert np.all(p.cmp_idx[i, p.cmp_cnt[i]:] == -1)


def test_gather_plan_rows_hold_logical_rows():
    """Every row the plan names holds exactly the logical row it stands for
    (a content check, independent of the translation formula)."""
    p = synth.make_problem("gp", "decode", [90, 300, 17], 4, 1, 8, 16, 32, 4, 10, seed=12)
    rows, counts = A.gather_plan(p, 64)
    P = p.page_size
    for i in range(p.num_queries):
        win_lo, win_len, n_c, n_sel = counts[i]
        for j in range(n_sel):
            r = rows[i, j]
            assert np.array_equal(p.k_cmp[r // P, r % P], p.k_cmp_logical[i][p.cmp_idx[i, j]])
        for j in range(win_len):
            r = rows[i, n_sel + j]
            assert np.array_equal(p.v_raw[r // P, r % P], p.v_raw_logical[i][win_lo + j])
        assert np.all(rows[i, n_sel + win_len:] == -1)
