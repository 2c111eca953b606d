"""Pins of the backward oracle (oracle/backward.py) against things other
than its own formulas:

* central finite differences of the forward oracle's loss <dO, O> with
  respect to every input element (q, the four caches, the sink) on tiny
  problems: a dropped term, a wrong sign or a transposed operand fails them;
* closed cases: one KV row and no sink (O = v, so dq = 0, dk = 0, dv = dO);
* invariances of the definition: with no sink, shifting every value row by
  a vector u shifts O by u, so the cache's dv rows of each KV head sum to
  the dO of its query heads; shifting every key of a set by u leaves the
  softmax unchanged, so the dk rows of each KV head sum to 0.
"""
import numpy as np
import pytest

import oracle
from oracle.backward import attention_backward, backward_values
from oracle.formats import bf16_to_f64
from sparse_paged_attention_amd import synth


def _problem(with_sink=True, ratio=4, topk=2, seed=3, window=5, mode="prefill"):
    positions = [(0, 12), (0, 7), (1, 8), (1, 3), (0, 0)]
    return synth.make_problem("fd", mode, [13, 9], 4, 2, 8, 4, window, ratio, topk, seed=seed,
                              query_positions=positions if mode == "prefill" else None,
                              with_sink=with_sink)


def _inputs(p):
    has_cmp = p.ratio > 0
    return dict(q=bf16_to_f64(p.q), k_raw=bf16_to_f64(p.k_raw), v_raw=bf16_to_f64(p.v_raw),
                k_cmp=bf16_to_f64(p.k_cmp) if has_cmp else None,
                v_cmp=bf16_to_f64(p.v_cmp) if has_cmp else None,
                sink=None if p.sink is None else p.sink.astype(np.float64))


def _loss(p, x, dO):
    """<dO, O> with O from the forward oracle's attend() over the problem's
    KV sets, gathered here from the float64 arrays in x."""
    P = p.page_size
    total = 0.0
    scale = float(np.float32(p.scale))
    for i in range(p.num_queries):
        s = oracle.kv_set(p, i)
        crow, wrow = oracle.physical_rows(p, s)
        Hkv, D = p.num_kv_heads, p.head_dim
        Kc = x["k_cmp"][crow // P, crow % P] if len(crow) else np.zeros((0, Hkv, D))
        Vc = x["v_cmp"][crow // P, crow % P] if len(crow) else np.zeros((0, Hkv, D))
        K = np.concatenate([Kc, x["k_raw"][wrow // P, wrow % P]])
        V = np.concatenate([Vc, x["v_raw"][wrow // P, wrow % P]])
        O, _ = oracle.attend(x["q"][i], K, V, scale, x["sink"])
        total += float(np.sum(dO[i] * O))
    return total


def _fd_check(p, seed):
    rng = np.random.default_rng(seed)
    x = _inputs(p)
    dO = rng.standard_normal(p.q.shape)
    g = backward_values(p, x["q"], x["k_raw"], x["v_raw"], x["k_cmp"], x["v_cmp"], x["sink"], dO)
    analytic = {"q": g.dq, "k_raw": g.dk_raw, "v_raw": g.dv_raw, "k_cmp": g.dk_cmp, "v_cmp": g.dv_cmp,
                "sink": g.dsink}
    h = 1e-6
    checked = 0
    for name, arr in x.items():
        if arr is None:
            assert analytic[name] is None
            continue
        fd = np.zeros_like(arr)
        flat = arr.reshape(-1)
        for e in range(flat.size):
            old = flat[e]
            flat[e] = old + h
            lp = _loss(p, x, dO)
            flat[e] = old - h
            lm = _loss(p, x, dO)
            flat[e] = old
            fd.reshape(-1)[e] = (lp - lm) / (2 * h)
        err = np.max(np.abs(fd - analytic[name])) if arr.size else 0.0
        assert err <= 1e-7 * max(1.0, np.max(np.abs(fd))), (name, err)
        checked += int(np.count_nonzero(fd))
    assert checked > 100          # the problem actually exercises the gradients


@pytest.mark.parametrize("case", ["csa_sink", "csa_nosink", "hca_all_groups", "window_only"])
def test_backward_matches_finite_differences(case):
    p = {"csa_sink": lambda: _problem(),
         "csa_nosink": lambda: _problem(with_sink=False, seed=4),
         "hca_all_groups": lambda: _problem(ratio=4, topk=0, seed=5),
         "window_only": lambda: _problem(ratio=0, topk=0, seed=6)}[case]()
    _fd_check(p, seed=11)


def test_single_row_no_sink_closed_form():
    """One KV row (position 0, window 1) and no sink: O = v exactly, so
    dq = 0, dk = 0 and dv = dO."""
    p = synth.make_problem("one", "prefill", [4], 2, 1, 8, 4, 1, 0, 0, seed=1,
                           query_positions=[(0, 0)], with_sink=False)
    x = _inputs(p)
    dO = np.random.default_rng(2).standard_normal(p.q.shape)
    g = backward_values(p, x["q"], x["k_raw"], x["v_raw"], None, None, None, dO)
    # zero up to the rounding of <dO, v> taken in two summation orders
    assert np.max(np.abs(g.dq)) < 1e-12 and np.max(np.abs(g.dk_raw)) < 1e-12
    row = int(p.raw_pt[0, 0]) * p.page_size
    np.testing.assert_allclose(g.dv_raw[row // p.page_size, row % p.page_size, 0], dO[0].sum(axis=0), rtol=1e-15)


def test_shift_invariances_without_sink():
    p = _problem(with_sink=False, seed=8)
    x = _inputs(p)
    dO = np.random.default_rng(9).standard_normal(p.q.shape)
    g = backward_values(p, x["q"], x["k_raw"], x["v_raw"], x["k_cmp"], x["v_cmp"], None, dO)
    group = p.num_q_heads // p.num_kv_heads
    for gk in range(p.num_kv_heads):
        dv_sum = g.dv_raw[:, :, gk].sum(axis=(0, 1)) + g.dv_cmp[:, :, gk].sum(axis=(0, 1))
        want = sum(dO[i, gk * group:(gk + 1) * group].sum(axis=0) for i in range(p.num_queries)
                   if oracle.kv_set(p, i).size > 0)
        np.testing.assert_allclose(dv_sum, want, rtol=1e-12, atol=1e-12)
        dk_sum = g.dk_raw[:, :, gk].sum(axis=(0, 1)) + g.dk_cmp[:, :, gk].sum(axis=(0, 1))
        np.testing.assert_allclose(dk_sum, 0.0, atol=1e-12)


def test_bf16_entry_decodes_inputs():
    p = _problem(seed=12)
    dO = synth.f32_to_bf16_bits(np.random.default_rng(13).standard_normal(p.q.shape).astype(np.float32))
    a = attention_backward(p, dO)
    x = _inputs(p)
    b = backward_values(p, x["q"], x["k_raw"], x["v_raw"], x["k_cmp"], x["v_cmp"], x["sink"], bf16_to_f64(dO))
    assert np.array_equal(a.dq, b.dq) and np.array_equal(a.dk_cmp, b.dk_cmp) and np.array_equal(a.dsink, b.dsink)
    with pytest.raises(NotImplementedError):
        attention_backward(synth.make_workload("mixed_fp8"), dO)
