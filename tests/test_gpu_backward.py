"""GPU parity of the backward pass (attn_bwd) with the float64 oracle
(oracle/backward.py).

The kernel takes the forward's own bf16 O and fp32 LSE (as a caller would),
rounds P and dS to bf16 for its MFMA products and adds dK and dV rows with
float atomics; the oracle recomputes O and LSE exactly.  Each gradient sums
terms of both signs, so its rounding error scales with the sum of the
terms' magnitudes, not with the result.  The tolerance is that forward-error
bound, computed here per element with u = 2^-8 (bf16 unit roundoff):
  Delta = <dO, O> from the bf16 O: |dDelta_h| <= u A_h, A_h = sum_d |O dO|
  dS = P (dP - Delta) rounded to bf16: |d ds_hj| <= u (|ds_hj| + p_hj A_h)
  dq_h <= scale sum_j (|ds_hj| + p_hj A_h) |k_j| u, and dk_j alike over h, q_h
  dv_j <= u sum_h p_hj |dO_h|  (P rounded to bf16)
  dsink_h <= u sum_i e^{sink_h - LSE_ih} A_ih
An element passes when |got - ref| <= 4 bound + 1e-6 rms(ref) (4 covers the
fp32 accumulation and the LSE's own error); no element may fail.
"""
import numpy as np
import pytest

from oracle.backward import attention_backward
from sparse_paged_attention_amd import synth

from gpu_helpers import announce, need_gpu, torch

pytestmark = pytest.mark.gpu

U = 2.0 ** -8


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()


def _dO(p, seed):
    rng = np.random.default_rng(seed)
    return synth.f32_to_bf16_bits(rng.standard_normal(p.q.shape).astype(np.float32))


def _run(p, dO_bits, want_dsink=True, repeat=1, qpb=0, fused=False):
    from sparse_paged_attention_amd import api
    dp = api.DeviceProblem.from_problem(p)
    o, lse = api.forward(dp)
    d_o = torch.from_numpy(dO_bits.view(np.int16)).cuda().view(torch.bfloat16)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    g = None
    for _ in range(repeat):
        g = api.backward(dp, o, lse, d_o, err_flag=err, want_dsink=want_dsink, grads=g, queries_per_block=qpb,
                         fused=fused)
    torch.cuda.synchronize()
    out = {k: (None if v is None else v.cpu().numpy().astype(np.float64)) for k, v in g.items()
           if not k.startswith("_")}
    return out, int(err.item())


def _bounds(p, dO_bits):
    """Per-element error bounds of the kernel's arithmetic (module docstring)."""
    import oracle
    from oracle.formats import bf16_to_f64
    P = p.page_size
    Hkv, D, Hq = p.num_kv_heads, p.head_dim, p.num_q_heads
    group = Hq // Hkv
    scale = float(np.float32(p.scale))
    q, dO = bf16_to_f64(p.q), bf16_to_f64(dO_bits)
    kr, vr = bf16_to_f64(p.k_raw), bf16_to_f64(p.v_raw)
    has_cmp = p.ratio > 0
    kc = bf16_to_f64(p.k_cmp) if has_cmp else None
    vc = bf16_to_f64(p.v_cmp) if has_cmp else None
    sink = None if p.sink is None else p.sink.astype(np.float64)
    b = {"dq": np.zeros_like(q), "dk_raw": np.zeros_like(kr), "dv_raw": np.zeros_like(vr),
         "dk_cmp": None if kc is None else np.zeros_like(kc), "dv_cmp": None if vc is None else np.zeros_like(vc),
         "d_sink": None if sink is None else np.zeros(Hq)}
    for i in range(p.num_queries):
        s = oracle.kv_set(p, i)
        crow, wrow = oracle.physical_rows(p, s)
        nc = len(crow)
        K = np.concatenate([kc[crow // P, crow % P] if nc else np.zeros((0, Hkv, D)), kr[wrow // P, wrow % P]])
        V = np.concatenate([vc[crow // P, crow % P] if nc else np.zeros((0, Hkv, D)), vr[wrow // P, wrow % P]])
        O, LSE = oracle.attend(q[i], K, V, scale, sink)
        for g in range(Hkv):
            hs = slice(g * group, (g + 1) * group)
            live = np.isfinite(LSE[hs])
            ls = np.where(live, LSE[hs], 0.0)
            pr = np.where(live[:, None], np.exp(scale * (q[i, hs] @ K[:, g].T) - ls[:, None]), 0.0)
            A = np.sum(np.abs(O[hs] * dO[i, hs]), axis=1)
            delta = np.sum(O[hs] * dO[i, hs], axis=1)
            ds = pr * (dO[i, hs] @ V[:, g].T - delta[:, None])
            m = np.abs(ds) + pr * A[:, None]                  # [group, N]
            b["dq"][i, hs] = U * scale * (m @ np.abs(K[:, g]))
            bk = U * scale * (m.T @ np.abs(q[i, hs]))
            bv = U * (pr.T @ np.abs(dO[i, hs]))
            for j, r in enumerate(crow):
                b["dk_cmp"][r // P, r % P, g] += bk[j]
                b["dv_cmp"][r // P, r % P, g] += bv[j]
            for j, r in enumerate(wrow):
                b["dk_raw"][r // P, r % P, g] += bk[nc + j]
                b["dv_raw"][r // P, r % P, g] += bv[nc + j]
            if sink is not None:
                b["d_sink"][hs] += U * np.where(live, np.exp(sink[hs] - ls), 0.0) * A
    return b


def _close(name, got, ref, bound):
    assert (got is None) == (ref is None), name
    if ref is None:
        return
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    rms = float(np.sqrt(np.mean(ref * ref))) if ref.size else 0.0
    excess = np.abs(got - ref) - (4.0 * bound + 1e-6 * rms)
    bad = np.argwhere(~(excess <= 0))
    assert bad.size == 0, (f"{name}: {len(bad)} of {ref.size} outside; first {bad[:3].tolist()} "
                           f"got {got[tuple(bad[0])]} ref {ref[tuple(bad[0])]} bound {bound[tuple(bad[0])]}")
    nz = bound > 0
    if nz.any():
        announce(f"  {name}: max |err| / bound = {np.max(np.abs(got - ref)[nz] / bound[nz]):.3f}")


def _check(p, label, seed=1, want_dsink=True, repeat=1, qpb=0, fused=False):
    announce(f"backward {label}: Nq={p.num_queries} Hq={p.num_q_heads} Hkv={p.num_kv_heads} "
             f"ratio={p.ratio} topk={p.topk} W={p.window} qpb={qpb} fused={fused}")
    dO = _dO(p, seed)
    got, err = _run(p, dO, want_dsink, repeat, qpb, fused)
    ref = attention_backward(p, dO)
    bd = _bounds(p, dO)
    _close("dq", got["dq"], ref.dq, bd["dq"])
    for k, r in (("dk_raw", ref.dk_raw), ("dv_raw", ref.dv_raw), ("dk_cmp", ref.dk_cmp), ("dv_cmp", ref.dv_cmp)):
        _close(k, got[k], None if r is None else repeat * r, None if r is None else repeat * bd[k])
    if want_dsink:
        _close("d_sink", got["d_sink"], None if ref.dsink is None else repeat * ref.dsink,
               None if ref.dsink is None else repeat * bd["d_sink"])
    return err


@pytest.mark.parametrize("qpb,fused", [(0, False), (1, False), (0, True), (1, True)])
def test_backward_prefill_csa(qpb, fused):
    """Query pairs (the library's choice here) and one query per workgroup,
    each with dK and dV from the KV-block pass (the workspace the library
    asks for) or from the fused kernel's atomics (a workspace that holds
    only the sink partials)."""
    p = synth.make_problem("bwd_csa", "prefill", [1500], 64, 1, 128, 16, 128, 4, 256, seed=81,
                           query_positions=[(0, t) for t in range(1400, 1464)], selection="score")
    assert _check(p, "prefill csa", qpb=qpb, fused=fused) == 0


def test_backward_pairs_across_sequences_and_odd_count():
    """Pairs whose queries sit in different sequences stream the two lists
    one after the other; an odd query count leaves the last pair with one
    query; positions far apart in one sequence have disjoint windows."""
    pos = [(0, 900), (1, 700), (1, 701), (0, 10), (0, 899), (1, 3), (0, 450), (0, 30), (1, 702)]
    p = synth.make_problem("bwd_mix", "prefill", [901, 703], 64, 1, 128, 16, 128, 4, 128, seed=89,
                           query_positions=pos, selection="random")
    assert _check(p, "pairs across sequences") == 0


def test_backward_group_listed_twice_pairs_match_single():
    """A list that names a group twice is outside the oracle's contract;
    every backward path counts the entry twice, as the forward does (the
    pair path falls back to the two lists one after the other; the
    KV-block pass takes the repeat as an extra item)."""
    from sparse_paged_attention_amd import api
    p = synth.make_problem("bwd_dup", "prefill", [700], 64, 1, 128, 16, 64, 4, 32, seed=90,
                           query_positions=[(0, t) for t in range(600, 608)], selection="random")
    p.cmp_idx[2, 5] = p.cmp_idx[2, 1]
    dp = api.DeviceProblem.from_problem(p)
    o, lse = api.forward(dp)
    d_o = torch.from_numpy(_dO(p, 3).view(np.int16)).cuda().view(torch.bfloat16)
    announce("backward: a group listed twice, pairs vs single")
    res = []
    for qpb, fused in ((2, False), (1, False), (1, True), (2, True)):
        g = api.backward(dp, o, lse, d_o, queries_per_block=qpb, fused=fused)
        torch.cuda.synchronize()
        res.append({k: v.cpu().numpy() for k, v in g.items() if v is not None and not k.startswith("_")})
    for other in res[1:]:
        for k in res[0]:
            a, b = res[0][k], other[k]
            scale = float(np.max(np.abs(b))) or 1.0
            assert np.max(np.abs(a - b)) <= 1e-5 * scale, k


def test_backward_decode_two_head_blocks():
    p = synth.make_problem("bwd_dec", "decode", [2100, 1700, 2500, 600], 128, 1, 128, 64, 128, 4, 512, seed=82)
    assert _check(p, "decode csa, 128 heads") == 0


def test_backward_hca_all_groups_gqa():
    """All-groups layer (ratio 128) with GQA: 2 KV heads of 40 query heads,
    so the second wave of each block has 8 real heads."""
    p = synth.make_problem("bwd_hca", "prefill", [4100, 3000], 80, 2, 128, 16, 128, 128, 0, seed=83,
                           query_positions=[(0, 4099), (0, 4000), (1, 2999), (1, 127), (0, 128), (1, 0)])
    assert _check(p, "hca gqa") == 0


def test_backward_window_only_ragged_no_sink():
    positions = [(0, t) for t in (0, 1, 5, 31, 32, 33, 127, 128, 129, 300)] + [(1, 7), (1, 64)]
    p = synth.make_problem("bwd_win", "prefill", [301, 65], 64, 1, 128, 16, 128, 0, 0, seed=84,
                           query_positions=positions, with_sink=False)
    assert _check(p, "window only") == 0


def test_backward_long_list_chunks():
    """More rows than one translation chunk (1024): a 1536-entry list plus
    the window."""
    p = synth.make_problem("bwd_long", "prefill", [8000], 64, 1, 128, 64, 128, 4, 1536, seed=85,
                           query_positions=[(0, 7999), (0, 7000), (0, 6200), (0, 500)])
    assert _check(p, "long lists") == 0


def test_backward_accumulates_and_skips_dsink():
    p = synth.make_problem("bwd_acc", "prefill", [700], 64, 1, 128, 16, 64, 4, 64, seed=86,
                           query_positions=[(0, t) for t in range(600, 620)])
    assert _check(p, "two calls accumulate", repeat=2) == 0
    assert _check(p, "no sink gradient", want_dsink=False) == 0


def test_backward_short_lists_and_bad_ids_flagged():
    """cmp_cnt below capacity (entries past it never read), and one list
    entry that names an incomplete group: it is masked as in the forward
    and flagged."""
    p = synth.make_problem("bwd_bad", "prefill", [900], 64, 1, 128, 16, 128, 4, 96, seed=87,
                           query_positions=[(0, t) for t in range(800, 816)])
    p.cmp_cnt[3] = 5
    p.cmp_cnt[4] = 0
    p.cmp_idx[3, 7:] = 10 ** 6           # past the count: never read
    from sparse_paged_attention_amd import api
    dp = api.DeviceProblem.from_problem(p)
    o, lse = api.forward(dp)
    dO = _dO(p, 5)
    d_o = torch.from_numpy(dO.view(np.int16)).cuda().view(torch.bfloat16)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    api.backward(dp, o, lse, d_o, err_flag=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    announce("backward: short counts")
    assert _check(p, "short counts", seed=5) == 0
    q = synth.make_problem("bwd_bad2", "prefill", [900], 64, 1, 128, 16, 128, 4, 96, seed=88,
                           query_positions=[(0, t) for t in range(800, 804)])
    q.cmp_idx[1, 2] = 5000                 # not a complete group at t = 801
    dq = api.DeviceProblem.from_problem(q)
    o, lse = api.forward(dq)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    d_o = torch.from_numpy(_dO(q, 6).view(np.int16)).cuda().view(torch.bfloat16)
    api.backward(dq, o, lse, d_o, err_flag=err)
    torch.cuda.synchronize()
    assert int(err.item()) & 2                   # the compressed-id bit


def test_backward_full_prefill_csa():
    """The workload bench.py times (prefill CSA, 2560 queries), every
    element against the oracle under the same bound, on the path bench.py
    times (the KV-block pass)."""
    p = synth.make_workload("prefill_csa")
    assert _check(p, "prefill_csa full", seed=5) == 0
