"""GPU parity with KV pages placed beyond byte offset 2^32 of their pools.

RL-Kernel "Fixed paged CK attention on ROCm": cache addressing stays 64-bit
once a K/V view spans more than 2 GB.  Each cache pool of a problem is laid out
again on the device in a pool of more than 4.5 GiB: its pages alternate
between the top of the new pool (beyond 4 GiB) and its bottom, the unused
pages hold NaN, and the page tables are remapped to match.  Where a page sits
does not change the result, so every kernel must still match the oracle run
on the original problem, and the gather export must name the remapped rows.
Each kernel path is covered: the decode kernel (bf16 and e4m3 pages, one and
several slices), the job-stream kernel, the prefill query pairs and the
one-query prefill, the 512-wide latent kernel (bf16 and e4m3 pages), the
backward and the gather."""
import dataclasses

import numpy as np
import pytest

import oracle
from oracle.compare import accept
from sparse_paged_attention_amd import synth

from gpu_helpers import announce, need_gpu, to_numpy_bf16, torch

pytestmark = pytest.mark.gpu

BIG = int(4.5 * (1 << 30))          # bytes of every relocated pool
FOUR_GIB = 1 << 32


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()


@pytest.fixture(autouse=True)
def _release():
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _page_map(old_pages, page_bytes):
    """New page id of every old page: even pages from the top of a pool of
    more than BIG bytes down, odd pages from its bottom up."""
    new_pages = max(-(-BIG // page_bytes), 2 * old_pages + 2)
    j = np.arange(old_pages)
    new = np.where(j % 2 == 0, new_pages - 1 - j // 2, j // 2).astype(np.int64)
    assert new.max() * page_bytes >= FOUR_GIB      # the top pages lie beyond 2^32
    return new_pages, new


def _relocate_pool(t, new_pages, new_ids, fill):
    big = torch.empty((new_pages,) + tuple(t.shape[1:]), dtype=t.dtype, device=t.device)
    big.view(torch.uint8).fill_(fill)
    big[torch.from_numpy(new_ids).to(t.device)] = t
    return big


def _remap_pt(pt, new_ids):
    out = pt.clone()
    valid = pt != int(synth.PT_PAD)
    out[valid] = torch.from_numpy(new_ids.astype(np.int32)).to(pt.device)[pt[valid].long()]
    return out


def relocate(dp):
    """A copy of the device problem whose pools exceed 4.5 GiB, with the pages
    spread below and beyond 4 GiB; returns (problem, raw map, cmp map)."""
    out = dataclasses.replace(dp)
    page_bytes = dp.k_raw[0].numel() * dp.k_raw.element_size()
    n_raw, raw_ids = _page_map(dp.k_raw.shape[0], page_bytes)
    out.k_raw = _relocate_pool(dp.k_raw, n_raw, raw_ids, 0xFF)        # bf16 0xFFFF: NaN
    out.v_raw = out.k_raw if dp.v_raw is dp.k_raw else _relocate_pool(dp.v_raw, n_raw, raw_ids, 0xFF)
    out.raw_pt = _remap_pt(dp.raw_pt, raw_ids)
    cmp_ids = None
    if dp.k_cmp is not None:
        page_bytes = dp.k_cmp[0].numel() * dp.k_cmp.element_size()
        n_cmp, cmp_ids = _page_map(dp.k_cmp.shape[0], page_bytes)
        fill = 0x7F if dp.cmp_fp8 else 0xFF                             # e4m3 0x7F: NaN (OCP)
        out.k_cmp = _relocate_pool(dp.k_cmp, n_cmp, cmp_ids, fill)
        out.v_cmp = out.k_cmp if dp.v_cmp is dp.k_cmp else _relocate_pool(dp.v_cmp, n_cmp, cmp_ids, fill)
        if dp.k_cmp_scale is not None:
            out.k_cmp_scale = _relocate_pool(dp.k_cmp_scale, n_cmp, cmp_ids, 0xFF)
            out.v_cmp_scale = (out.k_cmp_scale if dp.v_cmp_scale is dp.k_cmp_scale
                               else _relocate_pool(dp.v_cmp_scale, n_cmp, cmp_ids, 0xFF))
        out.cmp_pt = _remap_pt(dp.cmp_pt, cmp_ids)
    return out, raw_ids, cmp_ids


def _forward_check(p, label, num_splits=None, hpb=0, qpb=0):
    from sparse_paged_attention_amd import api
    dp = api.DeviceProblem.from_problem(p)
    big, _, _ = relocate(dp)
    announce(f"beyond 4 GiB {label}: pools {big.k_raw.shape[0]} raw pages, "
             f"{0 if big.k_cmp is None else big.k_cmp.shape[0]} compressed pages, splits={num_splits} "
             f"hpb={hpb} qpb={qpb}")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    O, L = api.forward(big, num_splits, err_flag=err, heads_per_block=hpb, queries_per_block=qpb)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    Oref, Lref = oracle.attention(p)
    rep = accept(to_numpy_bf16(O), L.cpu().numpy().astype(np.float64), Oref, Lref)
    assert rep.ok, f"{label}: {rep}"


def _small_prefill(seed=11):
    return synth.make_problem("prefill_far", "prefill", [300, 200], 64, 1, 128, 16, 64, 4, 32, seed=seed,
                              query_positions=[(0, t) for t in range(250, 265)] + [(1, t) for t in (0, 7, 199)],
                              selection="score")


@pytest.mark.parametrize("splits", [1, 4])
def test_decode_kernel_beyond_4gib(splits):
    _forward_check(synth.make_workload("decode_csa", batch=4), f"decode S{splits}", num_splits=splits)


@pytest.mark.parametrize("splits", [1, 4])
def test_decode_kernel_e4m3_beyond_4gib(splits):
    """S 1: the one-pass kernel (e4m3 rows kept as code addresses); S 4: the
    slice kernel and the merge."""
    _forward_check(synth.make_workload("mixed_fp8", batch=3), f"decode e4m3 S{splits}", num_splits=splits)


def test_decode_all_groups_beyond_4gib():
    _forward_check(synth.make_workload("decode_hca", batch=2), "decode all-groups S4", num_splits=4)


def test_job_stream_kernel_beyond_4gib():
    _forward_check(synth.make_workload("decode_csa", batch=3), "job streams S2", num_splits=2, hpb=64)
    _forward_check(synth.make_workload("tiny"), "job streams tiny (D 64)")


@pytest.mark.parametrize("qpb", [0, 1])
def test_prefill_kernels_beyond_4gib(qpb):
    _forward_check(_small_prefill(), f"prefill qpb={qpb}", qpb=qpb)


def test_latent_kernel_beyond_4gib():
    _forward_check(synth.make_workload("decode_latent", batch=2), "latent D512 S2", num_splits=2)


def test_latent_e4m3_beyond_4gib():
    p = synth.make_problem("lat_f8_far", "decode", [1300, 4096, 130], 64, 1, 512, 256, 128, 4, 200, seed=38,
                           shared_kv=True, cmp_fp8=True)
    _forward_check(p, "latent e4m3 D512 S2", num_splits=2)


def test_gather_beyond_4gib():
    from sparse_paged_attention_amd import api
    p = synth.make_workload("mixed_fp8", batch=3)
    dp = api.DeviceProblem.from_problem(p)
    big, raw_ids, cmp_ids = relocate(dp)
    cap = p.window + p.topk + 3
    rows, counts = api.build_gather(big, cap)
    torch.cuda.synchronize()
    rref, cref = oracle.gather_plan(p, cap)
    assert np.array_equal(counts.cpu().numpy(), cref)
    # the oracle's rows are in the original pools: move each to its new page
    P = p.page_size
    want = rref.copy()
    for i in range(p.num_queries):
        n_sel = int(cref[i, 3])
        for e in range(cap):
            r = int(rref[i, e])
            if r < 0:
                continue
            ids = cmp_ids if e < n_sel else raw_ids
            want[i, e] = int(ids[r // P]) * P + r % P
    got = rows.cpu().numpy()
    assert np.array_equal(got, want)
    # raw rows (bf16 K or V, Hkv * D * 2 bytes each) beyond byte offset 2^32 were named
    raw_row_bytes = p.num_kv_heads * p.head_dim * 2
    is_raw = np.arange(cap)[None, :] >= cref[:, 3:4]
    assert (got[is_raw & (got >= 0)] * raw_row_bytes >= FOUR_GIB).any()


def test_backward_beyond_4gib():
    from sparse_paged_attention_amd import api
    from oracle.backward import attention_backward
    from test_gpu_backward import _bounds, _close, _dO

    p = _small_prefill(seed=13)
    dO_bits = _dO(p, 3)
    dp = api.DeviceProblem.from_problem(p)
    big, raw_ids, cmp_ids = relocate(dp)
    announce(f"beyond 4 GiB backward: raw pool {big.k_raw.shape[0]} pages")
    o, lse = api.forward(big)
    d_o = torch.from_numpy(dO_bits.view(np.int16)).cuda().view(torch.bfloat16)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    g = api.backward(big, o, lse, d_o, err_flag=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    ref = attention_backward(p, dO_bits)
    bound = _bounds(p, dO_bits)
    raw_sel = torch.from_numpy(raw_ids).cuda()
    cmp_sel = torch.from_numpy(cmp_ids).cuda()
    got = {"dq": g["dq"], "dk_raw": g["dk_raw"][raw_sel], "dv_raw": g["dv_raw"][raw_sel],
           "dk_cmp": g["dk_cmp"][cmp_sel], "dv_cmp": g["dv_cmp"][cmp_sel], "d_sink": g["d_sink"]}
    # every page other than the placed ones stays zero in the large pools
    for name, ids in (("dk_raw", raw_sel), ("dv_raw", raw_sel), ("dk_cmp", cmp_sel), ("dv_cmp", cmp_sel)):
        g[name][ids] = 0.0
        assert float(g[name].abs().max().item()) == 0.0, name
    refs = {"dq": ref.dq, "dk_raw": ref.dk_raw, "dv_raw": ref.dv_raw, "dk_cmp": ref.dk_cmp, "dv_cmp": ref.dv_cmp,
            "d_sink": ref.dsink}
    for name in ("dq", "dk_raw", "dv_raw", "dk_cmp", "dv_cmp", "d_sink"):
        _close(name, got[name].cpu().numpy().astype(np.float64), refs[name], bound[name])
