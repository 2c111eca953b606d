"""The no-allocation decode entry point (attn_fwd_decode_noalloc) against the
workspace one (attn_fwd_decode), both through the C ABI: the split partials
live in the library's per-GPU scratch array instead of a caller workspace,
the kernels are the same, so the outputs must be identical, and both match
the oracle.  Two calls in a row, the second with a smaller input, then a
one-slice call and an e4m3 one."""
import ctypes

import numpy as np
import pytest

import oracle
from oracle.compare import accept
from sparse_paged_attention_amd import synth

from gpu_helpers import announce, need_gpu, to_numpy_bf16, torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()


def _both(p, splits):
    from sparse_paged_attention_amd import _lib, api
    lib = _lib.load()
    dp = api.DeviceProblem.from_problem(p)
    announce(f"no-alloc decode {p.name}: batch {p.num_seqs} splits {splits}")
    O1, L1 = api.forward(dp, splits)
    args = dp.args(splits)
    O2 = torch.full_like(O1, float("nan"))
    L2 = torch.full_like(L1, float("nan"))
    args.o, args.lse = O2.data_ptr(), L2.data_ptr()
    args.workspace, args.workspace_bytes = None, 0
    _lib.check(lib.attn_fwd_decode_noalloc(ctypes.byref(args), torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()
    assert torch.equal(O1.view(torch.int16), O2.view(torch.int16))
    assert torch.equal(L1.view(torch.int32), L2.view(torch.int32))
    Oref, Lref = oracle.attention(p)
    rep = accept(to_numpy_bf16(O2), L2.cpu().numpy().astype(np.float64), Oref, Lref)
    assert rep.ok, rep


def test_two_calls_second_smaller():
    _both(synth.make_workload("decode_csa", batch=12), 4)
    _both(synth.make_workload("decode_csa", batch=3), 2)


def test_one_slice_and_e4m3():
    _both(synth.make_workload("decode_hca", batch=2), 1)
    _both(synth.make_workload("mixed_fp8", batch=5), 8)


def test_oversize_call_is_refused():
    from sparse_paged_attention_amd import _lib, api
    lib = _lib.load()
    p = synth.make_workload("decode_csa", batch=2)
    dp = api.DeviceProblem.from_problem(p)
    args = dp.args(64)
    args.num_q_heads = args.num_q_heads * 64      # 4 * 64 * 2 * 8192 * 129 bytes of partials
    out = torch.empty(1, device="cuda")
    args.o = out.data_ptr()
    st = lib.attn_fwd_decode_noalloc(ctypes.byref(args), torch.cuda.current_stream().cuda_stream)
    assert st == -6, st
    assert b"no-allocation scratch" in lib.attn_last_error()
