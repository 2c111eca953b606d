"""Shared helpers for the GPU parity tests (HIP path vs the FP64 oracle)."""
import sys

import numpy as np
import pytest

import oracle
from oracle.compare import accept

torch = pytest.importorskip("torch")


def need_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU test run without a GPU")
    from sparse_paged_attention_amd import _lib
    _lib.load()


def announce(msg):
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def to_numpy_bf16(t):
    return t.float().cpu().numpy().astype(np.float64)


def run_hip(p, num_splits=None, err_flag=None, heads_per_block=0, queries_per_block=0):
    from sparse_paged_attention_amd import api
    dp = api.DeviceProblem.from_problem(p)
    O, L = api.forward(dp, num_splits, err_flag=err_flag, heads_per_block=heads_per_block,
                       queries_per_block=queries_per_block)
    torch.cuda.synchronize()
    return to_numpy_bf16(O), L.cpu().numpy().astype(np.float64), dp


def check_against_oracle(p, num_splits=None, queries=None, label="", heads_per_block=0,
                         queries_per_block=0):
    announce(f"{label or p.name}: Nq={p.num_queries} Hq={p.num_q_heads} D={p.head_dim} "
             f"splits={num_splits or p.num_splits} hpb={heads_per_block} qpb={queries_per_block}")
    O, L, _ = run_hip(p, num_splits, heads_per_block=heads_per_block, queries_per_block=queries_per_block)
    Oref, Lref = oracle.attention(p, queries)
    if queries is not None:
        O, L = O[queries], L[queries]
    rep = accept(O, L, Oref, Lref)
    assert rep.ok, f"{label or p.name}: {rep}"
    return rep, O, L
