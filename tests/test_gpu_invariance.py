"""Bitwise batch and chunk invariance: a query's O and LSE do not depend on
which other queries share its call.

* Decode (fixed split count): a query's slices, tiles and the merge, or
  with one slice the one-pass kernel's waves, read only its own rows, so
  any batch that contains it gives the same bits as long as the same kernel
  serves both calls.  With one slice the library takes the one-pass kernel
  only while its workgroups fit the chip, so bits may change where a batch
  crosses that size; a caller who needs them fixed passes two or more
  slices.
* Prefill with one query per job (queries_per_block 1): a chunked prefill
  gives the same bits as one call over all its queries.
* Prefill with query pairs (the library's default) streams the union of two
  queries' sets, so a query's tiles, and with them the rounding of its
  online softmax, depend on its partner: chunking may change bits, never
  the result beyond rounding (checked against the oracle).
"""
import dataclasses

import numpy as np
import pytest

import oracle
from oracle.compare import accept
from sparse_paged_attention_amd import synth

from gpu_helpers import announce, need_gpu, run_hip

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()


def _decode_subset(p, idx):
    idx = np.asarray(idx)
    return dataclasses.replace(
        p, num_seqs=len(idx), q=p.q[idx], seq_lens=p.seq_lens[idx], raw_pt=p.raw_pt[idx],
        cmp_pt=p.cmp_pt[idx], query_seq=np.arange(len(idx), dtype=np.int32), query_pos=p.query_pos[idx],
        cmp_idx=p.cmp_idx[idx], cmp_cnt=p.cmp_cnt[idx], k_raw_logical=None, v_raw_logical=None,
        k_cmp_logical=None, v_cmp_logical=None, k_cmp_scale_logical=None, v_cmp_scale_logical=None)


def _prefill_subset(p, idx):
    idx = np.asarray(idx)
    return dataclasses.replace(
        p, q=p.q[idx], query_seq=p.query_seq[idx], query_pos=p.query_pos[idx], cmp_idx=p.cmp_idx[idx],
        cmp_cnt=p.cmp_cnt[idx])


@pytest.mark.parametrize("hpb", [0, 64])
def test_decode_batch_invariance(hpb):
    p = synth.make_workload("decode_csa")
    announce(f"decode batch invariance hpb={hpb}")
    O, L, _ = run_hip(p, 4, heads_per_block=hpb)
    for idx in ([31, 7, 2, 19, 0, 11, 25, 3], list(range(0, 32, 3)), [5]):
        Os, Ls, _ = run_hip(_decode_subset(p, idx), 4, heads_per_block=hpb)
        assert np.array_equal(Os, O[idx]) and np.array_equal(Ls, L[idx]), idx


def test_decode_one_pass_batch_invariance():
    p = synth.make_workload("decode_csa")
    announce("decode batch invariance, one pass")
    O, L, _ = run_hip(p, 1)
    for idx in ([31, 7, 2, 19, 0, 11, 25, 3], list(range(1, 32, 5)), [30]):
        Os, Ls, _ = run_hip(_decode_subset(p, idx), 1)
        assert np.array_equal(Os, O[idx]) and np.array_equal(Ls, L[idx]), idx


def test_decode_fp8_batch_invariance():
    p = synth.make_workload("mixed_fp8")
    announce("fp8 decode batch invariance")
    O, L, _ = run_hip(p, 8)
    idx = [15, 3, 8, 0]
    Os, Ls, _ = run_hip(_decode_subset(p, idx), 8)
    assert np.array_equal(Os, O[idx]) and np.array_equal(Ls, L[idx])


def test_prefill_chunk_invariance_one_query_per_job():
    p = synth.make_problem("chunks", "prefill", [1500], 64, 1, 128, 16, 128, 4, 256, seed=61,
                           query_positions=[(0, t) for t in range(1400, 1500)], selection="score")
    announce("prefill chunk invariance, one query per job")
    O, L, _ = run_hip(p, 1, queries_per_block=1)
    for chunk in (list(range(0, 37)), list(range(37, 100)), list(range(1, 100, 2)), [99, 0, 50]):
        Oc, Lc, _ = run_hip(_prefill_subset(p, chunk), 1, queries_per_block=1)
        assert np.array_equal(Oc, O[chunk]) and np.array_equal(Lc, L[chunk]), chunk[:4]


def test_prefill_pairs_chunked_within_tolerance():
    """Query pairs: chunking changes the pairing (every query with an odd
    offset), so bits may change; the result still matches the oracle."""
    p = synth.make_problem("chunks2", "prefill", [1500], 64, 1, 128, 16, 128, 4, 256, seed=62,
                           query_positions=[(0, t) for t in range(1400, 1460)], selection="score")
    announce("prefill pairs, chunked")
    for chunk in (list(range(1, 60)), list(range(0, 60, 3))):
        q = _prefill_subset(p, chunk)
        Oc, Lc, _ = run_hip(q, 1, queries_per_block=2)
        Oref, Lref = oracle.attention(q)
        rep = accept(Oc, Lc, Oref, Lref)
        assert rep.ok, rep
