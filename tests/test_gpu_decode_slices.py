"""GPU parity of the decode kernel that gives each workgroup one KV slice of
one query and 128 query heads (sink-free partials merged by the exact LSE
merge when there are several slices).  Each case is compared with the FP64
oracle; where the job-stream kernel also applies (heads_per_block 64) it is
checked too.  Slices are cut by list capacity and window capacity, so some
are empty when a query's counts are short, and split counts up to 64 leave
most of them empty."""
import numpy as np
import pytest

from sparse_paged_attention_amd import synth

from gpu_helpers import announce, check_against_oracle, need_gpu, run_hip

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()


def _decode(name, seq_lens, hq, hkv, page, window, ratio, topk, seed=51, **kw):
    return synth.make_problem(name, "decode", seq_lens, hq, hkv, 128, page, window, ratio, topk, seed=seed, **kw)


@pytest.mark.parametrize("splits", [2, 16])
def test_decode_csa_split_counts(splits):
    check_against_oracle(synth.make_workload("decode_csa"), num_splits=splits, label=f"decode_csa slices S{splits}")


def test_both_decode_kernels():
    p = _decode("both", [5000, 700, 64, 3000], 128, 1, 64, 128, 4, 512)
    for s in (1, 4):
        check_against_oracle(p, num_splits=s, label=f"slices S{s}")
        check_against_oracle(p, num_splits=s, heads_per_block=64, label=f"job streams S{s}")


def test_short_counts_and_many_splits():
    """Lists shorter than their capacity and contexts shorter than the
    window: the later slices are empty (LSE -inf, weight 0 in the merge)."""
    rng = np.random.default_rng(3)
    p = _decode("short", rng.integers(1, 300, size=12), 128, 1, 16, 128, 4, 200)
    for s in (1, 3, 64):
        check_against_oracle(p, num_splits=s, label=f"short counts S{s}")


def test_head_blocks():
    """160 heads per KV head (a full and a partial 128-head block) and 40
    heads over two KV heads (one partial block each)."""
    check_against_oracle(_decode("h160", [900, 333], 160, 1, 32, 100, 4, 64), num_splits=2, label="160 heads")
    check_against_oracle(_decode("h40x2", [900, 333, 12], 80, 2, 32, 100, 4, 64), num_splits=3, label="40 heads x 2")


def test_all_groups_layer():
    p = _decode("hca", [32768, 5000, 129], 128, 1, 128, 128, 128, 0)
    for s in (1, 4, 7):
        check_against_oracle(p, num_splits=s, label=f"all groups S{s}")


def test_window_only_and_empty():
    p = _decode("win", [5, 200, 1, 129], 128, 1, 16, 128, 0, 0)
    check_against_oracle(p, num_splits=2, label="window only")
    for with_sink in (True, False):
        q = _decode("empty", [10, 3], 64, 1, 16, 0, 0, 0, with_sink=with_sink)
        announce(f"empty sets, sink={with_sink}")
        O, L, _ = run_hip(q, 2)
        assert np.all(O == 0)
        if with_sink:
            assert np.allclose(L, np.broadcast_to(q.sink, L.shape), atol=1e-6)
        else:
            assert np.all(L == -np.inf)


@pytest.mark.parametrize("splits", [1, 4, 8])
def test_mixed_fp8_slices(splits):
    """The mixed FP8/BF16 workload: e4m3 compressed rows (per-row fp32
    scales) widened in LDS, then the bf16 window; both decode kernels."""
    p = synth.make_workload("mixed_fp8")
    check_against_oracle(p, num_splits=splits, label=f"mixed_fp8 slices S{splits}")
    check_against_oracle(p, num_splits=splits, heads_per_block=64, label=f"mixed_fp8 job streams S{splits}")


def test_fp8_partial_compressed_tiles():
    """e4m3 compressed rows that do not fill their last tile (the window
    starts at the next tile), short lists, split counts that leave slices
    with no compressed row, and 80 heads over two KV heads."""
    rng = np.random.default_rng(11)
    p = _decode("f8p", rng.integers(20, 900, size=7), 160, 2, 16, 45, 4, 37, cmp_fp8=True)
    for s in (1, 3, 11):
        check_against_oracle(p, num_splits=s, label=f"fp8 partial tiles S{s}")


@pytest.mark.parametrize("splits", [1, 4, 8])
def test_fnuz_pages_slices(splits):
    """FNUZ e4m3 compressed pages (bias 8, max 240), quantised with scale
    amax/240 so the 0x7F / 0xFF codes occur, read by the decode-slice
    kernel; unowned page rows hold the FNUZ NaN code 0x80."""
    p = synth.make_problem("fnuz", "decode", [3000, 1500, 700, 5000, 129], 128, 1, 128, 64, 128, 4, 512, seed=44,
                           cmp_fp8=True, fp8_format="fnuz", selection="random")
    assert np.any(p.k_cmp == 0x7F) and np.any(p.v_cmp == 0xFF)
    check_against_oracle(p, splits, label=f"fnuz S={splits}")


def test_fnuz_pages_refused_outside_the_slice_kernel():
    from sparse_paged_attention_amd import api, _lib
    p = synth.make_problem("fnuz_pre", "prefill", [600], 64, 1, 128, 16, 128, 4, 64, seed=45, cmp_fp8=True,
                           fp8_format="fnuz", query_positions=[(0, t) for t in range(590, 598)])
    dp = api.DeviceProblem.from_problem(p)
    with pytest.raises(_lib.SpaError) as e:
        api.forward(dp, 1)
    assert e.value.status == -4
