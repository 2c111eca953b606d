"""Host logic of bench.py, no GPU: the one-GPU contract, the kernel-name
mirror of the library's selection, the algorithmic byte and FLOP counts,
and the traffic file's validity rule."""
import json
import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from sparse_paged_attention_amd import synth  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_kernel_names_follow_the_selection():
    pre = synth.make_workload("prefill_csa")
    assert bench.attention_kernel(pre, 1, 0, 0) == "attn_pair_kernel<3>"
    assert bench.attention_kernel(pre, 1, 0, 1) == "attn_fwd_kernel"
    dec = synth.make_workload("decode_csa", batch=2)
    assert bench.attention_kernel(dec, 4, 0, 0) == "attn_decode_kernel<false>"
    assert bench.attention_kernel(dec, 4, 64, 0) == "attn_fwd_kernel"
    fp8 = synth.make_workload("mixed_fp8", batch=2)
    assert bench.attention_kernel(fp8, 8, 0, 0) == "attn_decode_kernel<true>"
    # one slice of 512 listed + 128 window rows: the one-pass decode kernel
    assert bench.attention_kernel(dec, 1, 0, 0) == "attn_decode_rows_kernel<false, true, false>"
    assert bench.attention_kernel(fp8, 1, 0, 0) == "attn_decode_rows_kernel<true, true, false>"
    # 64 queries: the 32-head workgroups fit once, not twice
    mid = synth.make_workload("decode_csa", batch=64)
    assert bench.attention_kernel(mid, 1, 0, 0, cus=256) == "attn_decode_rows_kernel<false, false, false>"
    # a batch whose 32-head workgroups exceed the CUs keeps the 128-head kernel
    big = synth.make_workload("decode_csa", batch=128)
    assert bench.attention_kernel(big, 1, 0, 0, cus=256) == "attn_decode_kernel<false>"
    fnuz = synth.make_problem("fnuz", "decode", [3000, 700], 128, 1, 128, 64, 128, 4, 512, seed=44, cmp_fp8=True,
                              fp8_format="fnuz")
    assert bench.attention_kernel(fnuz, 1, 0, 0) == "attn_decode_rows_kernel<true, true, true>"
    fp8_64 = synth.make_workload("mixed_fp8", batch=64)
    assert bench.attention_kernel(fp8_64, 1, 0, 0, cus=256) == "attn_decode_rows_kernel<true, false, false>"
    lat = synth.make_workload("decode_latent", batch=2)
    assert bench.attention_kernel(lat, 4, 0, 0) == "attn_latent_kernel<false>"


def _counts(p):
    """(win_lo, win_len, n_c, n_sel) per query, from the problem itself."""
    rows = []
    for i in range(p.num_queries):
        t = int(p.seq_lens[i]) - 1 if p.mode == "decode" else int(p.query_pos[i])
        lo = max(0, t - p.window + 1)
        n_c = (t + 1) // p.ratio if p.ratio else 0
        rows.append((lo, t - lo + 1, n_c, int(p.cmp_cnt[i]) if p.topk else n_c))
    return np.array(rows, dtype=np.int64)


def test_algorithmic_work_separate_and_shared_rows():
    dec = synth.make_workload("decode_csa", batch=2)
    b, f, n = bench.algorithmic_work(dec, _counts(dec))
    # Q + O bf16, LSE, 640 entries of K and V rows (2 x 128 x 2 B), 512 list ids
    assert b == 2 * (128 * 128 * 2 * 2 + 128 * 4 + 640 * 512 + 512 * 4)
    assert f == 4 * 128 * 128 * 2 * 640 and n == 1280
    fnuz = synth.make_problem("fnuz", "decode", [3000, 700], 128, 1, 128, 64, 128, 4, 512, seed=44, cmp_fp8=True,
                              fp8_format="fnuz")
    assert bench.attention_kernel(fnuz, 1, 0, 0) == "attn_decode_rows_kernel<true, true, true>"
    fp8_64 = synth.make_workload("mixed_fp8", batch=64)
    assert bench.attention_kernel(fp8_64, 1, 0, 0, cus=256) == "attn_decode_rows_kernel<true, false, false>"
    lat = synth.make_workload("decode_latent", batch=2)
    b2, _, _ = bench.algorithmic_work(lat, _counts(lat))
    # one shared 512-wide row per entry
    assert b2 == 2 * (64 * 512 * 2 * 2 + 64 * 4 + 640 * 1024 + 512 * 4)


def test_traffic_needs_matching_source_and_config(tmp_path, monkeypatch):
    f = tmp_path / "traffic.json"
    h = bench.kernel_source_hash()
    f.write_text(json.dumps({"decode_csa": {"kernel_source": h, "bytes_per_launch": 123.0,
                                            "config": {"batch": 32, "num_splits": 4, "heads_per_block": 0,
                                                       "queries_per_block": 0}}}))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    cfg = {"batch": 32, "num_splits": 4, "heads_per_block": 0, "queries_per_block": 0}
    assert bench.measured_traffic("decode_csa", cfg) == 123.0
    assert bench.measured_traffic("decode_csa", dict(cfg, num_splits=8)) is None
    assert bench.measured_traffic("prefill_csa", cfg) is None
    f.write_text(json.dumps({"decode_csa": {"kernel_source": "0" * 16, "bytes_per_launch": 1.0, "config": cfg}}))
    assert bench.measured_traffic("decode_csa", cfg) is None


def test_rotation_reads_every_replica_before_repeating():
    """The graphs of exactly `steps` calls cover every replica once per pass,
    for any --steps (the replica of call k is k % reps)."""
    for steps, reps in ((20, 51), (200, 51), (7, 7), (1, 3)):
        G = max(1, -(-reps // steps))
        seen = [(g * steps + k) % reps for g in range(G) for k in range(steps)]
        assert set(seen) == set(range(reps))
        first = seen[:reps]
        assert len(set(first)) == reps        # no replica read twice before all are read


def test_cpu_model_is_reported():
    assert isinstance(bench.cpu_model(), str) and bench.cpu_model()
