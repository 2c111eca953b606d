#!/usr/bin/env python3
"""Benchmark of the sparse paged attention forward on one MI355X.

One step = one call of the whole hot path (KV-set metadata, page-table
gather, scores, online softmax with the sink, PV, epilogue and, with split-KV,
the exact LSE merge) over one batch of synthetic input already resident in
HBM.  The default workload is "Decode CSA": batch 32, one query per sequence
at context 4096, 128 query heads sharing one KV head, D 128, bf16, page 64,
window 128 + top-k 512 of 1024 ratio-4 groups.

Inputs are replicated on the device and the steps rotate through the
replicas: every replica is read once before any is read again, whatever
--steps is, so the bytes read between two reads of the same replica exceed
--rotate-mb (640 MB; the memory-side cache is 256 MB) and the KV rows each
step reads are not resident in any cache.  The replicas are split into
graphs of exactly --steps calls each; each timed measurement is one replay of
one such graph, and the graphs are replayed in turn.

Prints one JSON line (see --help for options).
"""
import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, TFLOP/s
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
# the sources whose change invalidates counter-measured traffic
KERNEL_SOURCES = [os.path.join(ROOT, "sparse_paged_attention_amd", "csrc", f)
                  for f in ("spa_attention.hip", "spa_pair.hip", "spa_decode.hip", "spa_decode_rows.hip", "spa_latent.hip",
                            "spa_kernel_util.h", "spa_device.h", "spa_internal.h", "spa_api.cpp")]
# sources of the top-k and backward kernels (their traffic entries carry these hashes)
TOPK_SOURCES = [os.path.join(ROOT, "sparse_paged_attention_amd", "csrc", f)
                for f in ("spa_topk.hip", "spa_internal.h", "spa_api.cpp")]
BWD_SOURCES = [os.path.join(ROOT, "sparse_paged_attention_amd", "csrc", f)
               for f in ("spa_backward.hip", "spa_kernel_util.h", "spa_device.h", "spa_internal.h", "spa_api.cpp")]
PAIR_ROWS_MAX = 1280           # rows a query pair's union can hold in the prefill pair kernel
DECODE_ROWS_MAX = 1280         # rows of one decode slice in the decode kernel


def attention_kernel(p, splits, hpb, qpb, cus=256):
    """Name of the attention kernel the library launches for this call: the
    prefill pair kernel when the call fits it and the library's choice (or
    the caller's) is query pairs, else the one-query-per-job kernel.  Mirrors
    the selection in spa_api.cpp (for a decode the library sizes itself: the
    one-pass kernel with one slice, the slice kernel with several)."""
    if p.head_dim == 512:
        return "attn_latent_kernel<true>" if p.cmp_fp8 else "attn_latent_kernel<false>"
    pairs_ok = (p.mode == "prefill" and p.head_dim == 128 and not p.cmp_fp8 and splits == 1
                and (p.ratio == 0 or p.topk > 0) and 2 * (p.topk + p.window) <= PAIR_ROWS_MAX)
    pairs = pairs_ok and (qpb == 2 or (qpb == 0 and hpb != 32))
    S = max(splits, 1)
    cap = 0 if p.ratio == 0 else p.topk if p.topk > 0 else p.cmp_pt.shape[1] * p.page_size
    cper = -(-cap // S)
    if p.cmp_fp8:
        cper = -(-cper // 32) * 32          # e4m3 rows fill whole tiles
    decode_ok = (p.mode == "decode" and p.head_dim == 128 and hpb == 0 and qpb == 0 and S <= 64
                 and cper + -(-p.window // S) <= DECODE_ROWS_MAX)
    if pairs:
        return "attn_pair_kernel<3>"
    rows_wgs = p.num_queries * p.num_kv_heads * -(-(p.num_q_heads // p.num_kv_heads) // 32)
    if decode_ok and S == 1 and rows_wgs <= cus:
        # room for twice the workgroups: each forms half of O's dimensions
        b = lambda x: "true" if x else "false"
        return (f"attn_decode_rows_kernel<{b(p.cmp_fp8)}, {b(2 * rows_wgs <= cus)}, "
                f"{b(p.cmp_fp8 and p.cmp_fp8_fnuz)}>")
    if decode_ok:
        return "attn_decode_kernel<true>" if p.cmp_fp8 else "attn_decode_kernel<false>"
    return "attn_fwd_kernel"



def kernel_source_hash(files=None):
    import hashlib
    h = hashlib.sha256()
    for f in (KERNEL_SOURCES if files is None else files):
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(workload, cfg, files=None, keys=("batch", "num_splits", "heads_per_block", "queries_per_block")):
    """HBM bytes per attention launch from the committed counter runs
    (FETCH_SIZE + WRITE_SIZE, scaled by the copy-kernel calibration), or
    None when none matches this workload, launch configuration and kernel
    source."""
    try:
        with open(TRAFFIC_FILE) as fh:
            data = json.load(fh)
    except (OSError, ValueError):
        return None
    e = data.get(workload)
    if not e or e.get("kernel_source") != kernel_source_hash(files):
        return None
    if any(e.get("config", {}).get(k) != cfg.get(k) for k in keys):
        return None
    return e.get("bytes_per_launch")


def copy_calibration(mib, steps):
    """A plain device-to-device copy of `mib` MiB, `steps` times: the known
    reference (mib MiB read and written per launch) for the FETCH_SIZE and
    WRITE_SIZE counters."""
    import torch
    n = int(mib * (1 << 20))
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    return {"copy_mib": mib, "launches": steps, "ms_per_copy": ms, "gbs_read_plus_write": 2 * n / (ms / 1e3) / 1e9}


def algorithmic_work(p, counts):
    """Bytes and FLOPs the method must move / compute for one call.

    Per query: Q and O (bf16), LSE (fp32), every KV entry of its set once
    (K and V rows, one row for a shared latent cache, plus the fp32 per-token
    scales for e4m3 rows) and the list
    indices; FLOPs = 4 * Hq * D * |KV set|.  Page-table reads, split
    partials and masked work are overhead and not counted."""
    Hq, Hkv, D = p.num_q_heads, p.num_kv_heads, p.head_dim
    sides = 1 if p.v_raw is p.k_raw else 2       # a shared latent row is K and V
    raw_entry = Hkv * sides * D * 2
    cmp_entry = Hkv * sides * D * (1 if p.cmp_fp8 else 2) + (Hkv * 2 * 4 if p.cmp_fp8 else 0)
    win_len = counts[:, 1].astype("int64")
    n_sel = counts[:, 3].astype("int64")
    nq = counts.shape[0]
    kv_bytes = int((win_len * raw_entry).sum() + (n_sel * cmp_entry).sum())
    idx_bytes = int(n_sel.sum() * 4) if p.topk > 0 else 0
    qo_bytes = nq * Hq * D * 2 * 2 + nq * Hq * 4
    flops = int(4 * Hq * D * (win_len + n_sel).sum())
    return kv_bytes + idx_bytes + qo_bytes, flops, int((win_len + n_sel).sum())


def cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(p, budget_s):
    """Time the FP64 oracle on the host over a bounded sample: one process,
    its BLAS limited to one thread, so `cores` is what it used."""
    import oracle
    from threadpoolctl import threadpool_limits
    nq = p.num_queries
    done = 0
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        while time.perf_counter() - t0 <= budget_s:
            oracle.attention(p, [done % nq])
            done += 1
        dt = time.perf_counter() - t0
    return {"value": done / dt, "unit": "queries/s", "cores": 1, "kind": "oracle",
            "cpu": cpu_model(), "host_cpus": len(os.sched_getaffinity(0)),
            "sample": f"{done} queries of the same workload (query i % {nq}), {dt:.1f} s, one process, "
                      f"numpy fp64 with one BLAS thread"}


def parse_args(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="decode_csa",
                    choices=["decode_csa", "decode_hca", "mixed_fp8", "prefill_csa", "tiny", "decode_latent",
                             "topk_decode", "topk_prefill", "bwd_prefill_csa"])
    ap.add_argument("--batch", type=int, default=0, help="decode batch override (0 = the workload's)")
    ap.add_argument("--topk-order", default="score", choices=["score", "id"],
                    help="top-k workloads: ids by descending score (attn_topk_select) or by id "
                         "(attn_topk_select_ids)")
    ap.add_argument("--context", type=int, default=0,
                    help="decode sequence length for every query (0 = the workload's); a sweep of the KV-set size")
    ap.add_argument("--splits", type=int, default=0, help="0 = the default for the workload")
    ap.add_argument("--heads-per-block", type=int, default=-1,
                    help="query heads per workgroup (32/64/128, 0 = library choice, -1 = workload default)")
    ap.add_argument("--queries-per-block", type=int, default=-1,
                    help="queries per workgroup (1/2/4, 0 = library choice, -1 = workload default)")
    ap.add_argument("--rotate-mb", type=float, default=640.0,
                    help="total size of the input replicas the timed steps rotate through")
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle timing (0 = skip)")
    ap.add_argument("--eager-only", action="store_true",
                    help="time host-launched calls only (no graph capture), e.g. under counter collection")
    ap.add_argument("--copy-mib", type=float, default=0.0,
                    help="instead of the attention: time a plain device copy of this many MiB "
                         "(the reference for the traffic counters)")
    return ap.parse_args(argv)


DEFAULTS = {   # (num_splits, heads_per_block, queries_per_block) per workload; 0 = library choice
    "decode_csa": (1, 0, 0), "decode_hca": (1, 0, 0), "mixed_fp8": (1, 0, 0), "prefill_csa": (1, 0, 0),
    "tiny": (1, 0, 0), "decode_latent": (5, 0, 0),
}


def eager_ms(launch, n):
    """Per-launch time of `n` host launches of `launch(stream, k)` (HIP
    events on the current stream); also the per-launch mean as an array."""
    import numpy as np
    import torch
    s = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(s)
    for k in range(n):
        launch(s.cuda_stream, k)
    e1.record(s)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / n
    return ms, np.array([ms])


def graph_replay_ms(launch, steps, reps=1, rounds=2, warm_s=0.3):
    """Per-call time of `launch(stream, k)` from HIP graph replays.

    Call k uses replica k % reps.  The calls are captured in G = ceil(reps /
    steps) graphs of exactly `steps` calls (graph g holds calls g*steps ..
    g*steps + steps - 1), so replaying the graphs in turn reads every replica
    once before any is read again.  The graphs are replayed in turn, untimed,
    until at least `warm_s` seconds have passed (one pass at least), so that
    the chip's clocks have settled whatever `steps` is: short passes timed
    right after the warm-up steps ran up to 17% slower per call on prefill.
    Then each measurement is one replay of one graph (HIP events on the
    capture stream); `rounds` passes over the G graphs.  Returns (median ms
    per call, per-measurement ms per call, G)."""
    import numpy as np
    import torch
    G = max(1, -(-reps // steps))
    cap_stream = torch.cuda.Stream()
    graphs = []
    with torch.cuda.stream(cap_stream):
        for k in range(3):
            launch(cap_stream.cuda_stream, k)
        cap_stream.synchronize()
        for g in range(G):
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph, stream=cap_stream):
                cs = torch.cuda.current_stream()
                for k in range(steps):
                    launch(cs.cuda_stream, g * steps + k)
            graphs.append(graph)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        while True:
            for graph in graphs:
                graph.replay()
            torch.cuda.synchronize()
            if time.perf_counter() - t0 >= warm_s:
                break
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * G * rounds)]
        n = 0
        for _ in range(rounds):
            for graph in graphs:
                ev[n].record(cap_stream)
                graph.replay()
                ev[n + 1].record(cap_stream)
                n += 2
        torch.cuda.synchronize()
    per = np.array([ev[2 * m].elapsed_time(ev[2 * m + 1]) / steps for m in range(G * rounds)])
    return float(np.median(per)), per, G


def run(workload, *, steps=200, warmup=20, splits=0, heads_per_block=-1, queries_per_block=-1,
        rotate_mb=640.0, batch=0, cpu_budget=0.0, problem=None, eager_only=False, context=0):
    """Time `steps` calls of the hot path; returns the result dict."""
    import ctypes

    import numpy as np
    import torch
    from sparse_paged_attention_amd import api, synth, _lib

    lib = _lib.load()
    dev = torch.device("cuda:0")
    p = problem if problem is not None else synth.make_workload(workload, batch=batch or None, context=context or None)
    d_splits, d_hpb, d_qpb = DEFAULTS.get(workload, (1, 0, 0))
    splits = splits or d_splits
    hpb = d_hpb if heads_per_block < 0 else heads_per_block
    qpb = d_qpb if queries_per_block < 0 else queries_per_block
    base = api.DeviceProblem.from_problem(p, device=dev)

    # metadata from the library itself, for the byte/FLOP accounting
    cap = p.window + (p.topk if p.topk else max(int(n) // max(p.ratio, 1) for n in p.seq_lens)) + 1
    _, counts = api.build_gather(base, cap)
    counts = counts.cpu().numpy()
    alg_bytes, alg_flops, kv_entries = algorithmic_work(p, counts)

    # replicas: the KV rows read per step plus Q/O, rotated so the set is HBM-cold
    reps = max(1, math.ceil(rotate_mb * 1e6 / max(alg_bytes, 1)))
    pools = {id(t): t for t in (base.k_raw, base.v_raw, base.k_cmp, base.v_cmp) if t is not None}
    pool_bytes = sum(t.numel() * t.element_size() for t in pools.values())
    reps = min(reps, max(1, int(48e9 // max(pool_bytes, 1))))
    replicas = []

    def clone_problem():
        # one clone per distinct tensor, so a shared latent cache stays shared
        memo = {}
        return api.DeviceProblem(**{k: (memo.setdefault(id(v), v.clone()) if isinstance(v, torch.Tensor) else v)
                                    for k, v in base.__dict__.items()})

    for r in range(reps):
        dp = base if r == 0 else clone_problem()
        a = dp.args(splits, hpb, qpb)
        o = torch.empty((p.num_queries, p.num_q_heads, p.head_dim), dtype=torch.bfloat16, device=dev)
        lse = torch.empty((p.num_queries, p.num_q_heads), dtype=torch.float32, device=dev)
        need = api.workspace_size(a)
        ws = torch.empty(max(need, 16), dtype=torch.uint8, device=dev) if need else None
        a.o = o.data_ptr()
        a.lse = lse.data_ptr()
        a.workspace = ws.data_ptr() if ws is not None else None
        a.workspace_bytes = ws.numel() if ws is not None else 0
        replicas.append((dp, a, o, lse, ws))
    fn = lib.attn_fwd_decode if p.mode == "decode" else lib.attn_fwd_prefill
    stream = torch.cuda.current_stream().cuda_stream
    prepared = [ctypes.byref(r[1]) for r in replicas]

    def step(k):
        st = fn(prepared[k % reps], stream)
        if st != 0:
            _lib.check(st)

    for k in range(warmup):
        step(k)
    torch.cuda.synchronize()

    # eager: host launches back to back (includes the Python + HIP launch cost)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t_wall0 = time.perf_counter()
    e0.record()
    for k in range(steps):
        step(k)
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall0
    eager_ms = e0.elapsed_time(e1) / steps

    def fwd_launch(s, k):
        st = fn(prepared[k % reps], s)
        if st != 0:
            _lib.check(st)

    kernel = attention_kernel(p, splits, hpb, qpb, torch.cuda.get_device_properties(0).multi_processor_count)
    n_graphs = 1
    if eager_only:
        ms_per_step, per = eager_ms, np.array([eager_ms])
        merge_ms = 0.0
    else:
        # the whole call: attention (+ the LSE merge when split)
        ms_per_step, per, n_graphs = graph_replay_ms(fwd_launch, steps, reps)
        # the merge kernel of a split call, timed alone through attn_merge_lse
        # on the partials each call left in its replica's workspace, so that
        # the attention kernel's own duration is the difference
        merge_ms = 0.0
        if splits > 1:
            rows = p.num_queries * p.num_q_heads
            lse_off = ((rows * p.head_dim * 4 * splits) + 255) // 256 * 256
            sink_ptr = base.sink.data_ptr() if base.sink is not None else None

            def merge_launch(s, k):
                _, a, o, lse, ws = replicas[k % reps]
                st = lib.attn_merge_lse(ws.data_ptr(), ws.data_ptr() + lse_off, splits, rows, p.head_dim,
                                        p.num_q_heads, sink_ptr, o.data_ptr(), lse.data_ptr(), s)
                if st != 0:
                    _lib.check(st)

            merge_ms, _, _ = graph_replay_ms(merge_launch, steps, reps)
    kernel_ms = ms_per_step - merge_ms

    nq = p.num_queries
    decode = p.mode == "decode"
    # the roofline of the whole call (attention, plus a separate merge kernel
    # where there is one); the attention kernel alone beside it
    if decode:
        roof = {"bound": "hbm", "achieved": alg_bytes / (ms_per_step / 1e3) / 1e9, "peak": HBM_PEAK_GBS,
                "unit": "GB/s"}
        kernel_achieved = alg_bytes / (kernel_ms / 1e3) / 1e9
    else:
        roof = {"bound": "mfma", "achieved": alg_flops / (ms_per_step / 1e3) / 1e12, "peak": BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s"}
        kernel_achieved = alg_flops / (kernel_ms / 1e3) / 1e12
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = None   # filled in below from the committed counter runs, if they match
    roof["kernel"] = kernel
    roof["launches_per_call"] = 2 if merge_ms > 0 else 1
    roof["kernel_ms"] = kernel_ms
    roof["kernel_ms_how"] = ("graph replay of the call minus graph replay of the merge alone" if merge_ms > 0
                             else "graph replay of the call (one kernel)")
    roof["kernel_achieved"] = kernel_achieved
    roof["kernel_frac"] = kernel_achieved / roof["peak"]
    roof["algorithmic_bytes_per_launch"] = alg_bytes
    roof["algorithmic_flops_per_launch"] = alg_flops

    out = {
        "metric": "decode queries/s + HBM GB/s; prefill TFLOP/s (frac. of MI355X peak)",
        "value": nq / (ms_per_step / 1e3),
        "unit": "queries/s" if decode else "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if not p.cmp_fp8 else "bf16+e4m3",
        "data": "synthetic",
        "config": {"workload": workload, "batch": p.num_seqs, "queries": nq,
                   "q_heads": p.num_q_heads, "kv_heads": p.num_kv_heads, "head_dim": p.head_dim,
                   "page_size": p.page_size, "window": p.window, "ratio": p.ratio, "topk": p.topk,
                   "kv_entries": kv_entries, "num_splits": splits, "heads_per_block": hpb,
                   "queries_per_block": qpb,
                   "replicas": reps, "rotated_mb": round(reps * alg_bytes / 1e6, 1), "graphs": n_graphs}
                  | ({"context": context} if context else {}),
        "roofline": roof,
        "cpu_baseline": cpu_baseline(p, cpu_budget) if cpu_budget > 0 else None,
        "timing": {"graph_replay_ms_per_step_min": float(per.min()),
                   "graph_replay_ms_per_step_max": float(per.max()),
                   "graph_replay_ms_per_step_p10": float(np.percentile(per, 10)),
                   "graph_replay_ms_per_step_p90": float(np.percentile(per, 90)),
                   "measurements": int(per.size),
                   "eager_ms_per_step": eager_ms,
                   "merge_ms": merge_ms,
                   "host_wall_ms_per_step": wall / steps * 1e3,
                   "tflops": alg_flops / (ms_per_step / 1e3) / 1e12,
                   "gbs_step": alg_bytes / (ms_per_step / 1e3) / 1e9},
    }
    out["roofline"]["traffic"] = None if context else measured_traffic(workload, out["config"])
    return out


TOPK_SHAPES = {   # rows, per-row counts (complete ratio-4 groups), k
    "topk_decode": "32 rows of 1024 complete groups (decode CSA, context 4096), k 512",
    "topk_prefill": "2560 rows, row t holding floor((t+1)/4) complete groups (prefill CSA), k 512",
}


def run_topk(workload, *, steps=200, warmup=20, cpu_budget=0.0, eager_only=False, order="score"):
    """Time attn_topk_select (order "score") or attn_topk_select_ids (order
    "id") on scores over the complete groups of the decode CSA or prefill
    CSA workload (seeded N(0,1) scores; the pages do not define the
    indexer's scoring).  One step = one call."""
    import numpy as np
    import torch
    from sparse_paged_attention_amd import api, _lib

    _lib.load()
    rng = np.random.default_rng(7)
    k = 512
    if workload == "topk_decode":
        n_valid = np.full(32, 1024, dtype=np.int32)
    else:
        n_valid = np.array([(t + 1) // 4 for t in range(2560)], dtype=np.int32)
    ld = int(n_valid.max())
    scores_h = rng.standard_normal((len(n_valid), ld)).astype(np.float32)
    rows = len(n_valid)
    # replicas rotated through so the scores are not L2-resident
    reps = max(1, int(64e6 // scores_h.nbytes))
    sc = [torch.from_numpy(scores_h).cuda() for _ in range(reps)]
    nv = torch.from_numpy(n_valid).cuda()
    lib = _lib.load()
    ids = torch.empty((rows, k), dtype=torch.int32, device="cuda")
    cnt = torch.empty(rows, dtype=torch.int32, device="cuda")

    by_id = order == "id"
    fn = lib.attn_topk_select_ids if by_id else lib.attn_topk_select

    def launch(stream, r):
        _lib.check(fn(sc[r % reps].data_ptr(), ld, nv.data_ptr(), rows, k, ids.data_ptr(), cnt.data_ptr(), stream))

    for r in range(warmup):
        api.topk_select(sc[r % reps], nv, k, by_id=by_id)
    torch.cuda.synchronize()
    ms, per = eager_ms(launch, steps) if eager_only else graph_replay_ms(launch, steps, reps)[:2]
    read_b = int(n_valid.sum()) * 4 + rows * 4
    write_b = rows * k * 4 + rows * 4
    achieved = (read_b + write_b) / (ms / 1e3) / 1e9
    cpu = None
    if cpu_budget > 0:
        import oracle
        t0 = time.perf_counter()
        done = 0
        while time.perf_counter() - t0 < cpu_budget:
            i = done % rows
            oracle.topk_select(scores_h[i:i + 1], n_valid[i:i + 1], k, by_id=by_id)
            done += 1
        dt = time.perf_counter() - t0
        cpu = {"value": done / dt, "unit": "rows/s", "cores": 1, "kind": "oracle",
               "sample": f"{done} rows of the same scores, {dt:.1f} s, numpy"}
    return {
        "metric": "top-k selection rows/s (the step before the attention core)",
        "value": rows / (ms / 1e3), "unit": "rows/s", "n_gpus": 1, "steps": steps, "warmup": warmup,
        "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": workload, "shape": TOPK_SHAPES[workload], "rows": rows, "k": k, "order": order,
                   "replicas": reps},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": None, "kernel": "topk_kernel",
                     "kernel_ms": ms, "kernel_ms_how": ("host-launched calls" if eager_only
                                                        else "graph replay of the step (one kernel)"),
                     "algorithmic_bytes_per_launch": read_b + write_b},
        "cpu_baseline": cpu,
    } | {"_traffic": measured_traffic(workload if order == "score" else f"{workload}.id",
                                      {"rows": rows, "k": k, "order": order}, TOPK_SOURCES, ("rows", "k", "order"))}


def run_backward(workload, *, steps=20, warmup=3, cpu_budget=0.0, rotate_mb=640.0, eager_only=False):
    """Time attn_bwd on the prefill CSA workload: one step = one backward call
    (the attention kernel's gradients plus the fixed-order sink reduction)
    from the forward's own O and LSE, with a seeded N(0,1) bf16 upstream
    gradient.  The gradient caches accumulate across steps (zeroing them is
    the caller's and is not timed)."""
    import ctypes
    import dataclasses

    import numpy as np
    import torch
    from sparse_paged_attention_amd import api, synth, _lib

    lib = _lib.load()
    p = synth.make_workload(workload.replace("bwd_", ""))
    base = api.DeviceProblem.from_problem(p)
    cap = p.window + p.topk + 1
    _, counts = api.build_gather(base, cap)
    counts = counts.cpu().numpy()
    _, fwd_flops, kv_entries = algorithmic_work(p, counts)
    alg_flops = fwd_flops // 4 * 10          # S, dP, dQ, dK, dV: 2 Hq D flops each per (query, entry)
    nq, Hq, D = p.num_queries, p.num_q_heads, p.head_dim
    rng = np.random.default_rng(5)
    dO_bits = synth.f32_to_bf16_bits(rng.standard_normal(p.q.shape).astype(np.float32))
    per_rep = nq * Hq * D * (2 * 3 + 4) + nq * Hq * 8   # q, dO, O (bf16), dq (f32), lse, sink parts
    reps = max(1, math.ceil(rotate_mb * 1e6 / per_rep))
    sets = []
    g = {
        "dk_raw": torch.zeros(base.k_raw.shape, dtype=torch.float32, device="cuda"),
        "dv_raw": torch.zeros(base.v_raw.shape, dtype=torch.float32, device="cuda"),
        "dk_cmp": torch.zeros(base.k_cmp.shape, dtype=torch.float32, device="cuda"),
        "dv_cmp": torch.zeros(base.v_cmp.shape, dtype=torch.float32, device="cuda"),
        "d_sink": torch.zeros(Hq, dtype=torch.float32, device="cuda"),
    }
    for r in range(reps):
        dp = dataclasses.replace(base, q=base.q.clone())
        o, lse = api.forward(dp)
        d_o = torch.from_numpy(dO_bits.view(np.int16)).cuda().view(torch.bfloat16)
        args = dp.args(1)
        args.o, args.lse = o.data_ptr(), lse.data_ptr()
        need = int(lib.attn_bwd_workspace_size(ctypes.byref(args)))
        kv_path = need > nq * Hq * 4
        ws = torch.empty(need, dtype=torch.uint8, device="cuda")
        args.workspace, args.workspace_bytes = ws.data_ptr(), ws.numel()
        dq = torch.empty(p.q.shape, dtype=torch.float32, device="cuda")
        gr = _lib.SpaBwdGrads()
        gr.d_o, gr.dq = d_o.data_ptr(), dq.data_ptr()
        for name in ("dk_raw", "dv_raw", "dk_cmp", "dv_cmp", "d_sink"):
            setattr(gr, name, g[name].data_ptr())
        sets.append((args, gr, (dp, o, lse, d_o, ws, dq)))
    torch.cuda.synchronize()

    def launch(stream, k):
        a, gr, _ = sets[k % reps]
        _lib.check(lib.attn_bwd(ctypes.byref(a), ctypes.byref(gr), stream))

    for k in range(warmup):
        launch(torch.cuda.current_stream().cuda_stream, k)
    torch.cuda.synchronize()
    ms, per = eager_ms(launch, steps) if eager_only else graph_replay_ms(launch, steps, reps)[:2]
    achieved = alg_flops / (ms / 1e3) / 1e12
    cpu = None
    if cpu_budget > 0:
        import oracle
        from oracle.backward import attention_backward
        t0 = time.perf_counter()
        done = 0
        stride = 37                       # a spread of positions, short and long sets
        while time.perf_counter() - t0 < cpu_budget:
            i = (done * stride) % nq
            sub = dataclasses.replace(p, q=p.q[[i]], query_seq=p.query_seq[[i]], query_pos=p.query_pos[[i]],
                                      cmp_idx=p.cmp_idx[[i]], cmp_cnt=p.cmp_cnt[[i]])
            attention_backward(sub, dO_bits[[i]])
            done += 1
        dt = time.perf_counter() - t0
        cpu = {"value": done / dt, "unit": "tokens/s", "cores": 1, "kind": "oracle",
               "sample": f"{done} query tokens of the workload (every 37th position), {dt:.1f} s, numpy fp64"}
    return {
        "metric": "backward tokens/s (dq, dk, dv, dsink from O and LSE)",
        "value": nq / (ms / 1e3), "unit": "tokens/s", "n_gpus": 1, "steps": steps, "warmup": warmup,
        "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": workload, "queries": nq, "q_heads": Hq, "kv_heads": p.num_kv_heads, "head_dim": D,
                   "window": p.window, "ratio": p.ratio, "topk": p.topk, "kv_entries": kv_entries,
                   "replicas": reps},
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved / BF16_PEAK_TFLOPS, "traffic": None,
                     "kernel": "attn_bwd_kernel<2, false> + attn_bwd_kv_kernel" if kv_path else "attn_bwd_kernel<2, true>",
                     "kernel_ms": ms, "kernel_ms_how": ("host-launched calls" if eager_only else
                                                        "graph replay of the step (every kernel of the call)"),
                     "algorithmic_flops_per_launch": alg_flops},
        "cpu_baseline": cpu,
        "timing": {"graph_replay_ms_per_step_min": float(per.min()), "graph_replay_ms_per_step_max": float(per.max())},
    } | {"_traffic": measured_traffic(workload, {"queries": nq}, BWD_SOURCES, ("queries",))}


def main():
    args = parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the library has no "
              f"multi-GPU path", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    if args.copy_mib > 0:
        print(json.dumps(copy_calibration(args.copy_mib, args.steps)), flush=True)
        return
    if args.workload.startswith("bwd_"):
        out = run_backward(args.workload, steps=min(args.steps, 50), warmup=min(args.warmup, 5),
                           cpu_budget=args.cpu_budget, eager_only=args.eager_only)
        out["roofline"]["traffic"] = out.pop("_traffic")
        print(json.dumps(out), flush=True)
        return
    if args.workload.startswith("topk_"):
        out = run_topk(args.workload, steps=args.steps, warmup=args.warmup, cpu_budget=args.cpu_budget,
                       eager_only=args.eager_only, order=args.topk_order)
        out["roofline"]["traffic"] = out.pop("_traffic")
        print(json.dumps(out), flush=True)
        return
    out = run(args.workload, steps=args.steps, warmup=args.warmup, splits=args.splits,
              heads_per_block=args.heads_per_block, queries_per_block=args.queries_per_block, rotate_mb=args.rotate_mb, batch=args.batch,
              cpu_budget=args.cpu_budget, eager_only=args.eager_only, context=args.context)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
