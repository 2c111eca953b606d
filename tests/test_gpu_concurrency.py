"""Graph capture and concurrency through the C ABI.

RL-Kernel PR "Roadmap item 24", section "MI300X validation", runs the joint
attention under a real HIP graph, on two streams and from concurrent host
threads; "Fixed paged CK attention on ROCm" compares bits across graph
replays.  Here:
  * calls captured in a HIP graph (torch.cuda.CUDAGraph) and replayed
    several times, with eager work and synchronisations between the replays,
    reproduce the eager call's bits on every replay (the decode kernel with
    the LSE merge, the prefill pair kernel, the top-k selection);
  * two host threads, each with its own stream, inputs, outputs and
    workspaces, launching in turn as fast as they can, reproduce the bits of
    the same calls made one after the other on one stream."""
import threading

import numpy as np
import pytest

from sparse_paged_attention_amd import synth

from gpu_helpers import announce, need_gpu, torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()


def _small_prefill(seed):
    return synth.make_problem("graph_prefill", "prefill", [300, 200], 64, 1, 128, 16, 64, 4, 32, seed=seed,
                              query_positions=[(0, t) for t in range(250, 270)] + [(1, t) for t in (0, 7, 199)],
                              selection="score")


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def _capture_and_replay(label, run, outs, side_work):
    """Eager run (reference bits), then capture `run` into a graph and replay
    it three times, clearing the outputs eagerly before each replay and
    doing other eager work in between; every replay must give the eager bits."""
    run()
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs]
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        run()                                    # warm on the capture stream
        s.synchronize()
        with torch.cuda.graph(g, stream=s):
            run()
    torch.cuda.synchronize()
    for r in range(3):
        for o in outs:
            o.zero_()
        side_work()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, x in zip(outs, ref):
            assert torch.equal(_bits(o), _bits(x)), f"{label}: replay {r} differs from the eager call"
    announce(f"graph replay {label}: 3 replays bitwise equal to eager")


def test_graph_replay_matches_eager():
    from sparse_paged_attention_amd import api
    other = api.DeviceProblem.from_problem(synth.make_workload("decode_hca", batch=2))

    def side_work():
        api.forward(other, 3)                   # unrelated eager calls between the replays

    # decode kernel + LSE merge (4 slices)
    dp = api.DeviceProblem.from_problem(synth.make_workload("decode_csa", batch=8))
    args = dp.args(4)
    O = torch.empty((dp.num_queries, dp.num_q_heads, dp.head_dim), dtype=torch.bfloat16, device="cuda")
    L = torch.empty((dp.num_queries, dp.num_q_heads), dtype=torch.float32, device="cuda")
    ws = torch.empty(api.workspace_size(args), dtype=torch.uint8, device="cuda")
    _capture_and_replay("decode S4", lambda: api.forward_args(dp, args, O, L, ws, None), [O, L], side_work)

    # prefill query pairs
    pp = api.DeviceProblem.from_problem(_small_prefill(21))
    pargs = pp.args(1)
    O2 = torch.empty((pp.num_queries, pp.num_q_heads, pp.head_dim), dtype=torch.bfloat16, device="cuda")
    L2 = torch.empty((pp.num_queries, pp.num_q_heads), dtype=torch.float32, device="cuda")
    _capture_and_replay("prefill pairs", lambda: api.forward_args(pp, pargs, O2, L2, None, None), [O2, L2], side_work)

    # top-k selection
    rng = np.random.default_rng(3)
    scores = torch.from_numpy(rng.standard_normal((32, 1024)).astype(np.float32)).cuda()
    nv = torch.full((32,), 1024, dtype=torch.int32, device="cuda")
    ids = torch.empty((32, 512), dtype=torch.int32, device="cuda")
    cnt = torch.empty(32, dtype=torch.int32, device="cuda")
    from sparse_paged_attention_amd import _lib
    lib = _lib.load()

    def topk():
        _lib.check(lib.attn_topk_select(scores.data_ptr(), 1024, nv.data_ptr(), 32, 512, ids.data_ptr(),
                                        cnt.data_ptr(), torch.cuda.current_stream().cuda_stream))

    _capture_and_replay("top-k", topk, [ids, cnt], side_work)


def test_two_host_threads_two_streams():
    from sparse_paged_attention_amd import api
    names = (("decode_csa", 6, 4), ("mixed_fp8", 5, 8))
    jobs = []
    for n, (name, batch, splits) in enumerate(names):
        dp = api.DeviceProblem.from_problem(synth.make_workload(name, batch=batch))
        pp = api.DeviceProblem.from_problem(_small_prefill(30 + n))
        jobs.append((dp, splits, pp))
    calls = 20

    def serial(job):
        dp, splits, pp = job
        outs = []
        for k in range(calls):
            outs.append(api.forward(dp, splits) if k % 2 == 0 else api.forward(pp, 1))
        torch.cuda.synchronize()
        return outs

    ref = [serial(j) for j in jobs]
    got = [None, None]
    errors = []

    def worker(n):
        try:
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                dp, splits, pp = jobs[n]
                outs = []
                for k in range(calls):
                    outs.append(api.forward(dp, splits) if k % 2 == 0 else api.forward(pp, 1))
                s.synchronize()
            got[n] = outs
        except Exception as e:          # reported by the main thread
            errors.append(e)

    threads = [threading.Thread(target=worker, args=(n,)) for n in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors
    torch.cuda.synchronize()
    for n in range(2):
        for k in range(calls):
            for a, b in zip(got[n][k], ref[n][k]):
                assert torch.equal(_bits(a), _bits(b)), (n, k)
    announce(f"two host threads x {calls} calls on two streams: bitwise equal to serial")
