"""The asynchronous entry points can be captured in a HIP graph and
replayed: every replay must reproduce the eager result bit for bit (and the
compressed calls' device byte counters).  Replays are separated by eager
work and synchronisations, and each one is checked."""
import numpy as np
import pytest
import torch

import ring_all_reduce_scatter_amd as rar
from ring_all_reduce_scatter_amd import inputs

from gpu_util import assert_bits_equal, to_dev, to_host

pytestmark = pytest.mark.gpu

N = 8


def _capture(fn, bufs):
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn(bufs)  # warm-up: creates the library's per-device streams and events outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn(bufs)
    torch.cuda.synchronize()
    return g


def _replay_matches_eager(fn, xs, dt, replays=3, counters=None):
    want = to_dev(xs, dt)
    fn(want)
    torch.cuda.synchronize()
    want_h = to_host(want, dt)
    want_c = rar.compressed_traffic(counters, N) if counters is not None else None
    pristine = to_dev(xs, dt)
    bufs = to_dev(xs, dt)
    g = _capture(fn, bufs)
    for k in range(replays):
        for b, p in zip(bufs, pristine):
            b.copy_(p)
        if counters is not None:
            counters.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        _ = torch.ones(1 << 20, device="cuda:0").sum().item()  # eager work between replays
        got = to_host(bufs, dt)
        for r in range(N):
            assert_bits_equal(got[r], want_h[r], f"replay {k} rank {r}")
        if counters is not None:
            assert rar.compressed_traffic(counters, N) == want_c, f"replay {k} byte counters"


@pytest.mark.parametrize("algo", [rar.ALGO_FUSED, rar.ALGO_STEPWISE])
def test_ring_allreduce_replays(algo):
    xs = inputs.gradient_like(N, 300_001, salt=1)
    _replay_matches_eager(lambda b: rar.ring_allreduce_ex(b, algo), xs, "f32")


@pytest.mark.parametrize("sched", [rar.SCHED_FUSED, rar.SCHED_STAGED, rar.SCHED_FORWARD, rar.SCHED_PIPELINED])
def test_bfp_compressed_replays(sched):
    count = N * 4096 * 3 + 1000
    xs = inputs.block_scaled(N, count, salt=2)
    cfg = rar.compress_cfg(unit_bytes=8192, schedule=sched)
    ws = torch.zeros(rar.compressed_workspace_bytes(N, count, rar.F16, cfg), dtype=torch.uint8, device="cuda:0")
    _replay_matches_eager(lambda b: rar.ring_allreduce_compressed(b, cfg, ws), xs, "f16", counters=ws)


def test_sparse_auto_replays():
    count = N * 4096 * 3 + 2500
    xs = inputs.sparse_mix(N, count, salt=3)
    cfg = rar.compress_cfg(method=rar.COMP_SPARSE_AUTO, mbits=4, unit_bytes=8192, schedule=rar.SCHED_STAGED)
    ws = torch.zeros(rar.compressed_workspace_bytes(N, count, rar.F16, cfg), dtype=torch.uint8, device="cuda:0")
    _replay_matches_eager(lambda b: rar.ring_allreduce_compressed(b, cfg, ws), xs, "f16", counters=ws)


def test_tree_and_broadcast_replay():
    xs = inputs.gradient_like(N, 100_003, salt=4)
    _replay_matches_eager(lambda b: rar.tree_allreduce_ex(b, rar.ALGO_STEPWISE), xs, "f32")
    _replay_matches_eager(lambda b: rar.broadcast_ex(b, 3, rar.ALGO_STEPWISE), xs, "f32")


def test_stateful_replays_follow_the_eager_sequence():
    """The state carries over between calls: replay k must equal eager call k."""
    count = N * 4096 + 517
    xs = inputs.block_scaled(N, count, salt=5)
    cfg = rar.compress_cfg()
    ws = torch.zeros(rar.compressed_workspace_bytes(N, count, rar.F16, cfg), dtype=torch.uint8, device="cuda:0")
    st_e = [torch.zeros(count, device="cuda:0") for _ in range(N)]
    eager = []
    for _ in range(3):
        b = to_dev(xs, "f16")
        rar.ring_allreduce_compressed_state(b, st_e, rar.FEEDBACK_ERROR, cfg, ws)
        eager.append((to_host(b, "f16"), to_host(st_e, "f32")))
    st = [torch.zeros(count, device="cuda:0") for _ in range(N)]
    pristine = to_dev(xs, "f16")
    bufs = to_dev(xs, "f16")
    g = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        rar.ring_allreduce_compressed_state(bufs, st, rar.FEEDBACK_ERROR, cfg, ws)
    for k in range(3):
        for b, p in zip(bufs, pristine):
            b.copy_(p)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got, gst = to_host(bufs, "f16"), to_host(st, "f32")
        for r in range(N):
            assert_bits_equal(got[r], eager[k][0][r], f"replay {k} rank {r}")
            assert_bits_equal(gst[r], eager[k][1][r], f"replay {k} state {r}")


def test_bucketed_fused_replays():
    sizes = inputs.bucket_sizes(40, lo_exp=3, hi_exp=15, salt=6)
    th = inputs.bucket_tensors(N, sizes, dtype="bf16", salt=6)
    cap = 64 << 10
    want = [to_dev(th[r], "bf16") for r in range(N)]
    ws = torch.empty(rar.bucketed_workspace_bytes(sizes, N, rar.BF16, cap), dtype=torch.uint8, device="cuda:0")
    rar.bucketed_allreduce(want, cap, ws)
    torch.cuda.synchronize()
    want_h = [to_host(want[r], "bf16") for r in range(N)]
    pristine = [to_dev(th[r], "bf16") for r in range(N)]
    dev = [to_dev(th[r], "bf16") for r in range(N)]
    g = _capture(lambda d: rar.bucketed_allreduce(d, cap, ws), dev)
    for k in range(3):
        for r in range(N):
            for t, p in zip(dev[r], pristine[r]):
                t.copy_(p)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for r in range(N):
            got = to_host(dev[r], "bf16")
            for t in range(len(sizes)):
                assert_bits_equal(got[t], want_h[r][t], f"replay {k} rank {r} tensor {t}")


def test_prepared_bucketed_launch_replays():
    """A graph holding only the fold launch of a prepared plan (the table and
    descriptors written once, outside the graph): every replay on restored
    inputs equals the eager result."""
    sizes = inputs.bucket_sizes(40, lo_exp=3, hi_exp=15, salt=7)
    th = inputs.bucket_tensors(N, sizes, dtype="bf16", salt=7)
    cap = 64 << 10
    want = [to_dev(th[r], "bf16") for r in range(N)]
    ws = torch.empty(rar.bucketed_workspace_bytes(sizes, N, rar.BF16, cap), dtype=torch.uint8, device="cuda:0")
    rar.bucketed_allreduce(want, cap, ws)
    torch.cuda.synchronize()
    want_h = [to_host(want[r], "bf16") for r in range(N)]
    pristine = [to_dev(th[r], "bf16") for r in range(N)]
    dev = [to_dev(th[r], "bf16") for r in range(N)]
    step = rar.BucketedAllreduce(dev, cap, ws)
    g = _capture(lambda d: step(), dev)
    for k in range(3):
        for r in range(N):
            for t, p in zip(dev[r], pristine[r]):
                t.copy_(p)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for r in range(N):
            got = to_host(dev[r], "bf16")
            for t in range(len(sizes)):
                assert_bits_equal(got[t], want_h[r][t], f"replay {k} rank {r} tensor {t}")
