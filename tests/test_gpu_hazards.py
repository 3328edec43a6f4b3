"""Ordering and hazard checks on the GPU.

* Guard bands: every rank buffer sits between two canary regions of one
  allocation; after each collective (all schedules, ragged sizes) every
  canary byte must be untouched, and so must the padding past each
  workspace's used size.
* The stepwise schedule enqueued all at once equals the same steps with a
  device synchronisation after every launch, bit for bit."""
import numpy as np
import pytest
import torch

import ring_all_reduce_scatter_amd as rar
from ring_all_reduce_scatter_amd import inputs

from gpu_util import DT_NAMES, assert_bits_equal, to_host

pytestmark = pytest.mark.gpu

GUARD = 4096  # bytes of canary on each side of every rank buffer
CANARY = 0xA7


class Guarded:
    """n rank buffers of `count` elements inside one byte allocation, each
    with GUARD canary bytes before and after (buffer starts stay 16-aligned)."""

    def __init__(self, host_arrays, dt):
        self.n = len(host_arrays)
        self.count = host_arrays[0].size
        es = 4 if dt == "f32" else 2
        self.nbytes = self.count * es
        self.slot = GUARD + (self.nbytes + 15) // 16 * 16 + GUARD
        self.raw = torch.full((self.n * self.slot,), CANARY, dtype=torch.uint8, device="cuda:0")
        tdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[dt]
        self.bufs = []
        for r, a in enumerate(host_arrays):
            lo = r * self.slot + GUARD
            view = self.raw[lo:lo + self.nbytes].view(tdt)
            src = torch.from_numpy(np.ascontiguousarray(a).view(np.int16 if dt == "bf16" else a.dtype))
            view.copy_(src.view(tdt).to("cuda:0") if dt == "bf16" else src.to("cuda:0"))
            self.bufs.append(view)

    def check(self, what):
        torch.cuda.synchronize()
        raw = self.raw.cpu().numpy()
        for r in range(self.n):
            lo = r * self.slot
            pre = raw[lo:lo + GUARD]
            post = raw[lo + GUARD + self.nbytes:lo + self.slot]
            assert np.all(pre == CANARY), f"{what}: canary before rank {r} overwritten"
            assert np.all(post == CANARY), f"{what}: canary after rank {r} overwritten"


def _ws(nbytes):
    """Workspace with a canary tail of GUARD bytes; returns (tensor view, full, used)."""
    full = torch.full((nbytes + GUARD,), CANARY, dtype=torch.uint8, device="cuda:0")
    return full[:max(nbytes, 16)], full, nbytes


def _ws_check(full, used, what):
    tail = full[used:].cpu().numpy()
    assert np.all(tail == CANARY), f"{what}: write past the workspace"


@pytest.mark.parametrize("dt", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("n,count", [(2, 1), (3, 1001), (5, 4096 * 3 + 77), (8, 100_003), (16, 33_333)])
def test_uncompressed_collectives_stay_in_bounds(dt, n, count):
    xs = inputs.gradient_like(n, count, dtype=dt, salt=n)
    for name, fn in (("fused allreduce", lambda b: rar.ring_allreduce_ex(b, rar.ALGO_FUSED)),
                     ("stepwise allreduce", lambda b: rar.ring_allreduce_ex(b, rar.ALGO_STEPWISE)),
                     ("fused reduce-scatter", lambda b: rar.reduce_scatter_ex(b, rar.ALGO_FUSED)),
                     ("tree fused", lambda b: rar.tree_allreduce_ex(b, rar.ALGO_FUSED)),
                     ("tree stepwise", lambda b: rar.tree_allreduce_ex(b, rar.ALGO_STEPWISE)),
                     ("broadcast", lambda b: rar.broadcast_ex(b, n - 1, rar.ALGO_FUSED)),
                     ("broadcast stepwise", lambda b: rar.broadcast_ex(b, 0, rar.ALGO_STEPWISE))):
        g = Guarded(xs, dt)
        fn(g.bufs)
        g.check(name)
    c2 = (count // n + 1) * n  # allgather needs count divisible by N
    ys = inputs.gradient_like(n, c2, dtype=dt, salt=3)
    for algo in (rar.ALGO_FUSED, rar.ALGO_STEPWISE):
        g = Guarded(ys, dt)
        rar.allgather_ex(g.bufs, algo)
        g.check(f"allgather algo {algo}")


@pytest.mark.parametrize("dt", ["f16", "bf16", "f32"])
@pytest.mark.parametrize("n,count", [(2, 129), (3, 4096 * 5 + 3), (8, 8 * 4096 * 3 + 1000)])
def test_compressed_paths_stay_in_bounds(dt, n, count):
    xs = inputs.sparse_mix(n, count, dtype=dt, salt=n) if dt != "f32" else inputs.gradient_like(n, count, salt=n)
    cfgs = [("bfp fused", rar.compress_cfg(unit_bytes=8192)),
            ("bfp staged", rar.compress_cfg(unit_bytes=8192, schedule=rar.SCHED_STAGED)),
            ("bfp forward", rar.compress_cfg(unit_bytes=8192, schedule=rar.SCHED_FORWARD)),
            ("bfp pipelined", rar.compress_cfg(unit_bytes=8192, schedule=rar.SCHED_PIPELINED)),
            ("bfp4 pipelined block 32", rar.compress_cfg(unit_bytes=4096, mbits=4, block=32,
                                                         schedule=rar.SCHED_PIPELINED)),
            ("bfp4 staged block 32", rar.compress_cfg(unit_bytes=4096, mbits=4, block=32, schedule=rar.SCHED_STAGED)),
            ("sparse auto", rar.compress_cfg(method=rar.COMP_SPARSE_AUTO, mbits=4, unit_bytes=8192,
                                             schedule=rar.SCHED_STAGED)),
            ("sparse auto pipelined", rar.compress_cfg(method=rar.COMP_SPARSE_AUTO, mbits=4, unit_bytes=8192,
                                                       schedule=rar.SCHED_PIPELINED))]
    for name, cfg in cfgs:
        g = Guarded(xs, dt)
        ws, full, used = _ws(rar.compressed_workspace_bytes(n, count, DT_NAMES[dt], cfg))
        rar.ring_allreduce_compressed(g.bufs, cfg, ws)
        g.check(name)
        _ws_check(full, used, name)
    # stateful: state buffers guarded too
    g = Guarded(xs, dt)
    sg = Guarded([np.zeros(count, np.float32) for _ in range(n)], "f32")
    cfg = rar.compress_cfg(block=128, mbits=8)
    ws, full, used = _ws(rar.compressed_workspace_bytes(n, count, DT_NAMES[dt], cfg))
    for fb in (rar.FEEDBACK_ERROR, rar.FEEDBACK_DELTA):
        rar.ring_allreduce_compressed_state(g.bufs, sg.bufs, fb, cfg, ws)
        g.check(f"stateful {fb}")
        sg.check(f"stateful {fb} state")
        _ws_check(full, used, "stateful")


@pytest.mark.parametrize("dt", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("count", [1, 8 * 256 * 2 + 1, 8 * 256 * 3 + 9, 4096 * 5 + 77])
@pytest.mark.parametrize("block,mbits", [(128, 8), (32, 4)])
def test_codec_stays_in_bounds(dt, count, block, mbits):
    """Standalone compress and decompress(-accumulate) write nothing past the
    message (exactly rar_bfp_bytes long) or the destination, including counts
    that end inside the last lane group or the second group of a lane."""
    xs = inputs.block_scaled(2, count, dtype=dt, salt=count) if dt != "f32" else inputs.gradient_like(2, count,
                                                                                                     salt=count)
    g = Guarded(xs, dt)
    nbytes = rar.bfp_bytes(count, block, mbits)
    msg, full, used = _ws(nbytes)
    rar.bfp_compress(g.bufs[0], block, mbits, msg)
    _ws_check(full, used, "compress")
    rar.bfp_decompress_accumulate(msg, count, block, mbits, g.bufs[1])
    g.check("decompress-accumulate")
    rar.bfp_decompress(msg, count, block, mbits, g.bufs[1])
    g.check("decompress")
    _ws_check(full, used, "message after decode")


def test_bucketed_and_ft_stay_in_bounds():
    n = 4
    sizes = inputs.bucket_sizes(25, lo_exp=2, hi_exp=14, salt=2)
    th = inputs.bucket_tensors(n, sizes, dtype="bf16", salt=2)
    # each tensor of each rank in its own guarded slot
    guarded = [[Guarded([th[r][t]], "bf16") for t in range(len(sizes))] for r in range(n)]
    dev = [[guarded[r][t].bufs[0] for t in range(len(sizes))] for r in range(n)]
    for algo in (rar.ALGO_FUSED, rar.ALGO_STEPWISE):
        ws, full, used = _ws(rar.bucketed_workspace_bytes(sizes, n, rar.BF16, 16 << 10, algo))
        rar.bucketed_allreduce(dev, 16 << 10, ws, algo=algo)
        for r in range(n):
            for t in range(len(sizes)):
                guarded[r][t].check(f"bucketed algo {algo} rank {r} tensor {t}")
        _ws_check(full, used, f"bucketed algo {algo}")
    xs = inputs.gradient_like(5, 70_001, salt=4)
    g = Guarded(xs, "f32")
    ws, full, used = _ws(rar.ft_workspace_bytes(5, 70_001, rar.F32))
    rar.ring_allreduce_ft(g.bufs, [(2, 3)], ws)
    g.check("fault-tolerant ring")
    _ws_check(full, used, "fault-tolerant ring")


@pytest.mark.parametrize("n", [3, 8])
def test_stepwise_async_equals_synchronised_steps(n):
    count = 4096 * 7 + 333
    xs = inputs.gradient_like(n, count, salt=n)
    a = Guarded(xs, "f32")
    rar.ring_allreduce_ex(a.bufs, rar.ALGO_STEPWISE)  # all 2(N-1) launches enqueued back to back
    b = Guarded(xs, "f32")
    for s in range(1, n):
        rar.rs_step(b.bufs, s)
        torch.cuda.synchronize()
    for s in range(1, n):
        rar.ag_step(b.bufs, s)
        torch.cuda.synchronize()
    for r in range(n):
        assert_bits_equal(to_host([a.bufs[r]], "f32")[0], to_host([b.bufs[r]], "f32")[0], f"rank {r}")
    a.check("async stepwise")
    b.check("synchronised stepwise")
