"""Buffers at device addresses whose bit 31 is set (the low 32 bits of every
address in them at or past 2^31).  The write-through stores of the streaming
kernels go through buffer descriptors built from 64-bit addresses; a
sign-extended low half once turned such addresses into wild ones.  Every
collective whose kernels store write-through gives the oracle's bits there:
the fused ring and tree folds, the stepwise ring's copies, the fused BFP
folds (binary16 and binary32), the stateful fold, the pipelined BFP and
SPARSE_AUTO rings and the bucketed fold."""
import numpy as np
import pytest
import torch

import oracle
import ring_all_reduce_scatter_amd as rar
from ring_all_reduce_scatter_amd import inputs

from gpu_util import DT_NAMES, assert_bits_equal, to_host, torch_dtype

pytestmark = pytest.mark.gpu


class HighArena:
    """Byte ranges, 256-byte aligned, inside one window of a 4 GiB+ arena in
    which every address has bit 31 set."""

    def __init__(self, need):
        self.arena = torch.empty((4 << 30) + need + (1 << 20), dtype=torch.uint8, device="cuda:0")
        low = self.arena.data_ptr() & 0xFFFFFFFF
        o = max(0, (1 << 31) - low)
        if (1 << 32) - low - o < need:  # the first window is too short: the next one
            o = (1 << 32) - low + (1 << 31)
        self.pos, self.end = o, o + need

    def take(self, count, dt):
        es = torch.empty((), dtype=torch_dtype(dt)).element_size()
        nbytes = count * es
        o = self.pos
        self.pos += -(-nbytes // 256) * 256
        assert self.pos <= self.end
        t = self.arena[o:o + nbytes].view(torch_dtype(dt))
        lo, hi = t.data_ptr() & 0xFFFFFFFF, (t.data_ptr() + nbytes - 1) & 0xFFFFFFFF
        assert lo >= 1 << 31 and hi >= lo, "range outside the bit-31 window"
        return t


def _place(arena, host, dt):
    out = []
    for h in host:
        t = arena.take(h.size, dt)
        src = torch.from_numpy(np.ascontiguousarray(h.view(np.int16) if dt == "bf16" else h))
        t.copy_(src.view(torch_dtype(dt)) if dt == "bf16" else src)
        out.append(t)
    return out


def test_uncompressed_collectives_at_high_addresses():
    arena = HighArena(96 << 20)
    # fused ring (whole tiles and a ragged tail), stepwise ring (copies), tree
    for n, count, dt, run in ((8, 8 * 2048 * 3 + 77, "f32", lambda b: rar.ring_allreduce(b)),
                              (5, 3 * 4096 + 1001, "f16", lambda b: rar.ring_allreduce_ex(b, rar.ALGO_STEPWISE)),
                              (4, 4 * 2048 * 4 + 13, "f32", lambda b: rar.tree_allreduce(b))):
        xs = inputs.gradient_like(n, count, dtype=dt, salt=31 + n)
        ref = [x.copy() for x in xs]
        (oracle.tree_allreduce if n == 4 else oracle.ring_allreduce)(ref, dt=DT_NAMES[dt])
        bufs = _place(arena, xs, dt)
        run(bufs)
        for r, g in enumerate(to_host(bufs, dt)):
            assert_bits_equal(g, ref[r], f"N={n} {dt} rank {r}")


@pytest.mark.parametrize("case", ["bfp8_f16_fused", "bfp8_f32_fused", "bfp8_f16_pipelined", "sparse_pipelined"])
def test_compressed_collectives_at_high_addresses(case):
    arena = HighArena(160 << 20)
    dt = "f32" if case == "bfp8_f32_fused" else "f16"
    es = 4 if dt == "f32" else 2
    if case == "sparse_pipelined":
        n, U = 4, 2 * 16384
        count = n * 2 * U + 999
        xs = inputs.sparse_mix(n, count, dtype=dt, salt=33)
        cfg = rar.compress_cfg(method=rar.COMP_SPARSE_AUTO, mbits=4, unit_bytes=U * es, schedule=rar.SCHED_PIPELINED)
        okw = dict(method=oracle.COMP_SPARSE_AUTO, mbits=4, unit=U)
    else:
        n, U = 8, 16384
        count = n * 3 * U + 555
        xs = inputs.block_scaled(n, count, dtype=dt, salt=34)
        sched = rar.SCHED_PIPELINED if case.endswith("pipelined") else rar.SCHED_FUSED
        cfg = rar.compress_cfg(block=128, mbits=8, unit_bytes=U * es, schedule=sched)
        okw = dict(mbits=8, unit=U)
    ref = [x.copy() for x in xs]
    osent, orecv = oracle.ring_allreduce_compressed(ref, dt=DT_NAMES[dt], **okw)
    bufs = _place(arena, xs, dt)
    ws = torch.empty(rar.compressed_workspace_bytes(n, count, DT_NAMES[dt], cfg), dtype=torch.uint8, device="cuda:0")
    rar.ring_allreduce_compressed(bufs, cfg, ws)
    assert rar.compressed_traffic(ws, n) == (osent, orecv)
    for r, g in enumerate(to_host(bufs, dt)):
        assert_bits_equal(g, ref[r], f"{case} rank {r}")


def test_stateful_fold_at_high_addresses():
    arena = HighArena(96 << 20)
    n, count = 8, 8 * 2048 * 2 + 300
    xs = inputs.block_scaled(n, count, dtype="f16", salt=35)
    st0 = [(np.random.default_rng([35, r]).standard_normal(count) * 1e-4).astype(np.float32) for r in range(n)]
    ref, rst = [x.copy() for x in xs], [s.copy() for s in st0]
    oracle.ring_allreduce_compressed_state(ref, rst, oracle.FB_ERROR, mbits=8, unit=16384, dt=DT_NAMES["f16"])
    bufs = _place(arena, xs, "f16")
    st = _place(arena, st0, "f32")
    cfg = rar.compress_cfg(block=128, mbits=8, unit_bytes=16384 * 2)
    ws = torch.empty(rar.compressed_workspace_bytes(n, count, rar.F16, cfg), dtype=torch.uint8, device="cuda:0")
    rar.ring_allreduce_compressed_state(bufs, st, rar.FEEDBACK_ERROR, cfg, ws)
    for r in range(n):
        assert_bits_equal(to_host([bufs[r]], "f16")[0], ref[r], f"rank {r}")
        assert_bits_equal(to_host([st[r]], "f32")[0], rst[r], f"state {r}")


def test_bucketed_fold_at_high_addresses():
    arena = HighArena(96 << 20)
    n, dt, cap = 8, "bf16", 256 << 10
    sizes = inputs.bucket_sizes(30, lo_exp=3, hi_exp=17, salt=36)
    th = inputs.bucket_tensors(n, sizes, dtype=dt, salt=36)
    ref = [[t.copy() for t in th[r]] for r in range(n)]
    osent, orecv = oracle.bucketed_allreduce(ref, cap, dt=DT_NAMES[dt])
    dev = [_place(arena, th[r], dt) for r in range(n)]
    ws = torch.empty(rar.bucketed_workspace_bytes(sizes, n, DT_NAMES[dt], cap), dtype=torch.uint8, device="cuda:0")
    rar.bucketed_allreduce(dev, cap, ws)
    assert rar.last_traffic(n) == (osent, orecv)
    for r in range(n):
        got = to_host(dev[r], dt)
        for t in range(len(sizes)):
            assert_bits_equal(got[t], ref[r][t], f"rank {r} tensor {t}")
