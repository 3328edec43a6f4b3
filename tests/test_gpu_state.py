"""GPU parity of the stateful fused BFP ring (error feedback and delta
coding) against the oracle: several allreduces in a row with fresh inputs,
rank buffers and per-rank state compared bit for bit after each call, and the
wire byte counters against the oracle's."""
import numpy as np
import pytest
import torch

import oracle
import ring_all_reduce_scatter_amd as rar
from ring_all_reduce_scatter_amd import inputs

from gpu_util import DT_NAMES, assert_bits_equal, to_dev, to_host

pytestmark = pytest.mark.gpu

FB = {"error": (rar.FEEDBACK_ERROR, oracle.FB_ERROR), "delta": (rar.FEEDBACK_DELTA, oracle.FB_DELTA)}


def _run(dt, n, count, block, mbits, fb, calls=3, kind="grad"):
    cfg = rar.compress_cfg(block=block, mbits=mbits)
    ws = torch.empty(rar.compressed_workspace_bytes(n, count, DT_NAMES[dt], cfg), dtype=torch.uint8,
                     device="cuda:0")
    st_dev = [torch.zeros(count, dtype=torch.float32, device="cuda:0") for _ in range(n)]
    st_ref = [np.zeros(count, dtype=np.float32) for _ in range(n)]
    for call in range(calls):
        if kind == "grad":
            xs = inputs.gradient_like(n, count, dtype=dt, salt=1000 * call + count + n)
        else:
            xs = inputs.block_scaled(n, count, dtype=dt, salt=1000 * call + count + n)
        ref = [x.copy() for x in xs]
        osent, orecv = oracle.ring_allreduce_compressed_state(ref, st_ref, FB[fb][1], block=block, mbits=mbits,
                                                              unit=cfg.unit_bytes // (4 if dt == "f32" else 2),
                                                              dt=DT_NAMES[dt])
        bufs = to_dev(xs, dt)
        rar.ring_allreduce_compressed_state(bufs, st_dev, FB[fb][0], cfg, ws)
        sent, recv = rar.compressed_traffic(ws, n)
        got = to_host(bufs, dt)
        gst = to_host(st_dev, "f32")
        for r in range(n):
            assert_bits_equal(got[r], ref[r], f"call {call} rank {r} result")
            assert_bits_equal(gst[r], st_ref[r], f"call {call} rank {r} state")
        assert (sent, recv) == (osent, orecv), f"call {call} traffic"


@pytest.mark.parametrize("fb", ["error", "delta"])
@pytest.mark.parametrize("dt", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("n", [1, 2, 3, 4, 8])
@pytest.mark.parametrize("block,mbits", [(128, 8), (128, 4), (32, 3), (256, 6), (512, 5)])
def test_stateful_ring_matches_oracle(fb, dt, n, block, mbits):
    _run(dt, n, 3 * 4096 + 517, block, mbits, fb)


@pytest.mark.parametrize("fb", ["error", "delta"])
@pytest.mark.parametrize("dt", ["f16", "f32"])
@pytest.mark.parametrize("n", [16, 64])
def test_stateful_ring_many_ranks_matches_oracle(fb, dt, n):
    """The generic-N stateful fold at 16 and 64 ranks."""
    _run(dt, n, n * 300 + 517, 128, 8, fb, calls=2)


@pytest.mark.parametrize("fb", ["error", "delta"])
def test_stateful_ring_ragged_and_multi_unit(fb):
    """Chunks longer than one 4 MiB unit, ragged tail, empty trailing chunk."""
    _run("f16", 5, (1 << 21) * 5 + 2049, 128, 8, fb, calls=2, kind="scaled")
    _run("f32", 16, 1000, 16, 2, fb, calls=2)


def test_first_error_feedback_call_equals_plain_compressed_ring():
    n, count = 8, 50_000
    xs = inputs.block_scaled(n, count, dtype="f16", salt=5)
    cfg = rar.compress_cfg()
    ws = torch.empty(rar.compressed_workspace_bytes(n, count, rar.F16, cfg), dtype=torch.uint8, device="cuda:0")
    a = to_dev(xs, "f16")
    rar.ring_allreduce_compressed(a, cfg, ws)
    b = to_dev(xs, "f16")
    st = [torch.zeros(count, dtype=torch.float32, device="cuda:0") for _ in range(n)]
    rar.ring_allreduce_compressed_state(b, st, rar.FEEDBACK_ERROR, cfg, ws)
    for r in range(n):
        assert_bits_equal(to_host([b[r]], "f16")[0], to_host([a[r]], "f16")[0], f"rank {r}")


def test_stateful_rejects_unsupported_configs():
    n, count = 2, 4096
    bufs = [torch.zeros(count, dtype=torch.float16, device="cuda:0") for _ in range(n)]
    st = [torch.zeros(count, dtype=torch.float32, device="cuda:0") for _ in range(n)]
    ws = torch.empty(1 << 16, dtype=torch.uint8, device="cuda:0")
    for cfg in (rar.compress_cfg(schedule=rar.SCHED_STAGED), rar.compress_cfg(method=rar.COMP_SPARSE_AUTO),
                rar.compress_cfg(method=rar.COMP_NONE), rar.compress_cfg(collective_mask=rar.OP_BROADCAST)):
        with pytest.raises(rar.RarError) as e:
            rar.ring_allreduce_compressed_state(bufs, st, rar.FEEDBACK_ERROR, cfg, ws)
        assert e.value.status == 6
    with pytest.raises(rar.RarError) as e:  # two ranks sharing one state buffer
        rar.ring_allreduce_compressed_state(bufs, [st[0], st[0]], rar.FEEDBACK_ERROR, rar.compress_cfg(), ws)
    assert e.value.status == 7
    with pytest.raises(ValueError):  # state must be float32
        rar.ring_allreduce_compressed_state(bufs, [st[0], bufs[1]], rar.FEEDBACK_ERROR, rar.compress_cfg(), ws)
    with pytest.raises(rar.RarError) as e:
        rar.ring_allreduce_compressed_state(bufs, st, 0, rar.compress_cfg(), ws)
    assert e.value.status == 1


@pytest.mark.slow
@pytest.mark.parametrize("fb", ["error", "delta"])
def test_stateful_bfp8_workload_full_size(fb):
    """N=8, T=128M fp16 per rank, 128-element blocks, 8-bit mantissas, with
    128M-float state per rank: two calls of the launch the benchmark times.
    Every element of the result and of every rank's state equals the
    oracle's, run over the whole workload on host threads (one unit index at
    a time, the state sliced alike)."""
    import full_size
    w = inputs.WORKLOADS["bfp8"]
    n, count, mbits, U = w["n"], w["count"], w["mbits"], w["unit_bytes"] // 2
    xs = inputs.block_scaled(n, count)
    cfg = rar.compress_cfg(mbits=mbits, unit_bytes=w["unit_bytes"])
    ws = torch.empty(rar.compressed_workspace_bytes(n, count, rar.F16, cfg), dtype=torch.uint8, device="cuda:0")
    st = [torch.zeros(count, dtype=torch.float32, device="cuda:0") for _ in range(n)]
    bufs = None
    for _ in range(2):
        bufs = to_dev(xs, "f16")
        rar.ring_allreduce_compressed_state(bufs, st, FB[fb][0], cfg, ws)
    for r in range(1, n):
        assert torch.equal(bufs[r].view(torch.int16), bufs[0].view(torch.int16)), f"rank {r} differs"
    got = to_host(bufs[:1], "f16")[0]
    got_st = to_host(st, "f32")
    del bufs, st
    L = rar.compressed_chunk_len(count, n, 128)
    want, want_st = full_size.compressed_ring_state(xs, [np.zeros(count, np.float32) for _ in range(n)], L, U,
                                                    FB[fb][1], 2, mbits=mbits)
    assert_bits_equal(got, want, "result")
    for r in range(n):
        assert_bits_equal(got_st[r], want_st[r], f"rank {r} state")
