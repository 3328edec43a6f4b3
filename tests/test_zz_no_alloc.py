"""The allocation-free compressed allreduce (rar_ring_allreduce_compressed_noalloc)
against rar_ring_allreduce_compressed, bit for bit, through the C ABI.

Two calls in a row on each schedule, the second on a smaller input, so a
result that leaned on what the first call left in the library's scratch
array would show.  The byte-exact comparison is the parity bar of the
compressed ring; the small case is also compared with the oracle."""
import numpy as np
import pytest
import torch

import oracle
import ring_all_reduce_scatter_amd as rar
from ring_all_reduce_scatter_amd import inputs

from gpu_util import DT_NAMES, assert_bits_equal, to_dev, to_host

pytestmark = pytest.mark.gpu

SCHEDULES = [
    ("bfp_fused", dict(method=rar.COMP_BFP, schedule=rar.SCHED_FUSED, mbits=8)),
    ("bfp_staged", dict(method=rar.COMP_BFP, schedule=rar.SCHED_STAGED, mbits=8)),
    ("bfp_forward", dict(method=rar.COMP_BFP, schedule=rar.SCHED_FORWARD, mbits=4)),
    ("sparse_auto", dict(method=rar.COMP_SPARSE_AUTO, schedule=rar.SCHED_STAGED, mbits=4)),
]


def _inputs(kind, n, count, dt, salt):
    if kind == "sparse_auto":
        return inputs.sparse_mix(n, count, dtype=dt, salt=salt)
    if dt == "f32":
        return inputs.gradient_like(n, count, salt=salt)
    return inputs.block_scaled(n, count, dtype=dt, salt=salt)


def _both(kind, kw, xs, dt, unit_elems):
    n, count = len(xs), xs[0].size
    es = 4 if dt == "f32" else 2
    cfg = rar.compress_cfg(unit_bytes=unit_elems * es, **kw)
    need = rar.compressed_workspace_bytes(n, count, DT_NAMES[dt], cfg)
    assert 0 < need <= rar.NOALLOC_SCRATCH_BYTES, (kind, need)
    ref = to_dev(xs, dt)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda:0")
    rar.ring_allreduce_compressed(ref, cfg, ws)
    got = to_dev(xs, dt)
    rar.ring_allreduce_compressed_noalloc(got, cfg)
    torch.cuda.synchronize()
    return to_host(got, dt), to_host(ref, dt)


@pytest.mark.parametrize("kind,kw", SCHEDULES, ids=[s[0] for s in SCHEDULES])
@pytest.mark.parametrize("dt", ["f16", "bf16", "f32"])
def test_noalloc_equals_workspace_call_twice(kind, kw, dt):
    # first call: 8 ranks, 4 MiB of the dtype per rank, 1 MiB units (several
    # units per chunk, most of the 32 MiB scratch for the staged schedules)
    es = 4 if dt == "f32" else 2
    n1, c1, u1 = 8, (4 << 20) // es, (1 << 20) // es
    xs1 = _inputs(kind, n1, c1, dt, salt=31)
    got, ref = _both(kind, kw, xs1, dt, u1)
    for r in range(n1):
        assert_bits_equal(got[r], ref[r], f"{kind} call 1 rank {r}")
    # second call, smaller and ragged: what the first left behind must not leak in
    n2, c2, u2 = 3, 3 * 5 * 2048 + 999, 2048
    xs2 = _inputs(kind, n2, c2, dt, salt=32)
    got, ref = _both(kind, kw, xs2, dt, u2)
    for r in range(n2):
        assert_bits_equal(got[r], ref[r], f"{kind} call 2 rank {r}")
    orc = [x.copy() for x in xs2]
    oracle.ring_allreduce_compressed(orc, method=kw["method"], mbits=kw["mbits"], unit=u2, dt=DT_NAMES[dt])
    for r in range(n2):
        assert_bits_equal(got[r], orc[r], f"{kind} call 2 rank {r} vs oracle")


def test_noalloc_refuses_more_than_its_scratch():
    """A staged call whose messages exceed the scratch array is refused
    before anything is enqueued (the buffers stay as they were)."""
    n, count = 8, 32 << 20  # 8 ranks x 64 MiB fp16: 16 message slots of ~2.1 MB
    cfg = rar.compress_cfg(schedule=rar.SCHED_STAGED)
    assert rar.compressed_workspace_bytes(n, count, rar.F16, cfg) > rar.NOALLOC_SCRATCH_BYTES
    bufs = [torch.full((count,), 1.0, dtype=torch.float16, device="cuda:0") for _ in range(n)]
    with pytest.raises(rar.RarError) as e:
        rar.ring_allreduce_compressed_noalloc(bufs, cfg)
    assert e.value.status == 4
    torch.cuda.synchronize()
    assert all(bool((b == 1.0).all()) for b in bufs)
    # the fused schedule needs only the byte counters at any size
    rar.ring_allreduce_compressed_noalloc(bufs, rar.compress_cfg(schedule=rar.SCHED_FUSED))
    torch.cuda.synchronize()
    assert all(bool((b == 8.0).all()) for b in bufs)
