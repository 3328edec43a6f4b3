"""The oracle's ring allreduce against torch.distributed's gloo backend, the
check the page "从零实现集合通信" prescribes in its section on verifying with
gloo: run the same tensors through gloo at the same world size and fail if
the two differ by more than float32 epsilon.  Reading of "epsilon" for sums
whose order differs: per element, FLT_EPSILON times the sum of |x_r| (the
scale every reordered float32 sum of N terms is accurate to within N-1 such
units); integer-valued inputs, where every order is exact, must match
exactly.  CPU only: gloo on CPU tensors, one process per rank, 127.0.0.1."""
import os
import socket

import numpy as np
import pytest
import torch
import torch.distributed as dist
import torch.multiprocessing as mp

from ring_all_reduce_scatter_amd import inputs

N = 4
COUNT = 50_003


def _free_port():
    with socket.socket() as s:
        s.bind(("127.0.0.1", 0))
        return s.getsockname()[1]


def _rank_main(rank, port, kind, out):
    os.environ["MASTER_ADDR"] = "127.0.0.1"
    os.environ["MASTER_PORT"] = str(port)
    dist.init_process_group("gloo", rank=rank, world_size=N)
    try:
        if kind == "int":
            x = inputs.integers(N, COUNT)[rank]
        else:
            x = inputs.gradient_like(N, COUNT, salt=3)[rank]
        t = torch.from_numpy(x.copy())
        dist.all_reduce(t, op=dist.ReduceOp.SUM)
        if rank == 0:
            out.put(t.numpy().tobytes())
    finally:
        dist.destroy_process_group()


def _gloo_sum(kind):
    ctx = mp.get_context("spawn")
    q = ctx.Queue()
    port = _free_port()
    procs = [ctx.Process(target=_rank_main, args=(r, port, kind, q)) for r in range(N)]
    for p in procs:
        p.start()
    res = np.frombuffer(q.get(timeout=120), dtype=np.float32).copy()
    for p in procs:
        p.join(timeout=60)
        assert p.exitcode == 0
    return res


@pytest.mark.parametrize("kind", ["int", "grad"])
def test_oracle_ring_matches_gloo(orc, kind):
    if kind == "int":
        xs = inputs.integers(N, COUNT)
    else:
        xs = inputs.gradient_like(N, COUNT, salt=3)
    bufs = [x.copy() for x in xs]
    orc.ring_allreduce(bufs)
    ref = _gloo_sum(kind)
    if kind == "int":
        assert np.array_equal(bufs[0], ref)
    else:
        scale = np.sum(np.abs(np.stack(xs).astype(np.float64)), axis=0)
        dev = np.abs(bufs[0].astype(np.float64) - ref.astype(np.float64))
        assert np.all(dev <= (N - 1) * np.finfo(np.float32).eps * scale)
    for b in bufs[1:]:
        assert np.array_equal(b, bufs[0])
