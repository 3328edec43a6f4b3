"""GPU parity of the shared-state hash, the majority re-send and the
fault-injected ring allreduce against the oracle (faults are forced from the
host: a failed rank is one the host scheduler stops launching steps for, so
every kernel runs to completion)."""
import numpy as np
import pytest
import torch

import oracle
import ring_all_reduce_scatter_amd as rar
from ring_all_reduce_scatter_amd import inputs

from gpu_util import DT_NAMES, assert_bits_equal, to_dev, to_host

pytestmark = pytest.mark.gpu


def _ws(nbytes):
    return torch.empty(max(nbytes, 16), dtype=torch.uint8, device="cuda:0")


@pytest.mark.parametrize("nbytes", [0, 1, 7, 8, 15, 16, 17, 31, 4097, (1 << 20) + 3, 9_000_016])
def test_rank_hashes_match_oracle(nbytes):
    g = np.random.default_rng(nbytes)
    n = 5
    host = [g.integers(0, 256, size=nbytes + 16, dtype=np.uint8) for _ in range(n)]
    dev = [torch.from_numpy(h).to("cuda:0") for h in host]
    got = rar.rank_hashes(dev, _ws(rar.HASH_WORKSPACE_BYTES), nbytes=nbytes)
    assert got == [oracle.hash64(h[:nbytes]) for h in host]


def test_rank_hashes_see_a_single_bit_and_sign_of_zero():
    x = inputs.gradient_like(1, 1 << 20, salt=2)[0]
    y = x.copy()
    y.view(np.uint32)[123_457] ^= 1
    z = np.zeros(1000, np.float32)
    dev = to_dev([x, y, x], "f32")
    h = rar.rank_hashes(dev, _ws(512))
    assert h[0] == h[2] != h[1]
    assert rar.rank_hashes(to_dev([z, -z], "f32"), _ws(512)) == [oracle.hash64(z), oracle.hash64(-z)]


@pytest.mark.parametrize("n", [2, 3, 5, 8, 64])
def test_shared_state_sync_matches_oracle(n):
    base = inputs.gradient_like(1, 300_001, salt=n)[0]
    host = [base.copy() for _ in range(n)]
    g = np.random.default_rng(n)
    for r in g.choice(n, size=(n - 1) // 2, replace=False):  # a minority diverges
        host[r][int(g.integers(0, base.size))] += 1.0
    ref = [h.copy() for h in host]
    oresent, ohashes, osent, orecv = oracle.shared_state_sync(ref)
    dev = to_dev(host, "f32")
    resent, hashes = rar.shared_state_sync(dev, _ws(512))
    assert resent == oresent and hashes == ohashes
    assert rar.last_traffic(n) == (osent, orecv)
    got = to_host(dev, "f32")
    for r in range(n):
        assert_bits_equal(got[r], ref[r], f"rank {r}")


PLANS = [[], [(2, 1)], [(0, 5)], [(4, 3), (1, 1)], [(3, 9), (5, 2), (6, 6)], [(7, 14)], [(1, 1), (6, 1)],
         [(2, 4, 5), (6, 4, 30)], [(0, 2, 3)]]  # (rank, step, stall ms) against a 20 ms deadline


@pytest.mark.parametrize("dt", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("plan", PLANS, ids=[str(p) for p in PLANS])
@pytest.mark.parametrize("count", [1000, 3 * 4096 + 77])
def test_ft_ring_matches_oracle(dt, plan, count):
    n = 8
    xs = inputs.gradient_like(n, count, dtype=dt, salt=count + len(plan))
    ref = [x.copy() for x in xs]
    orep = oracle.ring_allreduce_ft(ref, plan, deadline_ms=20, dt=DT_NAMES[dt])
    bufs = to_dev(xs, dt)
    ws = _ws(rar.ft_workspace_bytes(n, count, DT_NAMES[dt]))
    rep = rar.ring_allreduce_ft(bufs, plan, ws, deadline_ms=20)
    assert rep["status"] == orep["status"] == 0
    for key in ("attempts", "survivors", "dead_attempt", "dead_step", "dead_reason", "waited_ms"):
        assert rep[key] == orep[key], key
    assert rar.last_traffic(n) == (orep["sent"], orep["recv"])
    got = to_host(bufs, dt)
    for r in range(n):
        assert_bits_equal(got[r], ref[r], f"rank {r}")
        assert rep["hash"][r] == oracle.hash64(ref[r]), f"hash of rank {r}"
    assert len({rep["hash"][r] for r in rep["survivors"]}) == 1


@pytest.mark.parametrize("n", [1, 2, 3, 16, 64])
def test_ft_ring_other_rank_counts(n):
    count = 50_000
    xs = inputs.gradient_like(n, count, salt=n)
    plans = [[], [(0, 1)], [(n - 1, 2)], [(r, 1) for r in range(n)]]
    for plan in plans:
        ref = [x.copy() for x in xs]
        orep = oracle.ring_allreduce_ft(ref, plan)
        bufs = to_dev(xs, "f32")
        rep = rar.ring_allreduce_ft(bufs, plan, _ws(rar.ft_workspace_bytes(n, count, rar.F32)))
        assert rep["status"] == (rar.EABORT if orep["status"] == oracle.EABORT else 0), plan
        assert (rep["attempts"], rep["survivors"]) == (orep["attempts"], orep["survivors"]), plan
        got = to_host(bufs, "f32")
        for r in range(n):
            assert_bits_equal(got[r], ref[r], f"plan {plan} rank {r}")


@pytest.mark.slow
def test_ft_ring_grad_workload_full_size():
    """N=8, T=64M fp32 per rank (256 MiB); rank 3 fails before the fifth step.
    The seven survivors must hold the ring allreduce of their own inputs (a
    fresh ring over seven ranks in the oracle), rank 3 its input, and all
    survivor hashes must agree."""
    w = inputs.WORKLOADS["ring_grad"]
    n, count = w["n"], w["count"]
    xs = inputs.gradient_like(n, count)
    bufs = to_dev(xs, "f32")
    ws = _ws(rar.ft_workspace_bytes(n, count, rar.F32))
    rep = rar.ring_allreduce_ft(bufs, [(3, 5)], ws)
    del ws
    assert rep["status"] == 0 and rep["attempts"] == 2 and rep["survivors"] == [0, 1, 2, 4, 5, 6, 7]
    got = to_host(bufs, "f32")
    del bufs
    assert_bits_equal(got[3], xs[3], "failed rank keeps its input")
    surv = [xs[r] for r in rep["survivors"]]
    oracle.ring_allreduce(surv)
    for j, r in enumerate(rep["survivors"]):
        assert_bits_equal(got[r], surv[j], f"survivor {r}")
    assert len({rep["hash"][r] for r in rep["survivors"]}) == 1
    assert rep["hash"][0] == oracle.hash64(surv[0])
