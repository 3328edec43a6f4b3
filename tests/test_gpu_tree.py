"""GPU parity of the tree allreduce (fused and stepwise) and of the
size-based ring/tree selection against the oracle, bit for bit."""
import numpy as np
import pytest

import oracle
import ring_all_reduce_scatter_amd as rar
from ring_all_reduce_scatter_amd import inputs

from gpu_util import DT_NAMES, assert_bits_equal, to_dev, to_host

pytestmark = pytest.mark.gpu

ALGOS = {"fused": rar.ALGO_FUSED, "stepwise": rar.ALGO_STEPWISE}


@pytest.mark.parametrize("dt", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("n", [1, 2, 3, 4, 5, 6, 7, 8, 9, 16])
@pytest.mark.parametrize("count", [1, 1000, 4096 * 3 + 77, 100_003])
@pytest.mark.parametrize("algo", ["fused", "stepwise"])
def test_tree_matches_oracle(dt, n, count, algo):
    xs = inputs.gradient_like(n, count, dtype=dt, salt=count + 3 * n)
    ref = [x.copy() for x in xs]
    osent, orecv = oracle.tree_allreduce(ref, dt=DT_NAMES[dt])
    bufs = to_dev(xs, dt)
    rar.tree_allreduce_ex(bufs, ALGOS[algo])
    assert rar.last_traffic(n) == (osent, orecv)
    got = to_host(bufs, dt)
    for r in range(n):
        assert_bits_equal(got[r], ref[r], f"rank {r}")


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("n", [32, 64])
@pytest.mark.parametrize("algo", ["fused", "stepwise"])
def test_tree_many_ranks_matches_oracle(dt, n, algo):
    """32 and 64 ranks: rank counts past the fused tree kernel's table."""
    count = 50_001
    xs = inputs.gradient_like(n, count, dtype=dt, salt=count + 3 * n)
    ref = [x.copy() for x in xs]
    osent, orecv = oracle.tree_allreduce(ref, dt=DT_NAMES[dt])
    bufs = to_dev(xs, dt)
    rar.tree_allreduce_ex(bufs, ALGOS[algo])
    assert rar.last_traffic(n) == (osent, orecv)
    got = to_host(bufs, dt)
    for r in range(n):
        assert_bits_equal(got[r], ref[r], f"rank {r}")


@pytest.mark.parametrize("count,expect", [(1000, rar.ALLREDUCE_TREE), ((1 << 18) - 1, rar.ALLREDUCE_TREE),
                                          (1 << 18, rar.ALLREDUCE_RING), (1 << 20, rar.ALLREDUCE_RING)])
def test_auto_selects_by_size(count, expect):
    n = 4
    xs = inputs.gradient_like(n, count, salt=count)
    ref = [x.copy() for x in xs]
    (oracle.tree_allreduce if expect == rar.ALLREDUCE_TREE else oracle.ring_allreduce)(ref)
    bufs = to_dev(xs, "f32")
    chosen = rar.allreduce_auto(bufs)  # 1 MiB per rank: 2^18 fp32 elements
    assert chosen == expect
    got = to_host(bufs, "f32")
    for r in range(n):
        assert_bits_equal(got[r], ref[r], f"rank {r}")


def test_tree_integer_workload_exact():
    w = inputs.WORKLOADS["ring_int"]
    xs = inputs.integers(w["n"], w["count"])
    exact = np.sum(np.stack([x.astype(np.float64) for x in xs]), axis=0)
    for algo in ALGOS.values():
        bufs = to_dev(xs, "f32")
        rar.tree_allreduce_ex(bufs, algo)
        for g in to_host(bufs, "f32"):
            assert np.array_equal(g.astype(np.float64), exact)
