"""GPU parity of the uncompressed collectives against the CPU oracle, bit for
bit, through the C-ABI (fused and stepwise schedules, all three dtypes,
ranks 1..64, ragged and empty chunks), and the byte counters against the
oracle's."""
import numpy as np
import pytest

import oracle
import ring_all_reduce_scatter_amd as rar
from ring_all_reduce_scatter_amd import inputs

from gpu_util import DT_NAMES, assert_bits_equal, to_dev, to_host

pytestmark = pytest.mark.gpu

ALGOS = {"fused": rar.ALGO_FUSED, "stepwise": rar.ALGO_STEPWISE}


def _inputs(n, count, dt, salt):
    return inputs.gradient_like(n, count, dtype=dt, salt=salt)


def _oracle_dt(dt):
    return DT_NAMES[dt]


@pytest.mark.parametrize("dt", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("n", [1, 2, 3, 4, 5, 8, 16])
@pytest.mark.parametrize("count", [1, 1000, 4096 * 3 + 77, 100_003])
@pytest.mark.parametrize("algo", ["fused", "stepwise"])
def test_allreduce_matches_oracle(dt, n, count, algo):
    xs = _inputs(n, count, dt, salt=count + n)
    ref = [x.copy() for x in xs]
    osent, orecv = oracle.ring_allreduce(ref, dt=_oracle_dt(dt))
    bufs = to_dev(xs, dt)
    rar.ring_allreduce_ex(bufs, ALGOS[algo])
    sent, recv = rar.last_traffic(n)
    got = to_host(bufs, dt)
    for r in range(n):
        assert_bits_equal(got[r], ref[r], f"rank {r}")
    assert sent == osent and recv == orecv


@pytest.mark.parametrize("dt", ["f32", "f16", "bf16"])
def test_fused_fold_tile_orders_at_16_ranks(dt):
    """At 16 ranks the fused fold hands consecutive workgroups runs of
    consecutive tiles of one chunk (32 tiles for 16-bit data, the whole
    chunk for binary32): with 46 tiles per chunk and a ragged end, every
    element still equals the oracle's."""
    n = 16
    count = n * 92_460 + 77
    xs = _inputs(n, count, dt, salt=46)
    ref = [x.copy() for x in xs]
    osent, orecv = oracle.ring_allreduce(ref, dt=_oracle_dt(dt))
    bufs = to_dev(xs, dt)
    rar.ring_allreduce(bufs)
    assert rar.last_traffic(n) == (osent, orecv)
    got = to_host(bufs, dt)
    for r in range(n):
        assert_bits_equal(got[r], ref[r], f"rank {r}")


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("n", [2, 3, 8, 16, 64])
@pytest.mark.parametrize("algo", ["fused", "stepwise"])
def test_reduce_scatter_matches_oracle(dt, n, algo):
    count = 50_000
    xs = _inputs(n, count, dt, salt=7 * n)
    ref = [x.copy() for x in xs]
    oracle.reduce_scatter(ref, dt=_oracle_dt(dt))
    bufs = to_dev(xs, dt)
    rar.reduce_scatter_ex(bufs, ALGOS[algo])
    got = to_host(bufs, dt)
    L = rar.chunk_len(count, n)
    for r in range(n):
        lo, hi = min(r * L, count), min((r + 1) * L, count)
        assert_bits_equal(got[r][lo:hi], ref[r][lo:hi], f"rank {r} own chunk")
        if algo == "stepwise":  # the whole materialised state equals the oracle's
            assert_bits_equal(got[r], ref[r], f"rank {r} state")


@pytest.mark.parametrize("n", [2, 4, 5, 8, 16])
def test_single_steps_match_oracle_state(n):
    count = 3 * 4096 + 300
    xs = _inputs(n, count, "f32", salt=100 + n)
    ref = [x.copy() for x in xs]
    bufs = to_dev(xs, "f32")
    for s in range(1, n):
        oracle.rs_step(ref, s)
        rar.rs_step(bufs, s)
        got = to_host(bufs, "f32")
        for r in range(n):
            assert_bits_equal(got[r], ref[r], f"after RS step {s}, rank {r}")
    for s in range(1, n):
        oracle.ag_step(ref, s)
        rar.ag_step(bufs, s)
        got = to_host(bufs, "f32")
        for r in range(n):
            assert_bits_equal(got[r], ref[r], f"after AG step {s}, rank {r}")


@pytest.mark.parametrize("dt", ["f32", "f16"])
@pytest.mark.parametrize("n", [1, 2, 3, 8, 16])
@pytest.mark.parametrize("shard", [1, 333, 4096, 70_001])
@pytest.mark.parametrize("algo", ["fused", "stepwise"])
def test_allgather_matches_oracle(dt, n, shard, algo):
    xs = inputs.filler(n, n * shard, dtype=dt, salt=shard)
    ref = [x.copy() for x in xs]
    osent, orecv = oracle.allgather(ref, dt=_oracle_dt(dt))
    bufs = to_dev(xs, dt)
    rar.allgather_ex(bufs, ALGOS[algo])
    assert rar.last_traffic(n) == (osent, orecv)
    got = to_host(bufs, dt)
    for r in range(n):
        assert_bits_equal(got[r], ref[r], f"rank {r}")


@pytest.mark.parametrize("n", [1, 2, 3, 5, 8, 16])
@pytest.mark.parametrize("root", [0, 3])
@pytest.mark.parametrize("count", [1, 1001, 300_000])
@pytest.mark.parametrize("algo", ["fused", "stepwise"])
def test_broadcast_matches_oracle(n, root, count, algo):
    if root >= n:
        pytest.skip("root outside ring")
    xs = inputs.filler(n, count, salt=count + root)
    ref = [x.copy() for x in xs]
    osent, orecv = oracle.broadcast(ref, root=root)
    bufs = to_dev(xs, "f32")
    rar.broadcast_ex(bufs, root, ALGOS[algo])
    assert rar.last_traffic(n) == (osent, orecv)
    got = to_host(bufs, "f32")
    for r in range(n):
        assert_bits_equal(got[r], ref[r], f"rank {r}")


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("n", [32, 64])
@pytest.mark.parametrize("count", [1000, 70_001])
@pytest.mark.parametrize("algo", ["fused", "stepwise"])
def test_allreduce_many_ranks_matches_oracle(dt, n, count, algo):
    """Up to the largest ring the boundary takes (64 ranks): the fold's
    run-time rank loop, and 2(N-1) step launches."""
    xs = _inputs(n, count, dt, salt=count + n)
    ref = [x.copy() for x in xs]
    osent, orecv = oracle.ring_allreduce(ref, dt=_oracle_dt(dt))
    bufs = to_dev(xs, dt)
    rar.ring_allreduce_ex(bufs, ALGOS[algo])
    sent, recv = rar.last_traffic(n)
    got = to_host(bufs, dt)
    for r in range(n):
        assert_bits_equal(got[r], ref[r], f"rank {r}")
    assert sent == osent and recv == orecv


@pytest.mark.parametrize("n", [32, 64])
@pytest.mark.parametrize("algo", ["fused", "stepwise"])
def test_broadcast_and_allgather_many_ranks_match_oracle(n, algo):
    """A fan-out to 63 destinations (the whole 64-bit destination mask)."""
    xs = inputs.filler(n, 5003, salt=n)
    ref = [x.copy() for x in xs]
    osent, orecv = oracle.broadcast(ref, root=n - 1)
    bufs = to_dev(xs, "f32")
    rar.broadcast_ex(bufs, n - 1, ALGOS[algo])
    assert rar.last_traffic(n) == (osent, orecv)
    got = to_host(bufs, "f32")
    for r in range(n):
        assert_bits_equal(got[r], ref[r], f"broadcast rank {r}")
    xs = inputs.filler(n, n * 1001, salt=n + 1)
    ref = [x.copy() for x in xs]
    osent, orecv = oracle.allgather(ref, dt=_oracle_dt("f32"))
    bufs = to_dev(xs, "f32")
    rar.allgather_ex(bufs, ALGOS[algo])
    assert rar.last_traffic(n) == (osent, orecv)
    got = to_host(bufs, "f32")
    for r in range(n):
        assert_bits_equal(got[r], ref[r], f"allgather rank {r}")


def test_unaligned_shards_copy_exactly():
    """Shards whose byte offsets are not 16-byte aligned (head/tail paths)."""
    n, shard = 4, 37
    xs = inputs.filler(n, n * shard, dtype="f16", salt=1)
    ref = [x.copy() for x in xs]
    oracle.allgather(ref)
    bufs = to_dev(xs, "f16")
    rar.allgather(bufs)
    got = to_host(bufs, "f16")
    for r in range(n):
        assert_bits_equal(got[r], ref[r], f"rank {r}")


def test_empty_and_single_rank_are_noops():
    import torch
    xs = _inputs(3, 1000, "f32", salt=3)
    one = to_dev(xs[:1], "f32")
    rar.ring_allreduce(one)
    assert_bits_equal(to_host(one, "f32")[0], xs[0], "N=1")
    empty = [torch.empty(0, device="cuda:0") for _ in range(3)]
    rar.ring_allreduce(empty)


def test_ring_int_workload_exact():
    """N=4, T=1,048,576 integer-valued fp32: exact sums, equal to the brute-force sum."""
    w = inputs.WORKLOADS["ring_int"]
    xs = inputs.integers(w["n"], w["count"])
    exact = np.sum(np.stack([x.astype(np.float64) for x in xs]), axis=0)
    bufs = to_dev(xs, "f32")
    rar.ring_allreduce(bufs)
    for g in to_host(bufs, "f32"):
        assert np.array_equal(g.astype(np.float64), exact)
    sent, recv = rar.last_traffic(w["n"])
    S = w["count"] * 4
    assert sent == recv == [2 * S * (w["n"] - 1) // w["n"]] * w["n"]


@pytest.mark.slow
def test_ring_grad_workload_full_size():
    """N=8, T=64M fp32 (256 MiB per rank) in the fused launch the benchmark
    times: every element of every rank bit-exact against the oracle."""
    w = inputs.WORKLOADS["ring_grad"]
    xs = inputs.gradient_like(w["n"], w["count"])
    bufs = to_dev(xs, "f32")
    rar.ring_allreduce(bufs)
    got = to_host(bufs, "f32")
    del bufs
    oracle.ring_allreduce(xs)
    for r in range(w["n"]):
        assert_bits_equal(got[r], xs[r], f"rank {r}")


@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_16bit_rounding_edge_pairs_match_oracle(dt):
    """Pairs whose binary32 sums sit on rounding ties, in the subnormal range,
    at the overflow boundary and on cancellations: with N=2 every element is
    one local + received add, rounded to the 16-bit type."""
    import torch
    g = np.random.default_rng(21)
    n = 1 << 16
    if dt == "f16":
        a = g.integers(0, 1 << 16, size=n, dtype=np.uint32).astype(np.uint16).view(np.float16)
        b = g.integers(0, 1 << 16, size=n, dtype=np.uint32).astype(np.uint16).view(np.float16)
        fin = np.isfinite(a) & np.isfinite(b)
        a, b = a[fin].copy(), b[fin].copy()
        tiny = (g.integers(0, 1024, size=4096).astype(np.uint16) | (g.integers(0, 2, 4096).astype(np.uint16) << 15))
        a = np.concatenate([a, tiny.view(np.float16), np.full(64, 65504, np.float16)])
        b = np.concatenate([b, tiny[::-1].copy().view(np.float16), np.full(64, 16, np.float16)])
    else:
        bits_a = g.integers(0, 1 << 16, size=n, dtype=np.uint32).astype(np.uint16)
        bits_b = g.integers(0, 1 << 16, size=n, dtype=np.uint32).astype(np.uint16)
        fa = (bits_a.astype(np.uint32) << 16).view(np.float32)
        fb = (bits_b.astype(np.uint32) << 16).view(np.float32)
        fin = np.isfinite(fa) & np.isfinite(fb)
        a, b = bits_a[fin].copy(), bits_b[fin].copy()
        # same-binade pairs whose sums land on bf16 ties, and bf16 subnormals
        base = (g.integers(0x3f80, 0x4000, size=4096)).astype(np.uint16)
        a = np.concatenate([a, base, (g.integers(0, 0x80, 4096)).astype(np.uint16), np.full(64, 0x7f7f, np.uint16)])
        b = np.concatenate([b, (base ^ 1).astype(np.uint16), (g.integers(0, 0x80, 4096)).astype(np.uint16),
                            np.full(64, 0x7f7f, np.uint16)])
    ref = [a.copy(), b.copy()]
    oracle.ring_allreduce(ref, dt=DT_NAMES[dt])
    bufs = to_dev([a, b], dt)
    rar.ring_allreduce(bufs)
    got = to_host(bufs, dt)
    for r in range(2):
        assert_bits_equal(got[r], ref[r], f"rank {r}")
