"""GPU parity of the bucketed allreduce (greedy ~25 MB buckets, one ring
allreduce per bucket) against the oracle."""
import numpy as np
import pytest
import torch

import oracle
import ring_all_reduce_scatter_amd as rar
from ring_all_reduce_scatter_amd import inputs

from gpu_util import DT_NAMES, assert_bits_equal, to_dev, to_host

pytestmark = pytest.mark.gpu


def _run(tensors_host, dt, cap, algo=rar.ALGO_FUSED):
    n, nt = len(tensors_host), len(tensors_host[0])
    dev = [to_dev(tensors_host[r], dt) for r in range(n)]
    counts = [t.size for t in tensors_host[0]]
    ws = torch.empty(rar.bucketed_workspace_bytes(counts, n, DT_NAMES[dt], cap, algo), dtype=torch.uint8,
                     device="cuda:0")
    rar.bucketed_allreduce(dev, cap, ws, algo=algo)
    sent, recv = rar.last_traffic(n)
    return [to_host(dev[r], dt) for r in range(n)], sent, recv


@pytest.mark.parametrize("dt", ["bf16", "f32", "f16"])
@pytest.mark.parametrize("n", [2, 3, 4, 8, 16])
@pytest.mark.parametrize("algo", [rar.ALGO_FUSED, rar.ALGO_STEPWISE])
def test_bucketed_matches_oracle(dt, n, algo):
    sizes = inputs.bucket_sizes(40, lo_exp=3, hi_exp=15, salt=n)
    th = inputs.bucket_tensors(n, sizes, dtype=dt, salt=n)
    ref = [[t.copy() for t in th[r]] for r in range(n)]
    cap = 64 << 10
    osent, orecv = oracle.bucketed_allreduce(ref, cap, dt=DT_NAMES[dt])
    got, sent, recv = _run(th, dt, cap, algo)
    for r in range(n):
        for t in range(len(sizes)):
            assert_bits_equal(got[r][t], ref[r][t], f"rank {r} tensor {t}")
    assert sent == osent and recv == orecv


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("n", [24, 32, 64])
def test_bucketed_fold_multiple_of_8_ranks_matches_oracle(dt, n):
    """Rank counts that are multiples of 8 above 16: the fold's workgroup
    slots map XCD-major, each XCD taking N/8 chunks one after the other;
    every chunk's tiles must still be folded exactly once."""
    sizes = inputs.bucket_sizes(24, lo_exp=3, hi_exp=14, salt=n)
    th = inputs.bucket_tensors(n, sizes, dtype=dt, salt=n)
    ref = [[t.copy() for t in th[r]] for r in range(n)]
    cap = 48 << 10
    osent, orecv = oracle.bucketed_allreduce(ref, cap, dt=DT_NAMES[dt])
    got, sent, recv = _run(th, dt, cap)
    for r in range(n):
        for t in range(len(sizes)):
            assert_bits_equal(got[r][t], ref[r][t], f"rank {r} tensor {t}")
    assert sent == osent and recv == orecv


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("algo", [rar.ALGO_FUSED, rar.ALGO_STEPWISE])
def test_bucketed_with_empty_tensors_matches_oracle(dt, algo):
    """Zero-length tensors between, before and after others (they share a
    flat offset with their neighbour inside a bucket) change nothing."""
    n = 4
    sizes = [0, 5, 0, 300, 0, 0, 2049, 7, 0, 4096 * 3 + 1, 0, 16, 0]
    th = inputs.bucket_tensors(n, sizes, dtype=dt, salt=5)
    ref = [[t.copy() for t in th[r]] for r in range(n)]
    cap = 4096
    osent, orecv = oracle.bucketed_allreduce(ref, cap, dt=DT_NAMES[dt])
    got, sent, recv = _run(th, dt, cap, algo)
    for r in range(n):
        for t in range(len(sizes)):
            assert_bits_equal(got[r][t], ref[r][t], f"rank {r} tensor {t}")
    assert sent == osent and recv == orecv


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("n", [4, 16])
def test_bucketed_in_rank_arena_matches_oracle(dt, n):
    """The placement the benchmark uses (rank_tensors: every rank's tensors in
    one region, regions a power of two apart, tensors 256-element aligned)
    gives the oracle's bits too, for both schedules."""
    sizes = inputs.bucket_sizes(30, lo_exp=2, hi_exp=15, salt=10 + n)
    th = inputs.bucket_tensors(n, sizes, dtype=dt, salt=10 + n)
    ref = [[t.copy() for t in th[r]] for r in range(n)]
    cap = 48 << 10
    osent, orecv = oracle.bucketed_allreduce(ref, cap, dt=DT_NAMES[dt])
    tdt = {"bf16": torch.bfloat16, "f32": torch.float32}[dt]
    for algo in (rar.ALGO_FUSED, rar.ALGO_STEPWISE):
        arena, dev = rar.rank_tensors(n, sizes, tdt, "cuda:0")
        for r in range(n):
            for x, h in zip(dev[r], to_dev(th[r], dt)):
                x.copy_(h)
        ws = torch.empty(rar.bucketed_workspace_bytes(sizes, n, DT_NAMES[dt], cap, algo), dtype=torch.uint8,
                         device="cuda:0")
        rar.bucketed_allreduce(dev, cap, ws, algo=algo)
        sent, recv = rar.last_traffic(n)
        for r in range(n):
            got = to_host(dev[r], dt)
            for t in range(len(sizes)):
                assert_bits_equal(got[t], ref[r][t], f"algo {algo} rank {r} tensor {t}")
        assert sent == osent and recv == orecv


@pytest.mark.slow
def test_buckets_workload_full_size():
    """N=16 bf16, 200 log-uniform tensors (234,101,211 elements per rank),
    22 buckets of at most 25 MiB, in the placement the benchmark uses: every
    element of every tensor on every rank equals the oracle's (each bucket
    allreduced by the oracle on its own, on host threads), and the byte
    counters equal the oracle's."""
    import full_size
    w = inputs.WORKLOADS["buckets"]
    n, cap = w["n"], w["cap_bytes"]
    sizes = inputs.bucket_sizes(w["ntensors"])
    th = inputs.bucket_tensors(n, sizes)
    arena, dev = rar.rank_tensors(n, sizes, torch.bfloat16, "cuda:0")
    for r in range(n):
        for x, h in zip(dev[r], to_dev(th[r], "bf16")):
            x.copy_(h)
    ws = torch.empty(rar.bucketed_workspace_bytes(sizes, n, rar.BF16, cap), dtype=torch.uint8, device="cuda:0")
    rar.bucketed_allreduce(dev, cap, ws)
    sent, recv = rar.last_traffic(n)
    want, osent, orecv, nb = full_size.bucketed(th, cap, dt=oracle.BF16)
    assert nb == 22
    for r in range(n):
        got = to_host(dev[r], "bf16")
        for t in range(len(sizes)):
            assert_bits_equal(got[t], want[t], f"rank {r} tensor {t}")
    assert sent == osent and recv == orecv


def test_bucketed_large_tensors_both_schedules_agree():
    """Tensors big enough for full vector tiles, with ragged sizes."""
    n = 8
    sizes = [70_001, 3, 250_000, 128, 99_999, 1 << 17]
    th = inputs.bucket_tensors(n, sizes, dtype="f32", salt=11)
    ref = [[t.copy() for t in th[r]] for r in range(n)]
    cap = 1 << 20
    oracle.bucketed_allreduce(ref, cap)
    for algo in (rar.ALGO_FUSED, rar.ALGO_STEPWISE):
        got, _, _ = _run(th, "f32", cap, algo)
        for r in range(n):
            for t in range(len(sizes)):
                assert_bits_equal(got[r][t], ref[r][t], f"algo {algo} rank {r} tensor {t}")


def test_prepared_bucketed_allreduce_repeats():
    """BucketedAllreduce marshals the pointer table once; two calls on restored
    inputs give the one-shot call's bits both times."""
    n = 4
    sizes = inputs.bucket_sizes(30, lo_exp=3, hi_exp=14, salt=9)
    th = inputs.bucket_tensors(n, sizes, dtype="bf16", salt=9)
    cap = 32 << 10
    want, _, _ = _run(th, "bf16", cap)
    dev = [to_dev(th[r], "bf16") for r in range(n)]
    pristine = [to_dev(th[r], "bf16") for r in range(n)]
    ws = torch.empty(rar.bucketed_workspace_bytes(sizes, n, rar.BF16, cap), dtype=torch.uint8, device="cuda:0")
    step = rar.BucketedAllreduce(dev, cap, ws)
    for call in range(2):
        for r in range(n):
            for t, p in zip(dev[r], pristine[r]):
                t.copy_(p)
        step()
        for r in range(n):
            got = to_host(dev[r], "bf16")
            for t in range(len(sizes)):
                assert_bits_equal(got[t], want[r][t], f"call {call} rank {r} tensor {t}")


@pytest.mark.parametrize("dt,n", [("bf16", 16), ("f32", 3), ("f16", 8)])
def test_prepared_plan_launches_match_oracle(dt, n):
    """rar_bucketed_prepare once, rar_bucketed_launch twice on restored
    inputs, then a second, smaller tensor set prepared into the same
    workspace and launched: every launch gives the oracle's bits and the
    oracle's byte counters."""
    def run_set(sizes, salt, ws):
        th = inputs.bucket_tensors(n, sizes, dtype=dt, salt=salt)
        ref = [[t.copy() for t in th[r]] for r in range(n)]
        osent, orecv = oracle.bucketed_allreduce(ref, cap, dt=DT_NAMES[dt])
        dev = [to_dev(th[r], dt) for r in range(n)]
        pristine = [to_dev(th[r], dt) for r in range(n)]
        step = rar.BucketedAllreduce(dev, cap, ws)
        for call in range(2):
            for r in range(n):
                for t, p in zip(dev[r], pristine[r]):
                    t.copy_(p)
            step()
            assert rar.last_traffic(n) == (osent, orecv)
            for r in range(n):
                got = to_host(dev[r], dt)
                for t in range(len(sizes)):
                    assert_bits_equal(got[t], ref[r][t], f"set {salt} call {call} rank {r} tensor {t}")

    cap = 48 << 10
    big = inputs.bucket_sizes(50, lo_exp=3, hi_exp=15, salt=20 + n)
    small = inputs.bucket_sizes(12, lo_exp=3, hi_exp=12, salt=40 + n)
    need = max(rar.bucketed_workspace_bytes(s, n, DT_NAMES[dt], cap) for s in (big, small))
    ws = torch.empty(need, dtype=torch.uint8, device="cuda:0")
    run_set(big, 20 + n, ws)
    run_set(small, 40 + n, ws)
