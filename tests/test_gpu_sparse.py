"""GPU parity of the sparsity-aware compressed ring (values + uint32 indices
when a unit's zeros exceed the threshold, BFP otherwise) against the oracle,
bit for bit, and of the sparse + 4-bit workload with its broadcast and
allgather legs."""
import numpy as np
import pytest
import torch

import oracle
import ring_all_reduce_scatter_amd as rar
from ring_all_reduce_scatter_amd import inputs

from gpu_util import DT_NAMES, assert_bits_equal, nan_mask, to_dev, to_host

pytestmark = pytest.mark.gpu


SCHEDS = {"staged": rar.SCHED_STAGED, "pipelined": rar.SCHED_PIPELINED}


def _run_auto(xs, dt, mbits=4, unit_elems=4096, theta=0.5, block=128, sched="staged"):
    n, count = len(xs), xs[0].size
    es = 4 if dt == "f32" else 2
    cfg = rar.compress_cfg(method=rar.COMP_SPARSE_AUTO, mbits=mbits, block=block, unit_bytes=unit_elems * es,
                           sparsity_threshold=theta, schedule=SCHEDS[sched])
    ws = torch.empty(rar.compressed_workspace_bytes(n, count, DT_NAMES[dt], cfg), dtype=torch.uint8, device="cuda:0")
    bufs = to_dev(xs, dt)
    rar.ring_allreduce_compressed(bufs, cfg, ws)
    sent, recv = rar.compressed_traffic(ws, n)
    return to_host(bufs, dt), sent, recv


@pytest.mark.parametrize("sched", ["staged", "pipelined"])
@pytest.mark.parametrize("dt", ["f16", "bf16", "f32"])
@pytest.mark.parametrize("n", [1, 2, 3, 4, 8])
@pytest.mark.parametrize("mbits", [4, 8])
def test_sparse_auto_matches_oracle(dt, n, mbits, sched):
    count = n * 4096 * 3 + 2500  # several units and tiles per chunk, ragged last chunk
    xs = inputs.sparse_mix(n, count, dtype=dt, salt=n + mbits)
    ref = [x.copy() for x in xs]
    osent, orecv = oracle.ring_allreduce_compressed(ref, method=oracle.COMP_SPARSE_AUTO, mbits=mbits, unit=4096,
                                                    dt=DT_NAMES[dt])
    got, sent, recv = _run_auto(xs, dt, mbits=mbits, sched=sched)
    for r in range(n):
        assert_bits_equal(got[r], ref[r], f"rank {r}")
    assert sent == osent and recv == orecv


@pytest.mark.parametrize("sched", ["staged", "pipelined"])
@pytest.mark.parametrize("dt", ["f16", "f32"])
@pytest.mark.parametrize("n", [6, 16, 64])
def test_sparse_auto_more_ranks_matches_oracle(dt, n, sched):
    """SPARSE_AUTO over 6, 16 and 64 ranks: the pipelined gang protocol with
    more hops per unit, half the ranks sparse."""
    count = n * 4096 * 2 + 1500
    xs = inputs.sparse_mix(n, count, dtype=dt, salt=100 + n)
    ref = [x.copy() for x in xs]
    osent, orecv = oracle.ring_allreduce_compressed(ref, method=oracle.COMP_SPARSE_AUTO, mbits=4, unit=4096,
                                                    dt=DT_NAMES[dt])
    got, sent, recv = _run_auto(xs, dt, mbits=4, sched=sched)
    for r in range(n):
        assert_bits_equal(got[r], ref[r], f"rank {r}")
    assert sent == osent and recv == orecv


@pytest.mark.parametrize("sched", ["staged", "pipelined"])
@pytest.mark.parametrize("n", [2, 4, 8])
def test_all_sparse_equals_uncompressed_ring(n, sched):
    count = n * 8192
    xs = inputs.sparse_mix(n, count, sparse_ranks=n, density=0.01, salt=n)
    ref = [x.copy() for x in xs]
    oracle.ring_allreduce(ref)
    got, _, _ = _run_auto(xs, "f16", sched=sched)
    for r in range(n):
        assert np.array_equal(got[r], ref[r])  # lossless (+0 == -0)


@pytest.mark.parametrize("sched", ["staged", "pipelined"])
@pytest.mark.parametrize("theta", [0.1, 0.5, 0.9])
def test_threshold_values_match_oracle(theta, sched):
    n, count = 4, 4 * 6144
    xs = inputs.sparse_mix(n, count, sparse_ranks=2, density=0.3, salt=int(theta * 10))
    ref = [x.copy() for x in xs]
    osent, _ = oracle.ring_allreduce_compressed(ref, method=oracle.COMP_SPARSE_AUTO, mbits=4, unit=2048, theta=theta)
    got, sent, _ = _run_auto(xs, "f16", unit_elems=2048, theta=theta, sched=sched)
    for r in range(n):
        assert_bits_equal(got[r], ref[r], f"rank {r}")
    assert sent == osent


def _same_zero_ranks(n, unit, zeros, units, seed=70):
    """Every unit has the same `zeros` positions at +0 on every rank and
    positive values elsewhere, so every partial sum keeps exactly them."""
    g = np.random.default_rng(seed)
    mask = np.ones(units * unit, dtype=bool)
    for u in range(units):
        mask[u * unit + g.choice(unit, size=zeros, replace=False)] = False
    return [np.where(mask, g.uniform(0.25, 1.0, size=units * unit).astype(np.float16), np.float16(0)).astype(np.float16)
            for _ in range(n)]


@pytest.mark.parametrize("sched", ["staged", "pipelined"])
@pytest.mark.parametrize("n", [2, 4])
@pytest.mark.parametrize("unit,zeros,block", [(640, 448, 128), (80, 56, 16)])
def test_threshold_binary32_boundary_matches_oracle(n, unit, zeros, block, sched):
    """theta = 0.7 with exactly 0.7 * len zeros per unit: the binary32
    threshold (0.699999988...) sends every message sparse.  Library and
    oracle must take the same decision: results bit-exact, byte counters
    equal, and every message sparse (lossless: the plain ring's sums)."""
    L = 640
    xs = _same_zero_ranks(n, unit, zeros, n * L // unit, seed=70 + n)
    ref = [x.copy() for x in xs]
    osent, orecv = oracle.ring_allreduce_compressed(ref, method=oracle.COMP_SPARSE_AUTO, block=block, mbits=4,
                                                    unit=unit, theta=0.7)
    got, sent, recv = _run_auto(xs, "f16", unit_elems=unit, theta=0.7, block=block, sched=sched)
    for r in range(n):
        assert_bits_equal(got[r], ref[r], f"rank {r}")
    assert sent == osent and recv == orecv
    nnz = unit - zeros
    sparse_msg = 16 + -(-nnz * 2 // 16) * 16 + 4 * nnz
    assert sent == [2 * (n - 1) * (L // unit) * sparse_msg] * n
    plain = [x.copy() for x in xs]
    oracle.ring_allreduce(plain)
    for r in range(n):
        assert np.array_equal(got[r], plain[r])


@pytest.mark.parametrize("sched", ["staged", "pipelined"])
def test_exactly_half_zeros_goes_bfp(sched):
    unit = 256
    x0 = np.zeros(2 * unit, dtype=np.float16)
    x1 = np.zeros(2 * unit, dtype=np.float16)
    x0[: unit - 129] = 1.0
    x0[unit: unit + unit // 2] = 1.0
    ref = [x0.copy(), x1.copy()]
    osent, orecv = oracle.ring_allreduce_compressed(ref, method=oracle.COMP_SPARSE_AUTO, mbits=4, unit=unit)
    got, sent, recv = _run_auto([x0, x1], "f16", unit_elems=unit, sched=sched)
    assert sent == osent and recv == orecv
    for r in range(2):
        assert_bits_equal(got[r], ref[r], f"rank {r}")


@pytest.mark.slow
@pytest.mark.parametrize("sched", ["staged", "pipelined"])
def test_sparse_bfp4_workload_full_size(sched):
    """N=8, T=64M fp16, ranks 0-3 95% zeros, dense BFP-4, 4 MiB units, both
    schedules: every element of every rank equals the oracle's (the whole
    workload on host threads, one unit index at a time) and so do the byte
    counters, which show which messages went sparse."""
    import full_size
    w = inputs.WORKLOADS["sparse_bfp4"]
    n, count, mbits = w["n"], w["count"], w["mbits"]
    U = w["unit_bytes"] // 2
    xs = inputs.sparse_mix(n, count)
    got, sent, recv = _run_auto(xs, "f16", mbits=mbits, unit_elems=U, sched=sched)
    for r in range(1, n):
        assert np.array_equal(got[r].view(np.uint16), got[0].view(np.uint16)), r
    L = rar.compressed_chunk_len(count, n, 128)
    want, osent, orecv, _ = full_size.compressed_ring(xs, L, U, method=oracle.COMP_SPARSE_AUTO, mbits=mbits,
                                                       theta=w["theta"])
    assert_bits_equal(got[0], want, "rank 0")
    assert sent == osent and recv == orecv
    # wire bytes well under the uncompressed ring's 2*S*(N-1)/N per rank
    assert max(sent) < 2 * count * 2 * (n - 1) // n * 0.6


@pytest.mark.slow
def test_sparse_bfp4_workload_broadcast_and_allgather_full_size():
    """Broadcast of a 16M fp32 tensor from rank 0 and allgather of 16M fp32
    shards over 8 ranks (both uncompressed: the operator-aware policy keeps
    them lossless), bit-exact against the oracle."""
    w = inputs.WORKLOADS["sparse_bfp4"]
    n = w["n"]
    xs = inputs.filler(n, w["bcast_count"], salt=1)
    ref = [x.copy() for x in xs]
    oracle.broadcast(ref, root=0)
    bufs = to_dev(xs, "f32")
    rar.broadcast(bufs, 0)
    for r, g in enumerate(to_host(bufs, "f32")):
        assert_bits_equal(g, ref[r], f"broadcast rank {r}")
    del bufs
    shard = w["ag_shard"]
    xs = inputs.filler(n, n * shard, salt=2)
    ref = [x.copy() for x in xs]
    oracle.allgather(ref)
    bufs = to_dev(xs, "f32")
    rar.allgather(bufs)
    for r, g in enumerate(to_host(bufs, "f32")):
        assert_bits_equal(g, ref[r], f"allgather rank {r}")


@pytest.mark.parametrize("dt", ["f16", "f32"])
def test_pipelined_sparse_messages_match_oracle(dt):
    """Every message the pipelined SPARSE_AUTO schedule leaves in its slots
    (hop h of chunk c, unit u) equals the oracle's encode of that hop's
    partial: built hop by hop from the oracle's sparse and BFP primitives,
    with the unit's format chosen by the oracle's threshold rule.  In a
    slot, a sparse message's body follows the BFP area."""
    n, U, mbits, theta = 4, 8192, 4, 0.5
    es = 4 if dt == "f32" else 2
    count = n * 2 * U + 3000
    xs = inputs.sparse_mix(n, count, sparse_ranks=2, density=0.3, dtype=dt, salt=5)
    cfg = rar.compress_cfg(method=rar.COMP_SPARSE_AUTO, mbits=mbits, unit_bytes=U * es, sparsity_threshold=theta,
                           schedule=rar.SCHED_PIPELINED)
    ws = torch.empty(rar.compressed_workspace_bytes(n, count, DT_NAMES[dt], cfg), dtype=torch.uint8,
                     device="cuda:0")
    bufs = to_dev(xs, dt)
    rar.ring_allreduce_compressed(bufs, cfg, ws)
    host = ws.cpu().numpy()
    L = rar.compressed_chunk_len(count, n, 128)
    upc = -(-L // U)
    # a slot: header, the BFP area, then room for the all-non-zero sparse
    # body, which starts after the BFP area
    slot = -(-(16 + -(-rar.bfp_bytes(U, 128, mbits) // 16) * 16 + (-(-U * es // 16) * 16) + 4 * U) // 256) * 256
    odt = DT_NAMES[dt]
    checked = 0
    for c in range(n):
        lo, hi = min(c * L, count), min((c + 1) * L, count)
        for u in range(upc):
            ulo = lo + u * U
            if ulo >= hi:
                break
            ln = min(U, hi - ulo)
            p = xs[(c + 1) % n][ulo:ulo + ln].copy()
            for h in range(1, n + 1):
                zeros = int(np.count_nonzero(p == 0))
                if zeros > np.float64(np.float32(theta)) * ln:
                    body = oracle.sparse_encode(p, odt)
                    want = np.concatenate([body[:16], body[16:]])
                    kind = 1
                else:
                    body = oracle.bfp_encode(p, block=128, mbits=mbits, dt=odt)
                    want = np.concatenate([np.array([0, 0, 0, 0, 0, 0, 0, 0, ln & 0xff, (ln >> 8) & 0xff,
                                                     (ln >> 16) & 0xff, ln >> 24, 0, 0, 0, 0], np.uint8), body])
                    kind = 0
                base = 1024 + (((h - 1) * n + c) * upc + u) * slot
                if kind == 1:
                    spoff = 16 + -(-rar.bfp_bytes(ln, 128, mbits) // 16) * 16
                    got = np.concatenate([host[base:base + 16], host[base + spoff:base + spoff + want.size - 16]])
                else:
                    got = host[base:base + want.size]
                bad = np.flatnonzero(got != want)
                assert bad.size == 0, f"hop {h} chunk {c} unit {u} kind {kind}: {bad.size} bytes differ at {bad[:4]}"
                checked += 1
                if h < n:
                    nxt = xs[(c + h + 1) % n][ulo:ulo + ln].copy()
                    if kind == 1:
                        oracle.sparse_decode_acc(body, nxt, odt)
                    else:
                        oracle.bfp_decode_acc(body, nxt, block=128, mbits=mbits, dt=odt)
                    p = nxt
    assert checked > 0
    ref = [x.copy() for x in xs]
    oracle.ring_allreduce_compressed(ref, method=oracle.COMP_SPARSE_AUTO, mbits=mbits, unit=U, dt=odt)
    for r, g in enumerate(to_host(bufs, dt)):
        assert_bits_equal(g, ref[r], f"rank {r}")


@pytest.mark.parametrize("dt", ["f16", "bf16"])
@pytest.mark.parametrize("mbits", [4, 8])
def test_pipelined_sparse_special_values_match_oracle(dt, mbits):
    """Sparse and BFP units holding Inf, NaN, subnormals and the largest
    binary16 values, with a ragged last chunk, through the pipelined
    SPARSE_AUTO ring: results equal the oracle's (NaN where the oracle has
    NaN), and so do the byte counters."""
    n, U = 4, 4096
    count = n * 2 * U + 700
    g = np.random.default_rng(100 + mbits)
    xs = []
    for r in range(n):
        x = (g.standard_normal(count) * 1e-2).astype(np.float32)
        if r < 2:  # sparse ranks: the first hops of their chunks go as values + indices
            x[g.random(count) < 0.97] = 0.0
        x[0:128] = 0.0
        x[128:256] = np.float32(6.0e-8) * g.integers(-3, 4, 128)  # binary16 subnormals
        x[256:384] = np.float32(65504.0) * np.sign(g.standard_normal(128)).astype(np.float32) / n
        if r == 1:
            x[384 + 5] = np.inf          # in a sparse rank's values
            x[3 * U + 9] = -np.inf
        if r == 3:
            x[2 * U + 7] = np.nan        # in a dense unit
            x[count - 3] = np.nan        # in the ragged tail
        xs.append(inputs.cast(x, dt))
    ref = [x.copy() for x in xs]
    osent, orecv = oracle.ring_allreduce_compressed(ref, method=oracle.COMP_SPARSE_AUTO, mbits=mbits, unit=U,
                                                    dt=DT_NAMES[dt])
    got, sent, recv = _run_auto(xs, dt, mbits=mbits, unit_elems=U, sched="pipelined")
    for r in range(n):
        nan = nan_mask(ref[r], dt)
        assert np.array_equal(nan_mask(got[r], dt), nan), f"rank {r} NaN positions"
        assert_bits_equal(got[r][~nan], ref[r][~nan], f"rank {r}")
    assert sent == osent and recv == orecv


@pytest.mark.parametrize("dt", ["f16", "bf16", "f32"])
@pytest.mark.parametrize("pattern", ["one_dense_tile", "one_zero_tile"])
def test_pipelined_sparse_tiles_unlike_their_unit_match_oracle(dt, pattern):
    """Units of four tiles of the pipelined kernel in which one tile differs
    from the rest: a dense tile in a unit that goes sparse (the tile's own
    count says BFP, so it writes its BFP part before it learns the unit's
    decision and then writes its sparse part), or an all-zero tile in a unit
    that goes BFP.  Every hop's message has that shape; results and byte
    counters equal the oracle's."""
    n, mbits = 4, 4
    tile = 16384 if dt != "f32" else 8192  # elements per workgroup tile of the pipelined kernel
    U = 4 * tile
    count = n * 2 * U + 777
    L = rar.compressed_chunk_len(count, n, 128)
    g = np.random.default_rng(7)
    special = np.zeros(count, dtype=bool)  # the differing tile of every unit
    for c in range(n):
        for u in range(-(-L // U)):
            a = c * L + u * U
            special[min(a, count):min(a + tile, count, (c + 1) * L)] = True
    xs = []
    for r in range(n):
        x = (g.standard_normal(count) * 1e-2).astype(np.float32)
        x[x == 0] = np.float32(1e-3)  # no accidental zeros in the dense parts
        x[~special if pattern == "one_dense_tile" else special] = 0.0
        xs.append(inputs.cast(x, dt))
    ref = [x.copy() for x in xs]
    osent, orecv = oracle.ring_allreduce_compressed(ref, method=oracle.COMP_SPARSE_AUTO, mbits=mbits, unit=U,
                                                    dt=DT_NAMES[dt])
    got, sent, recv = _run_auto(xs, dt, mbits=mbits, unit_elems=U, sched="pipelined")
    for r in range(n):
        assert_bits_equal(got[r], ref[r], f"rank {r}")
    assert sent == osent and recv == orecv
