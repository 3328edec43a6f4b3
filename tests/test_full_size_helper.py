"""The piecewise oracle runs of tests/full_size.py equal one oracle run over
the whole buffers (bits, byte counters, block maxima, state), so the
full-size GPU tests compare against the oracle itself.  CPU only."""
import numpy as np
import pytest

from ring_all_reduce_scatter_amd import inputs

import full_size


@pytest.mark.parametrize("method,mbits", [(1, 8), (1, 4), (2, 4)])
@pytest.mark.parametrize("n", [2, 3, 8])
def test_unit_pieces_equal_whole_ring(orc, method, mbits, n):
    U = 2048
    L = 3 * U
    count = n * L
    if method == 2:
        xs = inputs.sparse_mix(n, count, sparse_ranks=max(1, n // 2), density=0.2, salt=n)
    else:
        xs = inputs.block_scaled(n, count, salt=n + mbits)
    whole = [x.copy() for x in xs]
    s, r, bm = orc.ring_allreduce_compressed(whole, method=method, mbits=mbits, unit=U, with_blockmax=True)
    got, gs, gr, gbm = full_size.compressed_ring(xs, L, U, method=method, mbits=mbits, with_blockmax=True)
    assert np.array_equal(got.view(np.uint16), whole[0].view(np.uint16))
    assert gs == s and gr == r
    assert np.array_equal(gbm, bm)


@pytest.mark.parametrize("fb", [1, 2])
def test_unit_pieces_equal_whole_stateful_ring(orc, fb):
    n, U = 4, 1024
    L = 2 * U
    xs = inputs.block_scaled(n, n * L, salt=fb)
    st_whole = [np.zeros(n * L, np.float32) for _ in range(n)]
    for _ in range(2):
        whole = [x.copy() for x in xs]
        orc.ring_allreduce_compressed_state(whole, st_whole, fb, unit=U)
    got, st = full_size.compressed_ring_state(xs, [np.zeros(n * L, np.float32) for _ in range(n)], L, U, fb, 2)
    assert np.array_equal(got.view(np.uint16), whole[0].view(np.uint16))
    for a, b in zip(st, st_whole):
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_bucket_pieces_equal_whole_bucketed(orc):
    n = 4
    sizes = inputs.bucket_sizes(40, lo_exp=3, hi_exp=14, salt=7)
    th = inputs.bucket_tensors(n, sizes, dtype="bf16", salt=7)
    whole = [[t.copy() for t in th[r]] for r in range(n)]
    cap = 40 << 10
    s, r = orc.bucketed_allreduce(whole, cap, dt=orc.BF16)
    got, gs, gr, nb = full_size.bucketed(th, cap, dt=orc.BF16)
    assert nb > 3
    for t in range(len(sizes)):
        assert np.array_equal(got[t], whole[0][t])
    assert gs == s and gr == r
