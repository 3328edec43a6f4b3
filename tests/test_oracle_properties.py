"""Randomised shapes for the oracle's ring (CPU only, hypothesis): any rank
count 1..12, any length 0..6000 (ragged and empty chunks), three dtypes.
Every rank must end with the closed-form fold of its chunk (ranks c+1, ...,
c+N-1, then c, each add local + received in the dtype's arithmetic), the
reduce-scatter must leave chunk r of rank r with that sum, and the byte
counters must add up to the table's totals."""
import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

from ring_all_reduce_scatter_amd import inputs

from test_oracle_ring import closed_form


def _chunk(count, n):
    return (-(-count // n) + 127) // 128 * 128 if n else 0


@settings(max_examples=80, deadline=None)
@given(n=st.integers(1, 12), count=st.integers(0, 6000), dt=st.sampled_from(["f32", "f16"]),
       salt=st.integers(0, 10_000))
def test_ring_matches_closed_form(orc, n, count, dt, salt):
    xs = inputs.gradient_like(n, count, dtype=dt, salt=salt)
    bufs = [x.copy() for x in xs]
    sent, recv = orc.ring_allreduce(bufs)
    if count:
        ref = closed_form(xs, dtype=np.float16 if dt == "f16" else np.float32)
        view = np.uint16 if dt == "f16" else np.uint32
        for b in bufs:
            assert np.array_equal(b.view(view), ref.view(view))
    es = 2 if dt == "f16" else 4
    # every element crosses N-1 links in each pass
    assert sum(sent) == sum(recv) == 2 * (n - 1) * count * es


@settings(max_examples=60, deadline=None)
@given(n=st.integers(2, 12), count=st.integers(1, 6000), salt=st.integers(0, 10_000))
def test_reduce_scatter_owner_chunk(orc, n, count, salt):
    xs = inputs.gradient_like(n, count, salt=salt)
    a = [x.copy() for x in xs]
    orc.reduce_scatter(a)
    b = [x.copy() for x in xs]
    orc.ring_allreduce(b)
    L = _chunk(count, n)
    for r in range(n):
        lo, hi = min(r * L, count), min((r + 1) * L, count)
        assert np.array_equal(a[r][lo:hi].view(np.uint32), b[r][lo:hi].view(np.uint32))
