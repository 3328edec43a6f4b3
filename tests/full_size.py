"""Whole-workload oracle runs for the full-size GPU parity tests.

The oracle is plain single-threaded C.  A compressed ring splits exactly into
independent pieces, so the full workloads are run piece by piece on a pool
of host threads (ctypes releases the GIL inside the C calls):

* Compressed ring (BFP or SPARSE_AUTO), chunk length L and unit U with
  L % U == 0: unit u of every chunk forms a ring of its own.  The piece
  for unit u holds, for every rank, the N units u of chunks 0..N-1 back to
  back, so its chunk c (length U) is chunk c's unit u: the same ring order,
  the same messages (one per unit and hop), the same results and byte
  counts.  The N pieces' counters add up to the whole ring's.
* Stateful BFP ring: the same pieces, with the state sliced alike.
* Bucketed allreduce: every bucket is an allreduce of its own.
"""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

import oracle


def workers():
    return max(1, min(16, os.cpu_count() or 1))


def _unit_slices(count, n, L, U):
    assert L % U == 0 and count == n * L, "pieces need whole units in equal chunks"
    upc = L // U
    return [[slice(c * L + u * U, c * L + (u + 1) * U) for c in range(n)] for u in range(upc)]


def compressed_ring(xs, L, U, method=oracle.COMP_BFP, mbits=8, theta=0.5, dt=None, with_blockmax=False):
    """The oracle's compressed ring over the whole of xs (rank 0's result,
    all ranks end equal), summed byte counters and, if asked, the per-block
    max of the messages that carried each block."""
    n, count = len(xs), xs[0].size
    pieces = _unit_slices(count, n, L, U)
    out = np.empty_like(xs[0])
    bm = np.zeros(count // 128, dtype=np.float64) if with_blockmax else None
    sent = np.zeros(n, dtype=np.uint64)
    recv = np.zeros(n, dtype=np.uint64)

    def run(sl):
        mini = [np.concatenate([x[s] for s in sl]) for x in xs]
        r = oracle.ring_allreduce_compressed(mini, method=method, mbits=mbits, theta=theta, unit=U, dt=dt,
                                             with_blockmax=with_blockmax)
        return sl, mini[0], r

    with ThreadPoolExecutor(workers()) as ex:
        for sl, res, r in ex.map(run, pieces):
            for c, s in enumerate(sl):
                out[s] = res[c * U:(c + 1) * U]
                if with_blockmax:
                    bm[s.start // 128:s.stop // 128] = r[2][c * U // 128:(c + 1) * U // 128]
            sent += np.asarray(r[0], dtype=np.uint64)
            recv += np.asarray(r[1], dtype=np.uint64)
    return out, [int(v) for v in sent], [int(v) for v in recv], bm


def compressed_ring_state(xs, states, L, U, feedback, calls, mbits=8, dt=None):
    """`calls` stateful BFP rings over the whole workload, each starting from
    the inputs xs and carrying the state: returns rank 0's last result and
    every rank's final state."""
    n, count = len(xs), xs[0].size
    pieces = _unit_slices(count, n, L, U)
    out = np.empty_like(xs[0])
    st_out = [s.copy() for s in states]

    def run(sl):
        mst = [np.concatenate([s[p] for p in sl]) for s in states]
        mini = None
        for _ in range(calls):
            mini = [np.concatenate([x[p] for p in sl]) for x in xs]
            oracle.ring_allreduce_compressed_state(mini, mst, feedback, mbits=mbits, unit=U, dt=dt)
        return sl, mini[0], mst

    with ThreadPoolExecutor(workers()) as ex:
        for sl, res, mst in ex.map(run, pieces):
            for c, s in enumerate(sl):
                out[s] = res[c * U:(c + 1) * U]
                for r in range(n):
                    st_out[r][s] = mst[r][c * U:(c + 1) * U]
    return out, st_out


def bucketed(tensors, cap, dt=None):
    """Every bucket of the greedy plan allreduced by the oracle on its own;
    returns rank 0's tensors and the summed byte counters."""
    n, nt = len(tensors), len(tensors[0])
    sizes = [t.size for t in tensors[0]]
    dtc = dt if dt is not None else oracle._dt_of(tensors[0][0])
    nb, plan = oracle.bucket_plan(sizes, dtc, cap)
    members = [[t for t in range(nt) if plan[t] == b] for b in range(nb)]
    out = [None] * nt
    sent = np.zeros(n, dtype=np.uint64)
    recv = np.zeros(n, dtype=np.uint64)

    def run(ms):
        sub = [[tensors[r][t].copy() for t in ms] for r in range(n)]
        s, rv = oracle.bucketed_allreduce(sub, cap, dt=dt)
        return ms, sub[0], s, rv

    with ThreadPoolExecutor(workers()) as ex:
        for ms, res, s, rv in ex.map(run, members):
            for k, t in enumerate(ms):
                out[t] = res[k]
            sent += np.asarray(s, dtype=np.uint64)
            recv += np.asarray(rv, dtype=np.uint64)
    return out, [int(v) for v in sent], [int(v) for v in recv], nb
