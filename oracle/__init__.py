"""CPU oracle for the ring all-reduce family (ctypes wrapper over liboracle.so).

TEST INFRASTRUCTURE.  Only the test-suite, the smoke check and the
benchmark's CPU-baseline leg may import this package.  The GPU library never
imports, links or calls it, and it imports nothing from the GPU library.

Every function takes host numpy arrays and runs the plain single-threaded C
reference in oracle.c.  Arrays of dtype float16 are binary16; bfloat16 data
is carried as uint16 bit patterns together with ``dt=BF16``.

Parity status of each function (what pins it is in the tests under
``tests/test_oracle_*.py``):
  f16/bf16 conversions ............ pinned (numpy / torch RNE conversions)
  ring RS / AG / allreduce ........ pinned (brute-force exact sums, closed-form
                                    fold order, post-conditions, byte table,
                                    torch.distributed gloo within float32 eps)
  allgather / broadcast ........... pinned (copies, byte table)
  BFP encode / decode ............. pinned (brute-force optimal rounding,
                                    exponent via frexp, exact round trips,
                                    tight error bound, hand-worked blocks)
  sparse encode / decode .......... pinned (numpy nonzero, round trip)
  compressed ring ................. pinned (integer-input exactness, error bound
                                    vs exact sum, sparse==uncompressed ring)
  bucket plan / bucketed allreduce  pinned (hand-worked plan, greedy rule
                                    properties, exact integer sums)
  stateful BFP ring (error feedback / delta)
                                    pinned (first call = plain BFP ring; exact
                                    conservation of value + residual; 1/T
                                    convergence of the mean; delta coding
                                    converging on constant inputs)
  tree allreduce .................. pinned (exact integer sums, hand-written
                                    balanced-tree expressions, byte counts)
  hash64 / shared-state sync ...... pinned (published splitmix64 outputs,
                                    sensitivity to every bit, position and
                                    length; hand-worked majority cases)
  fault-injected ring ............. pinned (no fault = plain ring; survivors'
                                    result = a fresh ring over the survivors;
                                    exact integer sums; hand-worked attempts
                                    and byte counts; failed ranks restored)
"""
import ctypes
import os

import numpy as np

F32, F16, BF16 = 0, 1, 2
COMP_BFP, COMP_SPARSE_AUTO = 1, 2

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

_c_size = ctypes.c_size_t
_c_vp = ctypes.c_void_p
_u64p = ctypes.POINTER(ctypes.c_uint64)


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import build as _build
        _build.build()
    lib = ctypes.CDLL(_LIB_PATH)
    sig = {
        "orc_f16_to_f32": (ctypes.c_float, [ctypes.c_uint16]),
        "orc_f32_to_f16": (ctypes.c_uint16, [ctypes.c_float]),
        "orc_bf16_to_f32": (ctypes.c_float, [ctypes.c_uint16]),
        "orc_f32_to_bf16": (ctypes.c_uint16, [ctypes.c_float]),
        "orc_chunk_len": (_c_size, [_c_size, ctypes.c_int, _c_size]),
        "orc_comp_chunk_len": (_c_size, [_c_size, ctypes.c_int, ctypes.c_int]),
        "orc_rs_step": (ctypes.c_int, [_c_vp, ctypes.c_int, _c_size, ctypes.c_int, ctypes.c_int]),
        "orc_ag_step": (ctypes.c_int, [_c_vp, ctypes.c_int, _c_size, ctypes.c_int, ctypes.c_int]),
        "orc_reduce_scatter": (ctypes.c_int, [_c_vp, ctypes.c_int, _c_size, ctypes.c_int, _u64p, _u64p]),
        "orc_ring_allreduce": (ctypes.c_int, [_c_vp, ctypes.c_int, _c_size, ctypes.c_int, _u64p, _u64p]),
        "orc_allgather": (ctypes.c_int, [_c_vp, ctypes.c_int, _c_size, ctypes.c_int, _u64p, _u64p]),
        "orc_broadcast": (ctypes.c_int, [_c_vp, ctypes.c_int, _c_size, ctypes.c_int, ctypes.c_int, _u64p, _u64p]),
        "orc_naive_sum_f64": (ctypes.c_int, [_c_vp, ctypes.c_int, _c_size, ctypes.c_int, _c_vp]),
        "orc_bfp_bytes": (_c_size, [_c_size, ctypes.c_int, ctypes.c_int]),
        "orc_bfp_encode": (ctypes.c_int, [_c_vp, ctypes.c_int, _c_size, ctypes.c_int, ctypes.c_int, _c_vp, _c_vp]),
        "orc_bfp_decode_acc": (ctypes.c_int, [_c_vp, _c_size, ctypes.c_int, ctypes.c_int, _c_vp, ctypes.c_int]),
        "orc_bfp_decode": (ctypes.c_int, [_c_vp, _c_size, ctypes.c_int, ctypes.c_int, _c_vp, ctypes.c_int]),
        "orc_sparse_bytes": (_c_size, [_c_size, ctypes.c_int]),
        "orc_count_zeros": (_c_size, [_c_vp, ctypes.c_int, _c_size]),
        "orc_sparse_encode": (_c_size, [_c_vp, ctypes.c_int, _c_size, _c_vp]),
        "orc_sparse_decode_acc": (ctypes.c_int, [_c_vp, _c_vp, ctypes.c_int]),
        "orc_sparse_decode": (ctypes.c_int, [_c_vp, _c_vp, ctypes.c_int]),
        "orc_ring_allreduce_compressed": (ctypes.c_int, [
            _c_vp, ctypes.c_int, _c_size, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
            ctypes.c_float, _c_size, _c_vp, _u64p, _u64p]),
        "orc_bucket_plan": (_c_size, [_c_vp, _c_size, ctypes.c_int, _c_size, _c_vp]),
        "orc_bucketed_allreduce": (ctypes.c_int, [_c_vp, _c_vp, _c_size, ctypes.c_int, ctypes.c_int,
                                                  _c_size, _u64p, _u64p]),
        "orc_fpenv_ok": (ctypes.c_int, []),
        "orc_convert": (ctypes.c_int, [_c_vp, ctypes.c_int, _c_vp, ctypes.c_int, _c_size]),
        "orc_ring_allreduce_compressed_state": (ctypes.c_int, [
            _c_vp, _c_vp, ctypes.c_int, _c_size, ctypes.c_int, ctypes.c_int, ctypes.c_int, _c_size, ctypes.c_int,
            _u64p, _u64p]),
        "orc_tree_reduce_round": (ctypes.c_int, [_c_vp, ctypes.c_int, _c_size, ctypes.c_int, ctypes.c_int]),
        "orc_tree_allreduce": (ctypes.c_int, [_c_vp, ctypes.c_int, _c_size, ctypes.c_int, _u64p, _u64p]),
        "orc_mix64": (ctypes.c_uint64, [ctypes.c_uint64]),
        "orc_hash64": (ctypes.c_uint64, [_c_vp, _c_size]),
        "orc_shared_state_sync": (ctypes.c_int, [_c_vp, ctypes.c_int, _c_size, _u64p, _u64p, _u64p]),
        "orc_ring_allreduce_ft": (ctypes.c_int, [_c_vp, ctypes.c_int, _c_size, ctypes.c_int, _c_vp, _c_vp, _c_vp,
                                                 ctypes.c_int, ctypes.c_int, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp,
                                                 _u64p, _u64p]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def lib():
    return _load()


# ---------------------------------------------------------------- helpers

def _dt_of(arr, dt=None):
    if dt is not None:
        return dt
    if arr.dtype == np.float32:
        return F32
    if arr.dtype == np.float16:
        return F16
    raise ValueError("pass dt=BF16 for uint16 bfloat16 bit patterns")


def _ptrs(arrays):
    for a in arrays:
        if not a.flags.c_contiguous:
            raise ValueError("oracle needs C-contiguous arrays")
    p = (ctypes.c_void_p * len(arrays))(*[a.ctypes.data for a in arrays])
    return p


def _traffic(n):
    return (ctypes.c_uint64 * n)(), (ctypes.c_uint64 * n)()


def _check(rc, what):
    if rc != 0:
        raise ValueError(f"oracle {what} rejected its arguments (status {rc})")


def es_of(dt):
    return 4 if dt == F32 else 2


# ---------------------------------------------------------------- scalars

def f16_to_f32(h):
    return lib().orc_f16_to_f32(int(h))


def f32_to_f16(x):
    return lib().orc_f32_to_f16(float(x))


def bf16_to_f32(h):
    return lib().orc_bf16_to_f32(int(h))


def f32_to_bf16(x):
    return lib().orc_f32_to_bf16(float(x))


def convert(x, sdt, ddt):
    """Array conversion: widen exactly, round to nearest even.  Returns
    float32, float16 or uint16 (bfloat16 bits) according to ddt."""
    x = np.ascontiguousarray(x)
    out = np.empty(x.size, dtype={F32: np.float32, F16: np.float16, BF16: np.uint16}[ddt])
    _check(lib().orc_convert(x.ctypes.data, sdt, out.ctypes.data, ddt, x.size), "convert")
    return out


def chunk_len(count, n, align=128):
    return lib().orc_chunk_len(count, n, align)


def comp_chunk_len(count, n, block):
    return lib().orc_comp_chunk_len(count, n, block)


def fpenv_ok():
    return bool(lib().orc_fpenv_ok())


# ---------------------------------------------------------------- collectives (in place)

def rs_step(bufs, s, dt=None):
    dt = _dt_of(bufs[0], dt)
    _check(lib().orc_rs_step(_ptrs(bufs), len(bufs), bufs[0].size, dt, s), "rs_step")


def ag_step(bufs, s, dt=None):
    dt = _dt_of(bufs[0], dt)
    _check(lib().orc_ag_step(_ptrs(bufs), len(bufs), bufs[0].size, dt, s), "ag_step")


def _collective(name, bufs, dt, *extra):
    dt = _dt_of(bufs[0], dt)
    n = len(bufs)
    sent, recv = _traffic(n)
    fn = getattr(lib(), name)
    _check(fn(_ptrs(bufs), n, bufs[0].size, dt, *extra, sent, recv), name)
    return list(sent), list(recv)


def ring_allreduce(bufs, dt=None):
    """In place; returns (sent_bytes, recv_bytes) per rank."""
    return _collective("orc_ring_allreduce", bufs, dt)


def tree_allreduce(bufs, dt=None):
    """Binomial-tree reduce into rank 0, then binomial broadcast; in place."""
    return _collective("orc_tree_allreduce", bufs, dt)


def tree_reduce_round(bufs, span, dt=None):
    dt = _dt_of(bufs[0], dt)
    _check(lib().orc_tree_reduce_round(_ptrs(bufs), len(bufs), bufs[0].size, dt, span), "tree_reduce_round")


def reduce_scatter(bufs, dt=None):
    return _collective("orc_reduce_scatter", bufs, dt)


def allgather(bufs, dt=None):
    return _collective("orc_allgather", bufs, dt)


def broadcast(bufs, root=0, dt=None):
    return _collective("orc_broadcast", bufs, dt, root)


def naive_sum_f64(bufs, dt=None):
    dt = _dt_of(bufs[0], dt)
    out = np.empty(bufs[0].size, dtype=np.float64)
    _check(lib().orc_naive_sum_f64(_ptrs(bufs), len(bufs), bufs[0].size, dt, out.ctypes.data), "naive_sum")
    return out


# ---------------------------------------------------------------- BFP

def bfp_bytes(count, block=128, mbits=8):
    return lib().orc_bfp_bytes(count, block, mbits)


def bfp_encode(x, block=128, mbits=8, dt=None, with_blockmax=False):
    dt = _dt_of(x, dt)
    n = x.size
    msg = np.zeros(bfp_bytes(n, block, mbits), dtype=np.uint8)
    bm = np.zeros((n + block - 1) // block, dtype=np.float64) if with_blockmax else None
    _check(lib().orc_bfp_encode(x.ctypes.data, dt, n, block, mbits, msg.ctypes.data,
                                bm.ctypes.data if bm is not None else None), "bfp_encode")
    return (msg, bm) if with_blockmax else msg


def bfp_decode_acc(msg, acc, block=128, mbits=8, dt=None):
    dt = _dt_of(acc, dt)
    _check(lib().orc_bfp_decode_acc(msg.ctypes.data, acc.size, block, mbits, acc.ctypes.data, dt),
           "bfp_decode_acc")


def bfp_decode(msg, count, block=128, mbits=8, out_dtype=np.float32, dt=None):
    out = np.zeros(count, dtype=out_dtype)
    dt = _dt_of(out, dt)
    _check(lib().orc_bfp_decode(msg.ctypes.data, count, block, mbits, out.ctypes.data, dt), "bfp_decode")
    return out


# ---------------------------------------------------------------- sparse

def sparse_bytes(nnz, dt):
    return lib().orc_sparse_bytes(nnz, dt)


def count_zeros(x, dt=None):
    dt = _dt_of(x, dt)
    return lib().orc_count_zeros(x.ctypes.data, dt, x.size)


def sparse_encode(x, dt=None):
    dt = _dt_of(x, dt)
    msg = np.zeros(sparse_bytes(x.size, dt), dtype=np.uint8)
    nbytes = lib().orc_sparse_encode(x.ctypes.data, dt, x.size, msg.ctypes.data)
    return msg[:nbytes].copy()


def sparse_decode_acc(msg, acc, dt=None):
    dt = _dt_of(acc, dt)
    _check(lib().orc_sparse_decode_acc(msg.ctypes.data, acc.ctypes.data, dt), "sparse_decode_acc")


def sparse_decode(msg, out):
    dt = _dt_of(out)
    _check(lib().orc_sparse_decode(msg.ctypes.data, out.ctypes.data, dt), "sparse_decode")


# ---------------------------------------------------------------- compressed ring

def ring_allreduce_compressed(bufs, method=COMP_BFP, block=128, mbits=8, theta=0.5,
                              unit=2097152, dt=None, with_blockmax=False):
    """In place; returns (sent, recv[, blockmax per block]).

    theta is the sparsity threshold of SPARSE_AUTO.  It is rounded to binary32
    (the type of a compression configuration's threshold field) and the
    decision is zeros > theta * len, that product taken in binary64."""
    dt = _dt_of(bufs[0], dt)
    n = len(bufs)
    count = bufs[0].size
    sent, recv = _traffic(n)
    bm = np.zeros((count + block - 1) // block, dtype=np.float64) if with_blockmax else None
    _check(lib().orc_ring_allreduce_compressed(
        _ptrs(bufs), n, count, dt, method, block, mbits, float(np.float32(theta)), unit,
        bm.ctypes.data if bm is not None else None, sent, recv), "ring_allreduce_compressed")
    if with_blockmax:
        return list(sent), list(recv), bm
    return list(sent), list(recv)


FB_ERROR, FB_DELTA = 1, 2


def ring_allreduce_compressed_state(bufs, state, feedback, block=128, mbits=8, unit=2097152, dt=None):
    """BFP ring with per-rank binary32 state (error feedback or delta
    encoding); bufs and state (float32 arrays, one per rank) in place."""
    dt = _dt_of(bufs[0], dt)
    n = len(bufs)
    for st in state:
        if st.dtype != np.float32 or st.size != bufs[0].size:
            raise ValueError("state must be float32 arrays of the buffer length")
    sent, recv = _traffic(n)
    _check(lib().orc_ring_allreduce_compressed_state(_ptrs(bufs), _ptrs(state), n, bufs[0].size, dt, block, mbits,
                                                     unit, feedback, sent, recv), "compressed_state")
    return list(sent), list(recv)


# ---------------------------------------------------------------- bucketing

def bucket_plan(counts, dt, cap_bytes):
    c = np.ascontiguousarray(np.asarray(counts, dtype=np.uint64))
    out = np.zeros(len(counts), dtype=np.int32)
    nb = lib().orc_bucket_plan(c.ctypes.data, len(counts), dt, cap_bytes, out.ctypes.data)
    return int(nb), out


def bucketed_allreduce(tensors, cap_bytes, dt=None):
    """tensors[r][t] = rank r's tensor t (numpy arrays, modified in place)."""
    n = len(tensors)
    nt = len(tensors[0])
    dt = _dt_of(tensors[0][0], dt)
    flat = [tensors[r][t] for r in range(n) for t in range(nt)]
    counts = np.ascontiguousarray(np.array([a.size for a in tensors[0]], dtype=np.uint64))
    sent, recv = _traffic(n)
    _check(lib().orc_bucketed_allreduce(_ptrs(flat), counts.ctypes.data, nt, n, dt, cap_bytes, sent, recv),
           "bucketed_allreduce")
    return list(sent), list(recv)


# ---------------------------------------------------------------- shared state and faults

EABORT = 2


def mix64(z):
    return int(lib().orc_mix64(z & 0xFFFFFFFFFFFFFFFF))


def hash64(a):
    a = np.ascontiguousarray(a)
    return int(lib().orc_hash64(a.ctypes.data, a.nbytes))


def shared_state_sync(bufs):
    """Majority-hash check over the rank buffers (numpy, same byte size);
    diverged ranks receive the majority buffer in place.  Returns
    (resent, hashes, sent, recv)."""
    n = len(bufs)
    nbytes = bufs[0].nbytes
    if any(b.nbytes != nbytes for b in bufs):
        raise ValueError("rank buffers must have one byte size")
    hashes = (ctypes.c_uint64 * n)()
    sent, recv = _traffic(n)
    resent = lib().orc_shared_state_sync(_ptrs(bufs), n, nbytes, hashes, sent, recv)
    if resent < 0:
        raise ValueError("oracle shared_state_sync rejected its arguments")
    return resent, list(hashes), list(sent), list(recv)


def ring_allreduce_ft(bufs, faults=(), deadline_ms=0, dt=None):
    """Ring allreduce with injected faults [(rank, step) or (rank, step,
    stall_ms), ...] and a receive deadline (see orc_ring_allreduce_ft).
    Returns a dict with status, attempts, dead_attempt, dead_step,
    dead_reason, waited_ms, survivors, sent, recv."""
    dt = _dt_of(bufs[0], dt)
    n = len(bufs)
    fs_ = [tuple(f) + (0,) * (3 - len(f)) for f in faults]
    fr = np.ascontiguousarray(np.array([f[0] for f in fs_] or [0], dtype=np.int32))
    fs = np.ascontiguousarray(np.array([f[1] for f in fs_] or [1], dtype=np.int32))
    fw = np.ascontiguousarray(np.array([f[2] for f in fs_] or [0], dtype=np.int32))
    da = np.zeros(n, dtype=np.int32)
    ds = np.zeros(n, dtype=np.int32)
    dr = np.zeros(n, dtype=np.int32)
    att = np.zeros(1, dtype=np.int32)
    waited = np.zeros(1, dtype=np.int64)
    sent, recv = _traffic(n)
    rc = lib().orc_ring_allreduce_ft(_ptrs(bufs), n, bufs[0].size, dt, fr.ctypes.data, fs.ctypes.data, fw.ctypes.data,
                                     len(fs_), deadline_ms, att.ctypes.data, da.ctypes.data, ds.ctypes.data,
                                     dr.ctypes.data, waited.ctypes.data, sent, recv)
    if rc not in (0, EABORT):
        raise ValueError(f"oracle ring_allreduce_ft rejected its arguments (status {rc})")
    return {"status": rc, "attempts": int(att[0]), "dead_attempt": da.tolist(), "dead_step": ds.tolist(),
            "dead_reason": dr.tolist(), "waited_ms": int(waited[0]),
            "survivors": [r for r in range(n) if da[r] == 0], "sent": list(sent), "recv": list(recv)}
