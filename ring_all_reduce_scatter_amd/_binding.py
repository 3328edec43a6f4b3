"""ctypes binding of librar.so (the C-ABI declared in include/rar.h).

Argument marshalling only: torch tensors supply device pointers and HIP
streams, and every step of every collective runs in the library's kernels.
Python names are the C names without the ``rar_`` prefix.  If the library is
not built, every call raises RuntimeError: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from typing import Sequence

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "librar.so")

F32, F16, BF16 = 0, 1, 2
ALGO_FUSED, ALGO_STEPWISE = 0, 1
COMP_NONE, COMP_BFP, COMP_SPARSE_AUTO = 0, 1, 2
OP_ALLREDUCE, OP_ALLGATHER, OP_BROADCAST = 1, 2, 4
SCHED_FUSED, SCHED_STAGED, SCHED_FORWARD, SCHED_PIPELINED = 0, 1, 2, 3
FEEDBACK_ERROR, FEEDBACK_DELTA = 1, 2
MAX_RANKS = 64
HASH_WORKSPACE_BYTES = 512
EABORT = 8

_c_vp = ctypes.c_void_p
_c_size = ctypes.c_size_t
_c_int = ctypes.c_int
_u64p = ctypes.POINTER(ctypes.c_uint64)


class Fault(ctypes.Structure):
    """Mirror of rar_fault: before `step` of a pass `rank` is gone
    (stall_ms = 0) or stops answering for stall_ms."""
    _fields_ = [("rank", ctypes.c_int), ("step", ctypes.c_int), ("stall_ms", ctypes.c_int)]


class FtReport(ctypes.Structure):
    """Mirror of rar_ft_report."""
    _fields_ = [("attempts", ctypes.c_int), ("nsurvivors", ctypes.c_int),
                ("survivors", ctypes.c_int * 64), ("dead_attempt", ctypes.c_int * 64),
                ("dead_step", ctypes.c_int * 64), ("dead_reason", ctypes.c_int * 64),
                ("waited_ms", ctypes.c_longlong), ("hash", ctypes.c_uint64 * 64)]


class BucketedPlan(ctypes.Structure):
    """rar_bucketed_plan: a prepared FUSED bucketed allreduce."""
    _fields_ = [("workspace", ctypes.c_void_p), ("desc_offset", ctypes.c_uint64), ("grid", ctypes.c_uint64),
                ("ntensors", ctypes.c_uint64), ("nranks", ctypes.c_int), ("dtype", ctypes.c_int),
                ("sent", ctypes.c_uint64 * 64), ("recv", ctypes.c_uint64 * 64)]


class CompressCfg(ctypes.Structure):
    """Mirror of rar_compress_cfg."""
    _fields_ = [
        ("method", ctypes.c_int),
        ("block", ctypes.c_int),
        ("mbits", ctypes.c_int),
        ("sparsity_threshold", ctypes.c_float),
        ("unit_bytes", ctypes.c_size_t),
        ("collective_mask", ctypes.c_uint),
        ("schedule", ctypes.c_int),
    ]


class RarError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_string(status)} (status {status})")


_SIGS = {
    "rar_chunk_len": (_c_size, [_c_size, _c_int]),
    "rar_ring_allreduce": (_c_int, [_c_vp, _c_int, _c_size, _c_int, _c_vp]),
    "rar_ring_allreduce_ex": (_c_int, [_c_vp, _c_int, _c_size, _c_int, _c_int, _c_vp]),
    "rar_reduce_scatter": (_c_int, [_c_vp, _c_int, _c_size, _c_int, _c_vp]),
    "rar_reduce_scatter_ex": (_c_int, [_c_vp, _c_int, _c_size, _c_int, _c_int, _c_vp]),
    "rar_allgather": (_c_int, [_c_vp, _c_int, _c_size, _c_int, _c_vp]),
    "rar_allgather_ex": (_c_int, [_c_vp, _c_int, _c_size, _c_int, _c_int, _c_vp]),
    "rar_broadcast": (_c_int, [_c_vp, _c_int, _c_size, _c_int, _c_int, _c_vp]),
    "rar_broadcast_ex": (_c_int, [_c_vp, _c_int, _c_size, _c_int, _c_int, _c_int, _c_vp]),
    "rar_rs_step": (_c_int, [_c_vp, _c_int, _c_size, _c_int, _c_int, _c_vp]),
    "rar_ag_step": (_c_int, [_c_vp, _c_int, _c_size, _c_int, _c_int, _c_vp]),
    "rar_last_traffic": (_c_int, [_u64p, _u64p, _c_int]),
    "rar_tree_allreduce": (_c_int, [_c_vp, _c_int, _c_size, _c_int, _c_vp]),
    "rar_tree_allreduce_ex": (_c_int, [_c_vp, _c_int, _c_size, _c_int, _c_int, _c_vp]),
    "rar_allreduce_auto": (_c_int, [_c_vp, _c_int, _c_size, _c_int, _c_size, ctypes.POINTER(ctypes.c_int),
                                    _c_vp]),
    "rar_bfp_bytes": (_c_size, [_c_size, _c_int, _c_int]),
    "rar_bfp_compress": (_c_int, [_c_vp, _c_int, _c_size, _c_int, _c_int, _c_vp, _c_vp]),
    "rar_bfp_decompress_accumulate": (_c_int, [_c_vp, _c_size, _c_int, _c_int, _c_vp, _c_int, _c_vp]),
    "rar_bfp_decompress": (_c_int, [_c_vp, _c_size, _c_int, _c_int, _c_vp, _c_int, _c_vp]),
    "rar_compress_cfg_default": (None, [ctypes.POINTER(CompressCfg)]),
    "rar_compressed_chunk_len": (_c_size, [_c_size, _c_int, _c_int]),
    "rar_compressed_workspace_bytes": (_c_size, [_c_int, _c_size, _c_int, ctypes.POINTER(CompressCfg)]),
    "rar_ring_allreduce_compressed": (_c_int, [_c_vp, _c_int, _c_size, _c_int, ctypes.POINTER(CompressCfg),
                                               _c_vp, _c_size, _c_vp]),
    "rar_ring_allreduce_compressed_noalloc": (_c_int, [_c_vp, _c_int, _c_size, _c_int,
                                                       ctypes.POINTER(CompressCfg), _c_vp]),
    "rar_ring_allreduce_compressed_state": (_c_int, [_c_vp, _c_vp, _c_int, _c_size, _c_int, _c_int,
                                                     ctypes.POINTER(CompressCfg), _c_vp, _c_size, _c_vp]),
    "rar_compressed_traffic": (_c_int, [_c_vp, _c_int, _u64p, _u64p, _c_vp]),
    "rar_rank_hashes": (_c_int, [_c_vp, _c_int, _c_size, _c_vp, _c_size, _u64p, _c_vp]),
    "rar_shared_state_sync": (_c_int, [_c_vp, _c_int, _c_size, _c_vp, _c_size, ctypes.POINTER(ctypes.c_int),
                                       _u64p, _c_vp]),
    "rar_ft_workspace_bytes": (_c_size, [_c_int, _c_size, _c_int]),
    "rar_ring_allreduce_ft": (_c_int, [_c_vp, _c_int, _c_size, _c_int, ctypes.POINTER(Fault), _c_int, _c_int,
                                       _c_vp, _c_size, ctypes.POINTER(FtReport), _c_vp]),
    "rar_bucket_plan": (_c_size, [_c_vp, _c_size, _c_int, _c_size, _c_vp]),
    "rar_bucketed_workspace_bytes": (_c_size, [_c_vp, _c_size, _c_int, _c_int, _c_size]),
    "rar_bucketed_allreduce": (_c_int, [_c_vp, _c_vp, _c_size, _c_int, _c_int, _c_size, _c_vp, _c_size,
                                        _c_vp]),
    "rar_bucketed_workspace_bytes_ex": (_c_size, [_c_vp, _c_size, _c_int, _c_int, _c_size, _c_int]),
    "rar_bucketed_allreduce_ex": (_c_int, [_c_vp, _c_vp, _c_size, _c_int, _c_int, _c_size, _c_int, _c_vp,
                                           _c_size, _c_vp]),
    "rar_bucketed_prepare": (_c_int, [_c_vp, _c_vp, _c_size, _c_int, _c_int, _c_size, _c_vp, _c_size,
                                      ctypes.POINTER(BucketedPlan), _c_vp]),
    "rar_bucketed_launch": (_c_int, [ctypes.POINTER(BucketedPlan), _c_vp]),
    "rar_status_string": (ctypes.c_char_p, [_c_int]),
    "rar_version": (ctypes.c_char_p, []),
}

_lib = None


def lib():
    """The loaded library; raises RuntimeError when it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build the HIP library first "
                "(python -m ring_all_reduce_scatter_amd.build)")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def status_string(status: int) -> str:
    return lib().rar_status_string(int(status)).decode()


def version() -> str:
    return lib().rar_version().decode()


def _check(rc: int, what: str) -> None:
    if rc != 0:
        raise RarError(rc, what)


# ------------------------------------------------------------------ marshalling

def dtype_code(t) -> int:
    import torch
    m = {torch.float32: F32, torch.float16: F16, torch.bfloat16: BF16}
    if t.dtype not in m:
        raise TypeError(f"unsupported dtype {t.dtype}")
    return m[t.dtype]


def _stream(stream, t):
    if stream is not None:
        return ctypes.c_void_p(int(stream) if isinstance(stream, int) else stream.cuda_stream)
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _dptr(t) -> int:
    """Device address of a tensor; host tensors are refused here, since the
    kernels would read host addresses as device memory."""
    if t.device.type != "cuda":
        raise ValueError(f"expected a GPU tensor, got one on {t.device}")
    return t.data_ptr()


def _flat(t, what: str):
    """A tensor whose storage the kernels may read as `numel` contiguous
    elements: strided or expanded views are refused (the kernels would walk
    past the view into other memory)."""
    if not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous")
    return t


def _need_bytes(t, nbytes: int, what: str):
    have = t.numel() * t.element_size()
    if have < nbytes:
        raise ValueError(f"{what} holds {have} bytes, {nbytes} are needed")


def _rank_ptrs(bufs: Sequence):
    if len(bufs) < 1:
        raise ValueError("need at least one rank buffer")
    t0 = bufs[0]
    for b in bufs:
        if b.dtype != t0.dtype or b.numel() != t0.numel() or b.device != t0.device:
            raise ValueError("rank buffers must share dtype, size and device")
        if not b.is_contiguous():
            raise ValueError("rank buffers must be contiguous")
    return (ctypes.c_void_p * len(bufs))(*[_dptr(b) for b in bufs])


def _call_bufs(name: str, bufs, *extra, stream=None):
    rc = getattr(lib(), name)(_rank_ptrs(bufs), len(bufs), bufs[0].numel(), dtype_code(bufs[0]), *extra,
                              _stream(stream, bufs[0]))
    _check(rc, name)


# ------------------------------------------------------------------ uncompressed collectives

def chunk_len(count: int, nranks: int) -> int:
    return lib().rar_chunk_len(count, nranks)


def ring_allreduce(bufs, stream=None):
    _call_bufs("rar_ring_allreduce", bufs, stream=stream)


def ring_allreduce_ex(bufs, algo: int, stream=None):
    _call_bufs("rar_ring_allreduce_ex", bufs, algo, stream=stream)


def reduce_scatter(bufs, stream=None):
    _call_bufs("rar_reduce_scatter", bufs, stream=stream)


def reduce_scatter_ex(bufs, algo: int, stream=None):
    _call_bufs("rar_reduce_scatter_ex", bufs, algo, stream=stream)


def allgather(bufs, stream=None):
    _call_bufs("rar_allgather", bufs, stream=stream)


def allgather_ex(bufs, algo: int, stream=None):
    _call_bufs("rar_allgather_ex", bufs, algo, stream=stream)


def broadcast(bufs, root: int = 0, stream=None):
    _call_bufs("rar_broadcast", bufs, root, stream=stream)


def broadcast_ex(bufs, root: int, algo: int, stream=None):
    _call_bufs("rar_broadcast_ex", bufs, root, algo, stream=stream)


def rs_step(bufs, step: int, stream=None):
    _call_bufs("rar_rs_step", bufs, step, stream=stream)


def ag_step(bufs, step: int, stream=None):
    _call_bufs("rar_ag_step", bufs, step, stream=stream)


ALLREDUCE_RING, ALLREDUCE_TREE = 0, 1
TREE_THRESHOLD_DEFAULT = 1 << 20


def tree_allreduce(bufs, stream=None):
    _call_bufs("rar_tree_allreduce", bufs, stream=stream)


def tree_allreduce_ex(bufs, algo: int, stream=None):
    _call_bufs("rar_tree_allreduce_ex", bufs, algo, stream=stream)


def allreduce_auto(bufs, threshold_bytes: int = 0, stream=None) -> int:
    """Tree below the threshold (bytes per rank), ring above; returns the choice."""
    chosen = ctypes.c_int(-1)
    _call_bufs("rar_allreduce_auto", bufs, threshold_bytes, ctypes.byref(chosen), stream=stream)
    return chosen.value


def last_traffic(nranks: int):
    sent = (ctypes.c_uint64 * nranks)()
    recv = (ctypes.c_uint64 * nranks)()
    _check(lib().rar_last_traffic(sent, recv, nranks), "rar_last_traffic")
    return list(sent), list(recv)


# ------------------------------------------------------------------ BFP

def bfp_bytes(count: int, block: int = 128, mbits: int = 8) -> int:
    return lib().rar_bfp_bytes(count, block, mbits)


def _bfp_msg_check(msg, count: int, block: int, mbits: int, dst, what: str):
    """count elements fit dst, and msg holds a whole message for them."""
    _flat(msg, f"{what}: message")
    _flat(dst, f"{what}: destination")
    if count < 0 or count > dst.numel():
        raise ValueError(f"{what}: count {count} is outside the destination's {dst.numel()} elements")
    need = bfp_bytes(count, block, mbits)
    if need:  # 0 = invalid block or mbits: the library reports it
        _need_bytes(msg, need, f"{what}: message")


def bfp_compress(src, block: int, mbits: int, dst, stream=None):
    """Encode all of src into dst, which must hold bfp_bytes(src.numel()) bytes."""
    _flat(src, "bfp_compress: source")
    _flat(dst, "bfp_compress: message")
    need = bfp_bytes(src.numel(), block, mbits)
    if need:
        _need_bytes(dst, need, "bfp_compress: message")
    rc = lib().rar_bfp_compress(_dptr(src), dtype_code(src), src.numel(), block, mbits, _dptr(dst),
                                _stream(stream, src))
    _check(rc, "rar_bfp_compress")


def bfp_decompress_accumulate(msg, count: int, block: int, mbits: int, acc, stream=None):
    _bfp_msg_check(msg, count, block, mbits, acc, "bfp_decompress_accumulate")
    rc = lib().rar_bfp_decompress_accumulate(_dptr(msg), count, block, mbits, _dptr(acc),
                                             dtype_code(acc), _stream(stream, acc))
    _check(rc, "rar_bfp_decompress_accumulate")


def bfp_decompress(msg, count: int, block: int, mbits: int, dst, stream=None):
    _bfp_msg_check(msg, count, block, mbits, dst, "bfp_decompress")
    rc = lib().rar_bfp_decompress(_dptr(msg), count, block, mbits, _dptr(dst), dtype_code(dst),
                                  _stream(stream, dst))
    _check(rc, "rar_bfp_decompress")


# ------------------------------------------------------------------ compressed allreduce

def compress_cfg_default() -> CompressCfg:
    cfg = CompressCfg()
    lib().rar_compress_cfg_default(ctypes.byref(cfg))
    return cfg


def compress_cfg(**kw) -> CompressCfg:
    """The library's default configuration with the given fields replaced.
    Unknown field names raise (a ctypes structure would otherwise keep them
    as plain Python attributes that the library never sees)."""
    cfg = compress_cfg_default()
    names = {f[0] for f in CompressCfg._fields_}
    for k, v in kw.items():
        if k not in names:
            raise TypeError(f"compress_cfg: unknown field {k!r} (fields: {', '.join(sorted(names))})")
        setattr(cfg, k, v)
    return cfg


def compressed_chunk_len(count: int, nranks: int, block: int = 128) -> int:
    return lib().rar_compressed_chunk_len(count, nranks, block)


def compressed_workspace_bytes(nranks: int, count: int, dtype: int, cfg: CompressCfg) -> int:
    return lib().rar_compressed_workspace_bytes(nranks, count, dtype, ctypes.byref(cfg))


def ring_allreduce_compressed(bufs, cfg: CompressCfg, workspace, stream=None):
    if workspace is not None:
        _flat(workspace, "workspace")
    rc = lib().rar_ring_allreduce_compressed(
        _rank_ptrs(bufs), len(bufs), bufs[0].numel(), dtype_code(bufs[0]), ctypes.byref(cfg),
        _dptr(workspace) if workspace is not None else None,
        workspace.numel() * workspace.element_size() if workspace is not None else 0,
        _stream(stream, bufs[0]))
    _check(rc, "rar_ring_allreduce_compressed")


NOALLOC_SCRATCH_BYTES = 32 << 20


def ring_allreduce_compressed_noalloc(bufs, cfg: CompressCfg, stream=None):
    """ring_allreduce_compressed without a workspace: the library's own
    scratch array holds the messages (RAR_EWORKSPACE beyond its size)."""
    rc = lib().rar_ring_allreduce_compressed_noalloc(_rank_ptrs(bufs), len(bufs), bufs[0].numel(),
                                                     dtype_code(bufs[0]), ctypes.byref(cfg), _stream(stream, bufs[0]))
    _check(rc, "rar_ring_allreduce_compressed_noalloc")


def ring_allreduce_compressed_state(bufs, state, feedback: int, cfg: CompressCfg, workspace, stream=None):
    """state: one float32 tensor of bufs[0].numel() elements per rank, zero
    before the first call and kept between calls."""
    if len(state) != len(bufs):
        raise ValueError("need one state tensor per rank")
    for s_ in state:
        if s_.numel() != bufs[0].numel() or s_.element_size() != 4 or not s_.is_contiguous():
            raise ValueError("state tensors must be contiguous float32 of the rank buffers' length")
    if workspace is not None:
        _flat(workspace, "workspace")
    rc = lib().rar_ring_allreduce_compressed_state(
        _rank_ptrs(bufs), (ctypes.c_void_p * len(state))(*[_dptr(t) for t in state]), len(bufs),
        bufs[0].numel(), dtype_code(bufs[0]), feedback, ctypes.byref(cfg),
        _dptr(workspace) if workspace is not None else None,
        workspace.numel() * workspace.element_size() if workspace is not None else 0,
        _stream(stream, bufs[0]))
    _check(rc, "rar_ring_allreduce_compressed_state")


TRAFFIC_BYTES = 2 * MAX_RANKS * 8  # the byte counters at the start of a compressed call's workspace


def compressed_traffic(workspace, nranks: int, stream=None):
    _flat(workspace, "workspace")
    _need_bytes(workspace, TRAFFIC_BYTES, "compressed_traffic: workspace")
    sent = (ctypes.c_uint64 * nranks)()
    recv = (ctypes.c_uint64 * nranks)()
    _check(lib().rar_compressed_traffic(_dptr(workspace), nranks, sent, recv, _stream(stream, workspace)),
           "rar_compressed_traffic")
    return list(sent), list(recv)


# ------------------------------------------------------------------ shared state, faults

def _nbytes(t):
    return t.numel() * t.element_size()


def _ws(workspace):
    if workspace is None:
        return (None, 0)
    _flat(workspace, "workspace")
    return (_dptr(workspace), _nbytes(workspace))


def rank_hashes(bufs, workspace, nbytes=None, stream=None):
    """64-bit hash of each rank buffer's first nbytes bytes (default: all)."""
    nb = _nbytes(bufs[0]) if nbytes is None else int(nbytes)
    for b in bufs:
        _flat(b, "rank_hashes: buffer")
        if nb < 0 or nb > _nbytes(b):
            raise ValueError(f"rank_hashes: nbytes {nb} is outside a buffer of {_nbytes(b)} bytes")
    out = (ctypes.c_uint64 * len(bufs))()
    ptrs = (ctypes.c_void_p * len(bufs))(*[_dptr(b) for b in bufs])
    _check(lib().rar_rank_hashes(ptrs, len(bufs), nb, *_ws(workspace), out, _stream(stream, bufs[0])),
           "rar_rank_hashes")
    return list(out)


def shared_state_sync(bufs, workspace, stream=None):
    """Majority-hash check; diverged ranks receive the majority buffer.
    Returns (resent, hashes before the re-send)."""
    resent = ctypes.c_int(0)
    out = (ctypes.c_uint64 * len(bufs))()
    _check(lib().rar_shared_state_sync(_rank_ptrs(bufs), len(bufs), _nbytes(bufs[0]), *_ws(workspace),
                                       ctypes.byref(resent), out, _stream(stream, bufs[0])),
           "rar_shared_state_sync")
    return resent.value, list(out)


def ft_workspace_bytes(nranks: int, count: int, dtype: int) -> int:
    return lib().rar_ft_workspace_bytes(nranks, count, dtype)


def ring_allreduce_ft(bufs, faults, workspace, deadline_ms: int = 0, stream=None):
    """Ring allreduce with injected faults [(rank, step) or (rank, step,
    stall_ms), ...] and a receive deadline.  Returns a dict: status (0 or
    EABORT), attempts, survivors, dead_attempt, dead_step, dead_reason,
    waited_ms, hash (per rank)."""
    n = len(bufs)
    fl = [tuple(f) + (0,) * (3 - len(f)) for f in faults]
    arr = (Fault * max(1, len(fl)))(*[Fault(int(r), int(s), int(w)) for r, s, w in fl])
    rep = FtReport()
    rc = lib().rar_ring_allreduce_ft(_rank_ptrs(bufs), n, bufs[0].numel(), dtype_code(bufs[0]), arr, len(fl),
                                     deadline_ms, *_ws(workspace), ctypes.byref(rep), _stream(stream, bufs[0]))
    if rc not in (0, EABORT):
        _check(rc, "rar_ring_allreduce_ft")
    return {"status": rc, "attempts": rep.attempts, "survivors": list(rep.survivors)[:rep.nsurvivors],
            "dead_attempt": list(rep.dead_attempt)[:n], "dead_step": list(rep.dead_step)[:n],
            "dead_reason": list(rep.dead_reason)[:n], "waited_ms": rep.waited_ms, "hash": list(rep.hash)[:n]}


# ------------------------------------------------------------------ bucketing

def _sizes(counts):
    return (ctypes.c_size_t * len(counts))(*[int(c) for c in counts])


def bucket_plan(counts, dtype: int, cap_bytes: int):
    out = (ctypes.c_int * max(1, len(counts)))()
    nb = lib().rar_bucket_plan(_sizes(counts), len(counts), dtype, cap_bytes, out)
    return int(nb), list(out)[:len(counts)]


def bucketed_workspace_bytes(counts, nranks: int, dtype: int, cap_bytes: int, algo: int = ALGO_FUSED) -> int:
    return lib().rar_bucketed_workspace_bytes_ex(_sizes(counts), len(counts), nranks, dtype, cap_bytes, algo)


class BucketedAllreduce:
    """A bucketed allreduce over fixed gradient tensors, prepared once.

    tensors[r][t] is rank r's tensor t (device tensors, updated in place on
    every call).  A training loop reduces the same gradient tensors every
    step, so the pointers are collected and checked here once; with the
    FUSED algorithm the library also writes the launch table and the fold
    descriptors into the workspace here (rar_bucketed_prepare, on `stream`,
    synchronised before returning) and each call launches the fold alone
    (rar_bucketed_launch).  The tensors and the workspace must stay alive and
    keep their storage, and nothing else may write the workspace, while this
    object is used."""

    def __init__(self, tensors, cap_bytes: int, workspace, algo: int = ALGO_FUSED, stream=None):
        n, nt = len(tensors), len(tensors[0])
        t0 = tensors[0][0]
        counts = [x.numel() for x in tensors[0]]
        flat = [x for row in tensors for x in row]
        if any(len(row) != nt for row in tensors) or any([x.numel() for x in row] != counts for row in tensors):
            raise ValueError("tensor t must have the same size on every rank")
        if any(x.dtype != t0.dtype for x in flat) or not all(x.is_contiguous() for x in flat):
            raise ValueError("tensors must share one dtype and be contiguous")
        self._keep = (tensors, workspace)
        self._ptrs = (ctypes.c_void_p * len(flat))(*[_dptr(x) for x in flat])
        self._counts = _sizes(counts)
        self._args = (nt, n, dtype_code(t0), cap_bytes, algo,
                      _dptr(workspace) if workspace is not None else None,
                      workspace.numel() * workspace.element_size() if workspace is not None else 0)
        self._t0 = t0
        self._plan = None
        if algo == ALGO_FUSED:
            plan = BucketedPlan()
            st = _stream(stream, t0)
            rc = lib().rar_bucketed_prepare(self._ptrs, self._counts, nt, n, dtype_code(t0), cap_bytes,
                                            self._args[5], self._args[6], ctypes.byref(plan), st)
            _check(rc, "rar_bucketed_prepare")
            import torch
            torch.cuda.synchronize(t0.device)  # later calls may come on any stream
            self._plan = plan

    def __call__(self, stream=None):
        if self._plan is not None:
            _check(lib().rar_bucketed_launch(ctypes.byref(self._plan), _stream(stream, self._t0)),
                   "rar_bucketed_launch")
            return
        rc = lib().rar_bucketed_allreduce_ex(self._ptrs, self._counts, *self._args, _stream(stream, self._t0))
        _check(rc, "rar_bucketed_allreduce_ex")


def rank_tensors(nranks: int, counts, dtype, device="cuda", align_elems: int = 256):
    """N simulated ranks' copies of a list of tensors, placed for the folds.

    Returns (arena, views) with views[r][t] rank r's tensor t.  Every rank's
    tensors lie in one region of the arena, tensor t at the same offset in
    each region (a multiple of align_elems), and the regions are a power of
    two bytes apart.  The fused folds read all N copies of an element at
    once; on MI355X copies a power of two apart spread evenly over the HBM
    channels, while copies at arbitrary distances collide (measured on a
    16-rank bf16 fold: 5.5 TB/s against 4.2-4.6 TB/s).  On real GPUs each
    rank's tensor sits in its own HBM, so this placement only removes an
    artefact of simulating the ranks on one device."""
    import torch
    offs, off = [], 0
    for c in counts:
        offs.append(off)
        off += -(-int(c) // align_elems) * align_elems
    es = torch.empty((), dtype=dtype).element_size()
    region = max(off * es, 1)
    stride_bytes = 1 << (region - 1).bit_length()
    stride = stride_bytes // es
    arena = torch.empty(nranks * stride, dtype=dtype, device=device)
    views = [[arena[r * stride + o: r * stride + o + int(c)] for o, c in zip(offs, counts)] for r in range(nranks)]
    return arena, views


def bucketed_allreduce(tensors, cap_bytes: int, workspace, stream=None, algo: int = ALGO_FUSED):
    """tensors[r][t]: rank r's gradient tensor t (device tensors, in place);
    one call of rar_bucketed_allreduce_ex (table, descriptors and fold)."""
    n, nt = len(tensors), len(tensors[0])
    t0 = tensors[0][0]
    counts = [x.numel() for x in tensors[0]]
    flat = [x for row in tensors for x in row]
    if any(len(row) != nt for row in tensors) or any([x.numel() for x in row] != counts for row in tensors):
        raise ValueError("tensor t must have the same size on every rank")
    if any(x.dtype != t0.dtype for x in flat) or not all(x.is_contiguous() for x in flat):
        raise ValueError("tensors must share one dtype and be contiguous")
    ptrs = (ctypes.c_void_p * len(flat))(*[_dptr(x) for x in flat])
    rc = lib().rar_bucketed_allreduce_ex(ptrs, _sizes(counts), nt, n, dtype_code(t0), cap_bytes, algo,
                                         _dptr(workspace) if workspace is not None else None,
                                         workspace.numel() * workspace.element_size() if workspace is not None
                                         else 0, _stream(stream, t0))
    _check(rc, "rar_bucketed_allreduce_ex")
