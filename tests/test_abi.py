"""The C-ABI library loads and exports every symbol include/rar.h declares;
host-only entry points (sizes, plans, argument checks) behave.  CPU only: no
call here reaches a kernel launch."""
import ctypes
import os
import re

import numpy as np
import pytest

import ring_all_reduce_scatter_amd as rar
from ring_all_reduce_scatter_amd import inputs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    text = open(os.path.join(ROOT, "include", "rar.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(rar_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = rar.lib()
    names = declared_functions()
    assert len(names) >= 20
    for name in names:
        assert hasattr(lib, name), name
        assert name in rar._binding._SIGS, f"binding lacks {name}"


def test_version_and_status_strings():
    assert "gfx950" in rar.version()
    assert rar.status_string(0) == "ok"
    assert "workspace" in rar.status_string(4)
    assert rar.status_string(99) == "unknown status"


@pytest.mark.parametrize("count,n", [(0, 1), (1, 4), (1 << 20, 4), (64 << 20, 8), (1000, 3), (12345, 16)])
def test_chunk_len_matches_oracle(orc, count, n):
    assert rar.chunk_len(count, n) == orc.chunk_len(count, n)
    assert rar.chunk_len(count, n) % 128 == 0
    assert rar.compressed_chunk_len(count, n, 512) == orc.comp_chunk_len(count, n, 512)


@pytest.mark.parametrize("count", [0, 1, 127, 128, 2097152, 1000003])
@pytest.mark.parametrize("block,mbits", [(128, 8), (128, 4), (16, 2), (512, 5)])
def test_bfp_bytes_matches_oracle(orc, count, block, mbits):
    assert rar.bfp_bytes(count, block, mbits) == orc.bfp_bytes(count, block, mbits)


def test_bfp_bytes_rejects_bad_args():
    assert rar.bfp_bytes(100, 100, 8) == 0
    assert rar.bfp_bytes(100, 128, 9) == 0
    assert rar.bfp_bytes(100, 8, 8) == 0


def test_compress_cfg_default_is_the_pages_starting_point():
    cfg = rar.compress_cfg_default()
    assert cfg.method == rar.COMP_BFP and cfg.block == 128 and cfg.mbits == 8
    assert cfg.sparsity_threshold == 0.5 and cfg.unit_bytes == 4 << 20
    assert cfg.collective_mask == rar.OP_ALLREDUCE and cfg.schedule == rar.SCHED_FUSED


def test_compressed_workspace_sizes():
    cfg = rar.compress_cfg_default()
    assert rar.compressed_workspace_bytes(8, 128 << 20, rar.F16, cfg) == 1024
    cfg.schedule = rar.SCHED_STAGED
    ws = rar.compressed_workspace_bytes(8, 128 << 20, rar.F16, cfg)
    slot = (16384 + 2097152 + 255) // 256 * 256
    assert ws == 1024 + 8 * 8 * slot
    cfg.schedule = rar.SCHED_FORWARD  # two slots per (rank, unit)
    assert rar.compressed_workspace_bytes(8, 128 << 20, rar.F16, cfg) == 1024 + 2 * 8 * 8 * slot
    cfg.schedule = rar.SCHED_STAGED
    cfg.unit_bytes = 1000  # not a multiple of the block
    assert rar.compressed_workspace_bytes(8, 1 << 20, rar.F16, cfg) == 0


def test_bucket_plan_matches_oracle(orc):
    sizes = inputs.bucket_sizes(200)
    for cap in (25 << 20, 1 << 20, 4 << 20):
        nb, plan = rar.bucket_plan(sizes, rar.BF16, cap)
        onb, oplan = orc.bucket_plan(sizes, orc.BF16, cap)
        assert nb == onb and plan == list(oplan)
    assert rar.bucket_plan([10, 20, 5, 100, 3, 3], rar.BF16, 60) == (4, [0, 0, 1, 2, 3, 3])


def test_bucketed_workspace_sizes():
    counts = [10, 20, 5, 100, 3, 3]
    # fused: 4 buckets; every tensor lies in chunk 0 of its bucket (chunks
    # of 128 elements), so 6 runs of one 2048-element tile each and 8
    # workgroups per tile of the fullest chunk (2, 1, 1, 2 tiles); a table of
    # 3 + 4*(1 + 8) + 4*6 + 8*6 = 111 words, rounded to 256 bytes, then a
    # descriptor of 16 + 8*8 = 80 bytes per workgroup
    table = 111 * 8 // 256 * 256 + 256
    assert rar.bucketed_workspace_bytes(counts, 8, rar.BF16, 60) == table + 8 * 6 * 80  # 3840, a multiple of 256
    # stepwise: 8 flat buffers of the largest padded bucket (100 bf16 -> 208 bytes -> 256)
    assert rar.bucketed_workspace_bytes(counts, 8, rar.BF16, 60, rar.ALGO_STEPWISE) == 8 * 256


def _fused_workspace_from_header(counts, n, dt, cap):
    """The FUSED workspace size as include/rar.h states it, from the bucket
    plan: a table of 3 + nb*(1 + n) + 4*nruns + n*nt words, then a
    descriptor of roundup(16 + 8n, 16) bytes per fold workgroup."""
    es = {rar.F32: 4, rar.F16: 2, rar.BF16: 2}[dt]
    tile = {rar.F32: 2048, rar.BF16: 2048, rar.F16: 4096}[dt]
    nb, plan = rar.bucket_plan(counts, dt, cap)
    padded = [-(-c * es // 16) * 16 // es for c in counts]
    nruns = wg = 0
    for b in range(nb):
        ts = [t for t in range(len(counts)) if plan[t] == b]
        total = sum(padded[t] for t in ts)
        L = -(-(-(-total // n)) // 128) * 128
        tiles = [0] * n
        off = 0
        for t in ts:
            pos, end = off, off + counts[t]
            while pos < end:  # the tensor's elements in chunk pos // L
                c = pos // L
                stop = min(end, (c + 1) * L)
                a, e = pos - off, stop - off
                tiles[c] += -(-(e - a // 64 * 64) // tile)
                nruns += 1
                pos = stop
            off += padded[t]
        wg += n * max(tiles)
    words = 3 + nb * (1 + n) + 4 * nruns + n * len(counts)
    stride = -(-(16 + 8 * n) // 16) * 16
    return -(-words * 8 // 256) * 256 + -(-wg * stride // 256) * 256


@pytest.mark.parametrize("dt", [rar.BF16, rar.F32, rar.F16])
@pytest.mark.parametrize("n", [2, 3, 8, 16])
def test_bucketed_workspace_follows_header_formula(dt, n):
    """Tensor sets with tensors across chunk ends, tensors smaller than a
    vector and empty tensors: the library's size equals the header's rule."""
    sets = [inputs.bucket_sizes(40, lo_exp=0, hi_exp=16, salt=n),
            [0, 5, 0, 300, 0, 0, 2049, 7, 0, 4096 * 3 + 1, 0, 16, 0],
            [70_001, 3, 250_000, 128, 99_999, 1 << 17]]
    for counts in sets:
        for cap in (4096, 48 << 10, 1 << 20):
            want = _fused_workspace_from_header(counts, n, dt, cap)
            assert rar.bucketed_workspace_bytes(counts, n, dt, cap) == want, (counts[:4], cap)


def test_bucketed_workspace_of_the_buckets_workload():
    w = inputs.WORKLOADS["buckets"]
    counts = inputs.bucket_sizes(w["ntensors"])
    got = rar.bucketed_workspace_bytes(counts, w["n"], rar.BF16, w["cap_bytes"])
    assert got == _fused_workspace_from_header(counts, w["n"], rar.BF16, w["cap_bytes"])
    assert got < 32 << 20  # 115,088 descriptors of 144 bytes and the table


class _FakeTensor:
    """Stands in for a device tensor in argument-error tests (never launched)."""

    def __init__(self, ptr, numel, dtype):
        import torch
        self._ptr, self._n, self.dtype = ptr, numel, dtype
        self.device = torch.device("cuda", 0)  # claims a GPU address; never launched

    def data_ptr(self):
        return self._ptr

    def numel(self):
        return self._n

    def is_contiguous(self):
        return True


def _fake(ptrs, numel=1024):
    import torch
    return [_FakeTensor(p, numel, torch.float32) for p in ptrs]


def test_argument_errors_are_reported_before_any_launch():
    base = 1 << 40
    with pytest.raises(rar.RarError) as e:
        rar.ring_allreduce(_fake([base + 8, base + 65536]), stream=0)
    assert e.value.status == 3  # misaligned
    with pytest.raises(rar.RarError) as e:
        rar.ring_allreduce(_fake([base, base + 1024]), stream=0)  # 4 KiB buffers 1 KiB apart
    assert e.value.status == 7
    with pytest.raises(rar.RarError) as e:
        rar.rs_step(_fake([base, base + 65536]), 2, stream=0)  # step must be 1..N-1
    assert e.value.status == 1
    with pytest.raises(rar.RarError) as e:
        rar.broadcast(_fake([base, base + 65536]), root=2, stream=0)
    assert e.value.status == 1
    with pytest.raises(rar.RarError) as e:
        rar.allgather(_fake([base, base + 65536, base + 131072], numel=1000), stream=0)
    assert e.value.status == 1
    # 65 ranks is beyond the limit
    lib = rar.lib()
    ptrs = (ctypes.c_void_p * 65)(*[base + i * 65536 for i in range(65)])
    assert lib.rar_ring_allreduce(ptrs, 65, 16, 0, None) == 1
    assert lib.rar_ring_allreduce(ptrs, 2, 16, 7, None) == 2  # dtype
    assert lib.rar_ring_allreduce_ex(ptrs, 2, 16, 0, 5, None) == 1  # algo


def test_noop_cases_need_no_device():
    base = 1 << 40
    rar.ring_allreduce(_fake([base, base + 65536], numel=0), stream=0)
    rar.ring_allreduce(_fake([base], numel=4096), stream=0)
    sent, recv = rar.last_traffic(1)
    assert sent == [0] and recv == [0]


def test_compressed_rejects_small_workspace():
    base = 1 << 40
    lib = rar.lib()
    ptrs = (ctypes.c_void_p * 2)(base, base + (1 << 20))
    cfg = rar.compress_cfg(schedule=rar.SCHED_STAGED)
    rc = lib.rar_ring_allreduce_compressed(ptrs, 2, 4096, rar.F16, ctypes.byref(cfg), base + (4 << 20), 64, None)
    assert rc == 4


def test_traffic_of_noop_allreduce_follows_byte_table():
    """count=0 still records the (zero) byte table; a valid count records it
    host-side before launching, which the GPU tests check against the oracle."""
    base = 1 << 40
    rar.ring_allreduce(_fake([base, base + 65536, base + 131072], numel=0), stream=0)
    assert rar.last_traffic(3) == ([0, 0, 0], [0, 0, 0])


def test_stateful_compressed_argument_errors():
    """Checks of rar_ring_allreduce_compressed_state that end before any launch."""
    base = 1 << 40
    lib = rar.lib()
    bufs = (ctypes.c_void_p * 2)(base, base + (1 << 20))
    state = (ctypes.c_void_p * 2)(base + (2 << 20), base + (3 << 20))
    ws = base + (8 << 20)
    count = 4096

    def call(st=state, fb=rar.FEEDBACK_ERROR, cfg=None, wsb=1 << 16):
        cfg = cfg if cfg is not None else rar.compress_cfg()
        return lib.rar_ring_allreduce_compressed_state(bufs, st, 2, count, rar.F16, fb, ctypes.byref(cfg), ws, wsb,
                                                       None)

    assert call(fb=0) == 1 and call(fb=3) == 1
    assert call(cfg=rar.compress_cfg(schedule=rar.SCHED_STAGED)) == 6
    assert call(cfg=rar.compress_cfg(method=rar.COMP_SPARSE_AUTO)) == 6
    assert call(cfg=rar.compress_cfg(collective_mask=rar.OP_ALLGATHER)) == 6
    assert call(cfg=rar.compress_cfg(mbits=9)) == 1
    assert call(st=(ctypes.c_void_p * 2)(base + (2 << 20), base + 4096)) == 7  # state inside rank 0's buffer
    assert call(st=(ctypes.c_void_p * 2)(base + (2 << 20), base + (2 << 20) + 8192)) == 7  # 16 KiB states overlap
    assert call(st=(ctypes.c_void_p * 2)(base + (2 << 20), base + (3 << 20) + 4)) == 3
    assert call(st=(ctypes.c_void_p * 2)(base + (2 << 20), None)) == 7
    assert call(wsb=64) == 4


def test_ft_workspace_and_argument_errors():
    assert rar.ft_workspace_bytes(4, 1000, rar.F32) == 512 + 4 * 4096
    assert rar.ft_workspace_bytes(0, 10, rar.F32) == 0
    base = 1 << 40
    lib = rar.lib()
    ptrs = (ctypes.c_void_p * 2)(base, base + (1 << 20))
    rep = rar.FtReport()
    faults = (rar.Fault * 1)(rar.Fault(2, 1))
    ws = base + (8 << 20)
    assert lib.rar_ring_allreduce_ft(ptrs, 2, 256, rar.F32, faults, 1, 0, ws, 1 << 20, ctypes.byref(rep), None) == 1
    faults[0] = rar.Fault(1, 0)
    assert lib.rar_ring_allreduce_ft(ptrs, 2, 256, rar.F32, faults, 1, 0, ws, 1 << 20, ctypes.byref(rep), None) == 1
    faults[0] = rar.Fault(1, 1, -5)
    assert lib.rar_ring_allreduce_ft(ptrs, 2, 256, rar.F32, faults, 1, 0, ws, 1 << 20, ctypes.byref(rep), None) == 1
    faults[0] = rar.Fault(1, 1)
    assert lib.rar_ring_allreduce_ft(ptrs, 2, 256, rar.F32, faults, 1, 0, ws, 64, ctypes.byref(rep), None) == 4
    assert lib.rar_ring_allreduce_ft(ptrs, 2, 256, rar.F32, faults, 1, 0, ws, 1 << 20, None, None) == 1
    hs = (ctypes.c_uint64 * 2)()
    assert lib.rar_rank_hashes(ptrs, 2, 64, ws, 100, hs, None) == 4
    assert lib.rar_rank_hashes(ptrs, 2, 64, ws + 8, 512, hs, None) == 3


def test_hash_of_empty_buffers_needs_no_device(orc):
    base = 1 << 40
    lib = rar.lib()
    ptrs = (ctypes.c_void_p * 3)(base, base, base)
    hs = (ctypes.c_uint64 * 3)()
    assert lib.rar_rank_hashes(ptrs, 3, 0, base, 512, hs, None) == 0
    assert list(hs) == [orc.hash64(np.zeros(0, np.uint8))] * 3


def _fault_plans(n, seed):
    """(rank, step, stall_ms) plans; stalls of 1-4 ms against a 2 ms deadline."""
    g = np.random.default_rng(seed)
    plans = [[], [(0, 1, 0)], [(n - 1, max(1, 2 * (n - 1)), 0)], [(r, 1, 0) for r in range(n)],
             [(0, 1, 1), (n - 1, 1, 3)]]
    for _ in range(20):
        k = int(g.integers(1, 5))
        plans.append([(int(g.integers(0, n)), int(g.integers(1, 2 * n)), int(g.choice([0, 0, 1, 3])))
                      for _ in range(k)])
    return plans


@pytest.mark.parametrize("n", [1, 2, 3, 5, 8, 16])
def test_ft_scheduler_matches_oracle_on_empty_buffers(orc, n):
    """count = 0 runs the fault scheduler on the host alone (no copies, no
    launches): attempts, failed ranks, steps and survivors match the oracle's."""
    base = 1 << 40
    lib = rar.lib()
    ptrs = (ctypes.c_void_p * n)(*[base + i * 4096 for i in range(n)])
    import time
    for plan in _fault_plans(n, n):
        arr = (rar.Fault * max(1, len(plan)))(*[rar.Fault(r, s, w) for r, s, w in plan])
        rep = rar.FtReport()
        t = time.perf_counter()
        rc = lib.rar_ring_allreduce_ft(ptrs, n, 0, rar.F32, arr, len(plan), 2, base, 512, ctypes.byref(rep), None)
        took_ms = (time.perf_counter() - t) * 1e3
        ref = orc.ring_allreduce_ft([np.zeros(0, np.float32) for _ in range(n)], plan, deadline_ms=2)
        assert list(rep.dead_reason)[:n] == ref["dead_reason"], plan
        assert rep.waited_ms == ref["waited_ms"] and took_ms >= rep.waited_ms * 0.99, plan
        assert rc == (rar.EABORT if ref["status"] == orc.EABORT else 0), plan
        assert rep.attempts == ref["attempts"], plan
        assert list(rep.survivors)[:rep.nsurvivors] == ref["survivors"], plan
        assert list(rep.dead_attempt)[:n] == ref["dead_attempt"], plan
        assert list(rep.dead_step)[:n] == ref["dead_step"], plan
        assert rar.last_traffic(n) == ([0] * n, [0] * n)


def test_binding_refuses_host_tensors():
    """A host tensor's address is not device memory: the binding stops it."""
    import torch
    x = [torch.zeros(1024), torch.zeros(1024)]
    with pytest.raises(ValueError, match="GPU tensor"):
        rar.ring_allreduce(x, stream=0)
    with pytest.raises(ValueError, match="GPU tensor"):
        rar.bfp_compress(x[0], 128, 8, torch.zeros(2048, dtype=torch.uint8), stream=0)


def test_rank_tensors_placement():
    """rank_tensors: tensor t at the same aligned offset in every rank's
    region, regions a power of two bytes apart and disjoint."""
    import torch
    counts = [5, 300, 7, 1, 4096]
    arena, views = rar.rank_tensors(3, counts, torch.bfloat16, "cpu", align_elems=64)
    base = arena.data_ptr()
    stride = (views[1][0].data_ptr() - base)
    assert stride > 0 and stride & (stride - 1) == 0
    for r in range(3):
        for t, c in enumerate(counts):
            x = views[r][t]
            assert x.numel() == c and x.is_contiguous()
            off = x.data_ptr() - base - r * stride
            assert off == views[0][t].data_ptr() - base and off % (64 * 2) == 0
            assert off + c * 2 <= stride
    ends = [(v.data_ptr(), v.data_ptr() + v.numel() * 2) for row in views for v in row]
    ends.sort()
    assert all(a[1] <= b[0] for a, b in zip(ends, ends[1:]))


def test_compress_cfg_rejects_unknown_fields():
    cfg = rar.compress_cfg(block=32, mbits=4)
    assert (cfg.block, cfg.mbits) == (32, 4)
    with pytest.raises(TypeError, match="unknown field 'mbit'"):
        rar.compress_cfg(mbit=4)


def test_workspace_overlapping_a_rank_buffer_is_refused():
    """A workspace that shares bytes with a rank (or state) buffer would be
    written while the kernels read those buffers: RAR_EOVERLAP before any
    launch, for every call that takes a workspace next to rank buffers."""
    base = 1 << 40
    lib = rar.lib()
    count = 4096  # 8 KiB of fp16 per rank
    bufs = (ctypes.c_void_p * 2)(base, base + (1 << 20))
    for sched in (rar.SCHED_FUSED, rar.SCHED_STAGED, rar.SCHED_FORWARD):
        cfg = rar.compress_cfg(schedule=sched, unit_bytes=4096)
        need = rar.compressed_workspace_bytes(2, count, rar.F16, cfg)
        call = lambda ws: lib.rar_ring_allreduce_compressed(bufs, 2, count, rar.F16, ctypes.byref(cfg), ws, need,
                                                            None)
        assert call(base + (1 << 20) + 4096) == 7, sched       # inside rank 1
        assert call(base + (1 << 20) - need + 16) == 7, sched  # its tail runs into rank 1
    state = (ctypes.c_void_p * 2)(base + (2 << 20), base + (3 << 20))
    cfg = rar.compress_cfg()
    need = rar.compressed_workspace_bytes(2, count, rar.F16, cfg)
    assert lib.rar_ring_allreduce_compressed_state(bufs, state, 2, count, rar.F16, rar.FEEDBACK_ERROR,
                                                   ctypes.byref(cfg), base + (3 << 20) + 1024, need, None) == 7
    ftws = rar.ft_workspace_bytes(2, count, rar.F16)
    rep = rar.FtReport()
    faults = (rar.Fault * 1)(rar.Fault(1, 1))
    assert lib.rar_ring_allreduce_ft(bufs, 2, count, rar.F16, faults, 0, 0, base + 8192 - 512, ftws,
                                     ctypes.byref(rep), None) == 7


def test_bucketed_refuses_overlapping_tensors_and_workspace():
    base = 1 << 40
    lib = rar.lib()
    counts = [1000, 3000]
    n = 2
    csz = (ctypes.c_size_t * 2)(*counts)
    need = rar.bucketed_workspace_bytes(counts, n, rar.BF16, 25 << 20)
    region = 1 << 20

    def call(tens, ws):
        arr = (ctypes.c_void_p * len(tens))(*tens)
        return lib.rar_bucketed_allreduce_ex(arr, csz, 2, n, rar.BF16, 25 << 20, rar.ALGO_FUSED, ws, need, None)

    ok = [base, base + 2048, base + region, base + region + 2048]
    ws = base + 4 * region
    # tensor 1 of rank 0 starts inside its tensor 0 (1000 bf16 = 2000 bytes)
    assert call([base, base + 1024, base + region, base + region + 2048], ws) == 7
    # rank 1's tensor 0 inside rank 0's tensor 1
    assert call([base, base + 2048, base + 4096, base + region + 2048], ws) == 7
    assert call(ok, base + region + 2048 + 16) == 7  # workspace inside rank 1's tensor 1
    assert call(ok, 0) == 4


def test_bucketed_plan_argument_errors():
    """rar_bucketed_prepare / rar_bucketed_launch refuse a missing or
    malformed plan before touching the device; a plan with nothing to fold
    launches nothing and reports its byte counters."""
    import ctypes
    from ring_all_reduce_scatter_amd import _binding as b
    L = b.lib()
    assert L.rar_bucketed_launch(None, None) == 1  # RAR_EINVAL
    plan = b.BucketedPlan()
    assert L.rar_bucketed_launch(ctypes.byref(plan), None) == 1  # RAR_EINVAL: nranks 0
    plan.nranks, plan.dtype = 4, rar.BF16
    plan.grid = 5  # workgroups to launch but no workspace
    assert L.rar_bucketed_launch(ctypes.byref(plan), None) == 1  # RAR_EINVAL
    plan.workspace, plan.desc_offset = 4096, 8  # descriptors not 16-byte aligned
    assert L.rar_bucketed_launch(ctypes.byref(plan), None) == 1  # RAR_EINVAL
    plan.grid, plan.workspace, plan.desc_offset = 0, None, 0
    for r in range(4):
        plan.sent[r], plan.recv[r] = 10 * r + 1, 10 * r + 2
    assert L.rar_bucketed_launch(ctypes.byref(plan), None) == 0
    assert rar.last_traffic(4) == ([1, 11, 21, 31], [2, 12, 22, 32])
    counts = (ctypes.c_size_t * 1)(8)
    assert L.rar_bucketed_prepare(None, counts, 1, 2, rar.BF16, 64, None, 0, None, None) == 1  # RAR_EINVAL
