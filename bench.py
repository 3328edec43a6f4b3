#!/usr/bin/env python3
"""Benchmark of the ring all-reduce hot path on one MI355X.

Headline: ring allreduce, N=8 simulated ranks, T=64M fp32 per rank (256 MiB),
gradient-like values N(0, 1e-3) with 1% outliers x100, fused schedule.  The
metric is the per-rank bus bandwidth 2*S*(N-1)/N / t (S = bytes per rank)
and the fraction of the HBM roofline the fused kernel reaches.  Further
legs on the same line: the BFP-8 compressed allreduce (N=8, T=128M fp16,
128-element blocks, block-scaled values) in the fused schedule ("bfp8") and
in the pipelined 4 MiB-unit schedule with every message materialised
("bfp8_pipelined"), and the sparse + BFP-4 allreduce (N=8, T=64M fp16)
pipelined and staged ("sparse_bfp4").  Inputs are generated on the host
once, copied into a pool of device sets, and every timed step runs on a
fresh set, so no restore happens inside the timed region.

Prints ONE JSON line.  --gpus above 1 is refused: all simulated ranks share
one GPU's HBM.
"""
import argparse
import hashlib
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "all-reduce bus GB/s (2T(N-1)/N per rank) and % of HBM peak, fp32 & BFP8"


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def host_info():
    model = platform.processor() or "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"cpu_model": model, "host_threads": os.cpu_count()}


_CSRC = "ring_all_reduce_scatter_amd/csrc/"
MIB = 1 << 20
# Kernels whose HBM traffic the counter passes measure: the name fragment
# that picks their dispatches in a rocprofv3 counter CSV, the algorithmic
# bytes of one launch in the counters run, and the sources that define them
# (the committed figures are used only while these are unchanged).
COUNTER_KERNELS = {
    "ring_fold_f32_n8": {
        "match": "::ring_fold_kernel<0, 8,", "workload": "N=8 x 64M fp32",
        "algorithmic": 2 * 8 * 256 * MIB, "sources": [_CSRC + "ring_kernels.hip", _CSRC + "common.hpp"]},
    "bfp_ring_fold_f16_n8": {
        "match": "::bfp_ring_fold_kernel<1, 8, 16,", "workload": "N=8 x 128M fp16, BFP-8",
        "algorithmic": 2 * 8 * 256 * MIB,
        "sources": [_CSRC + "bfp_kernels.hip", _CSRC + "bfp_device.hpp", _CSRC + "common.hpp"]},
    "bfp_ring_fold_state_f16_n8": {
        "match": "::bfp_ring_fold_state_q_kernel<1, 8, 32, 1>",
        "workload": "N=8 x 128M fp16, BFP-8, error feedback (128M fp32 state per rank)",
        "algorithmic": 2 * 8 * 256 * MIB + 2 * 8 * 512 * MIB,
        "sources": [_CSRC + "bfp_kernels.hip", _CSRC + "bfp_device.hpp", _CSRC + "common.hpp"]},
    "rank_hash_f32_n8": {
        "match": "::rank_hash_kernel", "workload": "N=8 x 256 MiB",
        "algorithmic": 8 * 256 * MIB, "sources": [_CSRC + "hash_kernels.hip", _CSRC + "common.hpp"]},
    "bfp_pipe_f16_n8": {
        "match": "::bfp_pipe_h16_kernel<8, 1, true>", "workload": "N=8 x 128M fp16, BFP-8, pipelined, 4 MiB units",
        # inputs read once, outputs written once, every message (N per chunk and unit) written once
        "algorithmic": 2 * 8 * 256 * MIB + 8 * 8 * 8 * (16384 + 2 * MIB),
        "sources": [_CSRC + "pipe_kernels.hip", _CSRC + "h16_codec.hpp", _CSRC + "bfp_device.hpp",
                    _CSRC + "common.hpp"]},
    "bucket_fold_bf16_n16": {
        "match": "::bucket_fold_kernel<2, 16,", "workload": "N=16 bf16, 200 gradient tensors in 25 MiB buckets",
        # every rank's copy of every gradient element read once and written once
        "algorithmic": lambda: 2 * 16 * 2 * _bucket_elements(),
        "sources": [_CSRC + "bucket_kernels.hip", _CSRC + "common.hpp", _CSRC + "api.hip"]},
}


# Multi-launch pipelines whose HBM bytes per call the counter passes measure:
# every dispatch of the listed kernels in the counters run belongs to one of
# `calls` calls of that pipeline.
PIPELINE_COUNTERS = {
    "bfp8_allreduce_staged": {
        "matches": ["::bfp_encode_kernel<", "::bfp_decode_kernel<", "::bfp_decode_fanout_kernel<"], "calls": 3,
        "workload": "staged BFP-8 allreduce, N=8 x 128M fp16, 4 MiB units",
        "sources": [_CSRC + "bfp_kernels.hip", _CSRC + "bfp_device.hpp", _CSRC + "common.hpp", _CSRC + "api.hip"]},
    "sparse_bfp4_allreduce_staged": {
        "matches": ["::comp_count_kernel<", "::comp_write_kernel<", "::comp_decode_acc_kernel<",
                    "::comp_decode_fanout_kernel<"], "calls": 3,
        "workload": "staged sparse + BFP-4 allreduce, N=8 x 64M fp16, ranks 0-3 95% zeros",
        "sources": [_CSRC + "sparse_kernels.hip", _CSRC + "bfp_device.hpp", _CSRC + "common.hpp", _CSRC + "api.hip"]},
    "sparse_bfp4_allreduce_pipelined": {
        "matches": ["::sparse_pipe_kernel<", "zero_u64_kernel"], "calls": 3,
        "workload": "pipelined sparse + BFP-4 allreduce, N=8 x 64M fp16, ranks 0-3 95% zeros",
        "sources": [_CSRC + "sparse_pipe_kernels.hip", _CSRC + "block_scan.hpp", _CSRC + "h16_codec.hpp",
                    _CSRC + "bfp_device.hpp", _CSRC + "common.hpp", _CSRC + "api.hip"]},
}


def pipeline_traffic(key):
    """HBM bytes per call of a multi-launch pipeline from profiles/counters.json,
    or None when absent or taken on other sources."""
    try:
        with open(os.path.join(ROOT, "profiles", "counters.json")) as f:
            rec = json.load(f).get("pipelines", {}).get(key)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_sha") != source_sha(PIPELINE_COUNTERS[key]["sources"]):
        return None
    return rec.get("hbm_bytes_per_call")


def _bucket_elements():
    from ring_all_reduce_scatter_amd import inputs
    return sum(inputs.bucket_sizes(inputs.WORKLOADS["buckets"]["ntensors"]))


def _algorithmic(k):
    return k["algorithmic"]() if callable(k["algorithmic"]) else k["algorithmic"]
# validation copy of the counters run: 256 MiB read and 256 MiB written
CALIBRATION = {"match": "copy_jobs_kernel", "bytes": 256 * MIB}
# HBM bytes are measured, not calibrated: the TCC counts every read request
# sent to DRAM and every write request written to DRAM in 32-byte units (a
# 64-byte request counts 2, a 128-byte one 4).  The 128-byte read requests
# and TCC_BUBBLE (which FETCH_SIZE takes as the 128-byte reads) come in the
# same pass: on gfx950 TCC_BUBBLE stays near zero while the reads are
# 128-byte requests, so FETCH_SIZE charges them 64 bytes and reads half.
PMC_COUNTERS = ["TCC_EA0_RDREQ_DRAM_32B_sum", "TCC_EA0_WRREQ_WRITE_DRAM_32B_sum", "TCC_EA0_RDREQ_128B_sum",
                "TCC_BUBBLE_sum"]
# R = the repository root, OUT = any directory for the profiler's files
PMC_COMMANDS = [
    "cd /tmp && export TMPDIR=/tmp && timeout -s KILL 300 rocprofv3 --pmc " + " ".join(PMC_COUNTERS) +
    " --output-format csv -d $OUT/pmc_dram -o pmc -- python -u $R/bench.py --counters",
    "python bench.py --ingest-counters $OUT/pmc_dram/pmc_counter_collection.csv",
]


def source_sha(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def counter_traffic(key, sources):
    """HBM bytes per launch from the committed rocprofv3 counter summary,
    or None when the kernel source changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", "counters.json")
    if not os.path.exists(path):
        return None
    try:
        with open(path) as f:
            rec = json.load(f).get(key)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_sha") != source_sha(sources):
        return None
    return rec.get("hbm_bytes_per_launch")


def make_sets(pristine, nsets):
    """nsets device copies of the rank buffers (one allocation per set)."""
    import torch
    n, count = len(pristine), pristine[0].numel()
    sets = []
    for _ in range(nsets):
        big = torch.empty(n * count, dtype=pristine[0].dtype, device=pristine[0].device)
        views = [big[r * count:(r + 1) * count] for r in range(n)]
        for v, p in zip(views, pristine):
            v.copy_(p)
        sets.append(views)
    return sets


class LegTimes(tuple):
    """(wall ms per step, mean event ms, min event ms) with .median_ms."""
    median_ms = None


def time_leg(run, sets, warmup, steps):
    """Warm up on set 0, then time `steps` calls, each on a fresh set.
    Returns wall ms per step and the HIP-event kernel ms (mean, min); the
    median of the event times is the result's median_ms."""
    import torch
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        run(sets[0])
    torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        starts[i].record(stream)
        run(sets[1 + i % (len(sets) - 1)])
        ends[i].record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ev = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    out = LegTimes(((t1 - t0) * 1e3 / steps, sum(ev) / len(ev), min(ev)))
    out.median_ms = sorted(ev)[len(ev) // 2]
    return out


def time_graph_leg(run, sets, steps):
    """Like time_leg, but each set's call is captured once in a HIP graph and
    the timed steps replay the graphs (one per set, so inputs stay fresh)."""
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run(sets[0])  # library streams and events exist before any capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graphs = []
    for b in sets[1:]:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            run(b)
        graphs.append(g)
    torch.cuda.synchronize()
    graphs[0].replay()  # first replay uploads the graph
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    t0 = time.perf_counter()
    for i in range(steps):
        starts[i].record(stream)
        graphs[1 + i % (len(graphs) - 1) if len(graphs) > 1 else 0].replay()
        ends[i].record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ev = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    del graphs
    return (t1 - t0) * 1e3 / steps, sum(ev) / len(ev), min(ev)


def busbw(bytes_per_rank, n, ms):
    return 2.0 * bytes_per_rank * (n - 1) / n / (ms * 1e-3) / 1e9


class pinned_core:
    """Run the enclosed CPU work on one host core (the last one this process
    may use), restoring the previous affinity afterwards."""

    def __enter__(self):
        self.prev = os.sched_getaffinity(0)
        self.core = max(self.prev)
        os.sched_setaffinity(0, {self.core})
        return self

    def __exit__(self, *exc):
        os.sched_setaffinity(0, self.prev)
        return False


def copy_peak(reps=10):
    """Achievable HBM rate of a plain copy on this GPU: 2 GiB read and 2 GiB
    written (the fused folds' 4 GiB per launch) by the library's copy kernel
    (a 2-rank broadcast) and by torch's device-to-device copy, median of
    `reps` launches each, timed with HIP events on the launch stream; the
    faster of the two is the peak."""
    import torch

    import ring_all_reduce_scatter_amd as rar
    count = 512 << 20
    bufs = [torch.full((count,), float(r + 1), device="cuda:0") for r in range(2)]
    stream = torch.cuda.current_stream()

    def median_ms(run):
        run()
        torch.cuda.synchronize()
        ms = []
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            run()
            b.record(stream)
            b.synchronize()
            ms.append(a.elapsed_time(b))
        ms.sort()
        return ms[len(ms) // 2]

    rates = {"copy_jobs_kernel": median_ms(lambda: rar.broadcast(bufs, 0)),
             "torch copy_ (device to device)": median_ms(lambda: bufs[1].copy_(bufs[0]))}
    name = min(rates, key=rates.get)
    t = rates[name]
    return {"value": round(2 * count * 4 / (t * 1e-3) / 1e9, 1), "unit": "GB/s", "kernel": name,
            "bytes": 2 * count * 4,
            "ms": {k: round(v, 4) for k, v in rates.items()}}


def fp32_leg(args):
    import numpy as np
    import torch

    import ring_all_reduce_scatter_amd as rar
    from ring_all_reduce_scatter_amd import inputs

    w = inputs.WORKLOADS["ring_grad"]
    n, count = w["n"], w["count"]
    log(f"[bench] fp32 leg: generating N={n} x T={count} inputs")
    xs = inputs.gradient_like(n, count)
    pristine = [torch.from_numpy(x).to("cuda:0") for x in xs]
    nsets = 1 + min(args.steps, args.max_sets)
    sets = make_sets(pristine, nsets)
    del pristine
    S = count * 4
    log(f"[bench] fp32 leg: timing {args.steps} steps on {nsets - 1} sets")
    tl = time_leg(lambda bufs: rar.ring_allreduce(bufs), sets, args.warmup, args.steps)
    ms, kern_ms, kern_min = tl
    sent, recv = rar.last_traffic(n)  # logical bytes per rank of the last call
    first = [t.cpu().numpy() for t in sets[1]]
    del sets
    torch.cuda.empty_cache()
    alg_bytes = 2 * n * S  # every rank's input read once and output written once
    achieved = alg_bytes / (kern_ms * 1e-3) / 1e9
    sources = COUNTER_KERNELS["ring_fold_f32_n8"]["sources"]
    res = {
        "n": n, "count": count, "S": S, "ms": ms, "kern_ms": kern_ms, "kern_min_ms": kern_min,
        "kern_median_ms": tl.median_ms,
        "bytes_per_rank": {"sent": sent, "recv": recv},
        "busbw": busbw(S, n, ms),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": counter_traffic("ring_fold_f32_n8", sources),
                     "kernel": "ring_fold_kernel<f32, N=8>", "algorithmic_bytes_per_launch": alg_bytes},
    }
    parity = None
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        log("[bench] fp32 leg: oracle on the full workload (single thread), about 10 s of runs")
        times = []
        with pinned_core() as pin:
            bufs = [x.copy() for x in xs]
            t = time.perf_counter()
            oracle.ring_allreduce(bufs)
            times.append(time.perf_counter() - t)
            parity = all(np.array_equal(first[r].view(np.uint32), bufs[r].view(np.uint32)) for r in range(n))
            # further runs in place on the same buffers (the work per run is the same)
            while sum(times) < 10.0 and len(times) < 99:
                t = time.perf_counter()
                oracle.ring_allreduce(bufs)
                times.append(time.perf_counter() - t)
        med = sorted(times)[len(times) // 2]
        cpu = {"value": round(busbw(S, n, med * 1e3), 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
               "sample": f"the whole workload (N={n}, T={count} fp32 per rank), median of {len(times)} "
                         f"single-thread runs ({med:.2f} s each, {sum(times):.1f} s in all) pinned to host core "
                         f"{pin.core}", **host_info()}
    if parity is None:
        parity = sampled_fp32_parity(xs, first, rar.chunk_len(count, n))
        res["parity_first_timed_output"] = parity
    else:
        res["parity_first_timed_output"] = "bit-exact (all elements)" if parity else "MISMATCH"
    res["cpu_baseline"] = cpu
    return res


def sampled_fp32_parity(xs, first, L, K=4096):
    """Windows of K elements from every chunk re-run in a small ring where
    each window keeps its chunk index (elements are independent)."""
    import numpy as np

    import oracle
    n, count = len(xs), xs[0].size
    g = np.random.default_rng(5)
    mini = [np.zeros(n * K, dtype=np.float32) for _ in range(n)]
    offs = []
    for c in range(n):
        hi = min((c + 1) * L, count)
        o = c * L + int(g.integers(0, max(1, hi - c * L - K)))
        offs.append(o)
        for r in range(n):
            mini[r][c * K:(c + 1) * K] = xs[r][o:o + K]
    oracle.ring_allreduce(mini)
    for c in range(n):
        for r in range(n):
            if not np.array_equal(first[r][offs[c]:offs[c] + K].view(np.uint32), mini[r][c * K:(c + 1) * K].view(np.uint32)):
                return "MISMATCH"
    return f"bit-exact on {n} sampled windows of {K} elements on every rank"


def bfp8_leg(args):
    import numpy as np
    import torch

    import ring_all_reduce_scatter_amd as rar
    from ring_all_reduce_scatter_amd import inputs

    w = inputs.WORKLOADS["bfp8"]
    n, count, mbits, block = w["n"], w["count"], w["mbits"], w["block"]
    log(f"[bench] bfp8 leg: generating N={n} x T={count} fp16 inputs")
    xs = inputs.block_scaled(n, count)
    pristine = [torch.from_numpy(x).to("cuda:0") for x in xs]
    nsets = 1 + min(args.steps, args.max_sets)
    sets = make_sets(pristine, nsets)
    cfg = rar.compress_cfg(block=block, mbits=mbits, unit_bytes=w["unit_bytes"], schedule=rar.SCHED_FUSED)
    ws = torch.empty(rar.compressed_workspace_bytes(n, count, rar.F16, cfg), dtype=torch.uint8, device="cuda:0")
    S = count * 2
    log(f"[bench] bfp8 leg: timing {args.steps} steps")
    ms, kern_ms, kern_min = time_leg(lambda bufs: rar.ring_allreduce_compressed(bufs, cfg, ws), sets,
                                     args.warmup, args.steps)
    sent, _ = rar.compressed_traffic(ws, n)
    got0 = sets[1][0].cpu().numpy()
    fused_out = sets[1][0].clone()
    same = all(torch.equal(sets[1][r].view(torch.int16), sets[1][0].view(torch.int16)) for r in range(n))
    # the same calls through the pipelined schedule (every message written to
    # the workspace and read back by its receiver), on fresh copies of the sets
    del ws
    for st in sets:
        for v, p in zip(st, pristine):
            v.copy_(p)
    del pristine
    pcfg = rar.compress_cfg(block=block, mbits=mbits, unit_bytes=w["unit_bytes"], schedule=rar.SCHED_PIPELINED)
    pws = torch.empty(rar.compressed_workspace_bytes(n, count, rar.F16, pcfg), dtype=torch.uint8, device="cuda:0")
    log(f"[bench] bfp8 leg: pipelined schedule, timing {args.steps} steps")
    ptl = time_leg(lambda bufs: rar.ring_allreduce_compressed(bufs, pcfg, pws), sets, args.warmup, args.steps)
    psame = bool(torch.equal(sets[1][0].view(torch.int16), fused_out.view(torch.int16)))
    del sets, pws, fused_out
    torch.cuda.empty_cache()
    alg_bytes = 2 * n * S
    achieved = alg_bytes / (kern_ms * 1e-3) / 1e9
    sources = COUNTER_KERNELS["bfp_ring_fold_f16_n8"]["sources"]
    res = {
        "metric": "BFP-8 compressed all-reduce effective bus GB/s (2T(N-1)/N fp16 bytes per rank)",
        "value": round(busbw(S, n, ms), 2), "unit": "GB/s", "ms_per_step": round(ms, 4),
        "dtype": "f16 buffers, 8-bit BFP messages",
        "wire_busbw_GBs": round(sent[0] / (ms * 1e-3) / 1e9, 2),
        "wire_bytes_per_rank": sent[0],
        "config": {"workload": f"compressed ring allreduce, N={n} ranks, T={count} fp16 per rank (256 MiB), "
                               f"block {block}, {mbits}-bit mantissas, x = s_b*N(0,1e-3), s_b=2^U(-12,0)",
                   "schedule": "fused"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": counter_traffic("bfp_ring_fold_f16_n8", sources),
                     "kernel": "bfp_ring_fold_kernel<f16, N=8, block 128>", "algorithmic_bytes_per_launch": alg_bytes},
        "ranks_identical": bool(same),
    }
    pk = COUNTER_KERNELS["bfp_pipe_f16_n8"]
    own = _algorithmic(pk)
    res["pipelined"] = {
        "schedule": "pipelined: 4 MiB units, every message written to the workspace and read back by its "
                    "receiver, one launch",
        "value": round(busbw(S, n, ptl[0]), 2), "unit": "GB/s", "ms_per_step": round(ptl[0], 4),
        "kernel_ms": round(ptl[1], 4), "kernel_ms_median": round(ptl.median_ms, 4),
        "frac_of_roofline": round(alg_bytes / (ptl[1] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "own_algorithmic_bytes": own,
        "frac_of_roofline_own_bytes": round(own / (ptl[1] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "traffic": counter_traffic("bfp_pipe_f16_n8", pk["sources"]),
        "kernel": "bfp_pipe_h16_kernel<N=8, 8-bit>",
        "equals_fused_bits": psame,
    }
    if not args.no_cpu_baseline:
        import oracle
        sample = count // 16
        log(f"[bench] bfp8 leg: oracle on a sample of T={sample} per rank")
        xs_s = inputs.block_scaled(n, sample, salt=1)
        times = []
        with pinned_core() as pin:
            for _ in range(3):
                bufs = [x.copy() for x in xs_s]
                t = time.perf_counter()
                oracle.ring_allreduce_compressed(bufs, mbits=mbits, unit=w["unit_bytes"] // 2)
                times.append(time.perf_counter() - t)
        dt = sorted(times)[1]
        res["cpu_baseline"] = {"value": round(busbw(sample * 2, n, dt * 1e3), 5), "unit": "GB/s", "cores": 1,
                               "kind": "oracle",
                               "sample": f"N={n}, T={sample} fp16 per rank (1/16 of the workload, same value "
                                         f"recipe), median of 3 single-thread runs ({dt:.1f} s each, "
                                         f"{sum(times):.1f} s in all) pinned to host core {pin.core}"}
        res["parity_first_timed_output"] = sampled_bfp_parity(xs, got0, rar.compressed_chunk_len(count, n, block),
                                                              mbits)
    return res


def sparse_leg(args):
    """The sparse + BFP-4 workload (N=8, T=64M fp16, ranks 0-3 95% zeros, 4 MiB
    units) through the single-launch pipelined SPARSE_AUTO schedule; its first
    timed output is compared bit for bit with the staged schedule's."""
    import torch

    import ring_all_reduce_scatter_amd as rar
    from ring_all_reduce_scatter_amd import inputs

    w = inputs.WORKLOADS["sparse_bfp4"]
    n, count = w["n"], w["count"]
    log(f"[bench] sparse leg: generating N={n} x T={count} fp16 inputs")
    xs = inputs.sparse_mix(n, count)
    pristine = [torch.from_numpy(x).to("cuda:0") for x in xs]
    del xs
    steps = max(3, min(args.steps, 10))
    sets = make_sets(pristine, 1 + steps)
    S = count * 2
    out = {}
    firsts = {}
    for name, sched in (("pipelined", rar.SCHED_PIPELINED), ("staged", rar.SCHED_STAGED)):
        for st in sets:
            for v, p in zip(st, pristine):
                v.copy_(p)
        cfg = rar.compress_cfg(method=rar.COMP_SPARSE_AUTO, mbits=w["mbits"], unit_bytes=w["unit_bytes"],
                               sparsity_threshold=w["theta"], schedule=sched)
        ws = torch.empty(rar.compressed_workspace_bytes(n, count, rar.F16, cfg), dtype=torch.uint8, device="cuda:0")
        log(f"[bench] sparse leg: {name} schedule, timing {steps} steps")
        tl = time_leg(lambda b: rar.ring_allreduce_compressed(b, cfg, ws), sets, 2, steps)
        sent, _ = rar.compressed_traffic(ws, n)
        firsts[name] = sets[1][0].clone()
        key = f"sparse_bfp4_allreduce_{name}"
        tr = pipeline_traffic(key)
        out[name] = {"value": round(busbw(S, n, tl[0]), 2), "unit": "GB/s", "ms_per_step": round(tl[0], 4),
                     "kernel_ms": round(tl[1], 4), "kernel_ms_median": round(tl.median_ms, 4),
                     "frac_of_roofline": round(2 * n * S / (tl[1] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                     "wire_bytes_rank0": sent[0], "traffic_per_call": tr}
        if tr:
            out[name]["frac_of_roofline_own_bytes"] = round(tr / (tl[1] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)
        del ws
    same = bool(torch.equal(firsts["pipelined"].view(torch.int16), firsts["staged"].view(torch.int16)))
    del sets, pristine, firsts
    torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        import oracle
        sample = count // 4
        log(f"[bench] sparse leg: oracle on a sample of T={sample} per rank")
        xs_s = inputs.sparse_mix(n, sample, salt=1)
        dt, tot, core = oracle_runs(lambda: [x.copy() for x in xs_s], lambda b: oracle.ring_allreduce_compressed(
            b, method=oracle.COMP_SPARSE_AUTO, block=128, mbits=w["mbits"], theta=w["theta"],
            unit=w["unit_bytes"] // 2), 3)
        del xs_s
        out["pipelined"]["cpu_baseline"] = {
            "value": round(busbw(sample * 2, n, dt * 1e3), 5), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"N={n}, T={sample} fp16 per rank (1/4 of the workload, same recipe; each chunk one "
                      f"{w['unit_bytes'] >> 20} MiB unit), median of 3 single-thread runs ({dt:.1f} s each, "
                      f"{tot:.1f} s in all) pinned to host core {core}"}
    return {"metric": "sparse + BFP-4 compressed all-reduce effective bus GB/s (2T(N-1)/N fp16 bytes per rank)",
            "config": {"workload": f"sparsity-aware compressed ring allreduce, N={n} ranks, T={count} fp16 per rank, "
                                   f"ranks 0-{n // 2 - 1} 95% zeros, threshold {w['theta']}, dense messages BFP "
                                   f"4-bit on 128-element blocks, {w['unit_bytes'] >> 20} MiB units"},
            **out["pipelined"], "schedule": "pipelined (one cooperative launch)", "staged": out["staged"],
            "pipelined_equals_staged_bits": same}


def sampled_bfp_parity(xs, got0, L, mbits, per_chunk=64):
    """Re-run sampled blocks through the oracle in a small ring where each
    block keeps its chunk index (blocks are independent in the BFP ring)."""
    import numpy as np

    import oracle
    n, count = len(xs), xs[0].size
    g = np.random.default_rng(7)
    K = per_chunk
    mini = [np.zeros(n * K * 128, dtype=np.float16) for _ in range(n)]
    picks = []
    for c in range(n):
        nblk = (min((c + 1) * L, count) - c * L) // 128
        bl = np.sort(g.choice(nblk, size=K, replace=False)) + c * L // 128
        picks.append(bl)
        for r in range(n):
            for k, b in enumerate(bl):
                mini[r][(c * K + k) * 128:(c * K + k + 1) * 128] = xs[r][b * 128:(b + 1) * 128]
    oracle.ring_allreduce_compressed(mini, mbits=mbits, unit=K * 128)
    for c in range(n):
        for k, b in enumerate(picks[c]):
            a = got0[b * 128:(b + 1) * 128].view(np.uint16)
            e = mini[0][(c * K + k) * 128:(c * K + k + 1) * 128].view(np.uint16)
            if not np.array_equal(a, e):
                return "MISMATCH"
    return f"bit-exact on {n * K} sampled blocks"


def oracle_runs(make, call, runs):
    """Single-thread oracle calls on a pinned host core, each on fresh inputs
    from make() (prepared outside the timed part): median seconds, total
    seconds, the core."""
    times = []
    with pinned_core() as pin:
        for _ in range(runs):
            a = make()
            t = time.perf_counter()
            call(a)
            times.append(time.perf_counter() - t)
    times.sort()
    return times[len(times) // 2], sum(times), pin.core


def extra_legs(args):
    """Secondary schedules and collectives (reported, not the headline)."""
    import numpy as np
    import torch

    import ring_all_reduce_scatter_amd as rar
    from ring_all_reduce_scatter_amd import inputs

    out = {}
    steps = max(3, min(args.steps, 10))
    w = inputs.WORKLOADS["ring_grad"]
    n, count = w["n"], w["count"]
    xs = inputs.gradient_like(n, count)
    pristine = [torch.from_numpy(x).to("cuda:0") for x in xs]
    sets = make_sets(pristine, 1 + steps)
    S = count * 4
    ms, k, _ = time_leg(lambda b: rar.ring_allreduce_ex(b, rar.ALGO_STEPWISE), sets, 2, steps)
    out["fp32_allreduce_stepwise"] = {"ms": round(ms, 4), "busbw_GBs": round(busbw(S, n, ms), 1),
                                      "frac_of_roofline": round(2 * n * S / (k * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    ms, k, _ = time_leg(lambda b: rar.reduce_scatter(b), sets, 2, steps)
    out["fp32_reduce_scatter_fused"] = {"ms": round(ms, 4),
                                        "busbw_GBs": round(S * (n - 1) / n / (ms * 1e-3) / 1e9, 1),
                                        "frac_of_roofline": round((n * S + S) / (k * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    # tree allreduce at the same size (binomial reduce + broadcast, fused: N reads + N writes)
    ms, k, _ = time_leg(lambda b: rar.tree_allreduce(b), sets, 2, steps)
    out["fp32_tree_allreduce_fused"] = {"ms": round(ms, 4), "busbw_GBs": round(busbw(S, n, ms), 1),
                                        "frac_of_roofline": round(2 * n * S / (k * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    # shared-state hash of every rank's buffer (reads N*S bytes; one host sync)
    hws = torch.empty(rar.HASH_WORKSPACE_BYTES, dtype=torch.uint8, device="cuda:0")
    ms, k, _ = time_leg(lambda b: rar.rank_hashes(b, hws), sets, 2, steps)
    out["rank_hashes_fp32_8x256MiB"] = {
        "ms": round(ms, 4), "read_GBs": round(n * S / (k * 1e-3) / 1e9, 1),
        "frac_of_roofline": round(n * S / (k * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "traffic": counter_traffic("rank_hash_f32_n8", COUNTER_KERNELS["rank_hash_f32_n8"]["sources"])}
    # fault-tolerant ring: no fault, and rank 3 failing before step 5 (snapshot,
    # 4 abandoned steps, restore, a 7-rank stepwise pass, hashes)
    fws = torch.empty(rar.ft_workspace_bytes(n, count, rar.F32), dtype=torch.uint8, device="cuda:0")
    for nm, plan in (("ft_ring_fp32_no_fault", []), ("ft_ring_fp32_rank3_fails_before_step5", [(3, 5)])):
        ms, k, _ = time_leg(lambda b: rar.ring_allreduce_ft(b, plan, fws), sets, 1, min(steps, 4))
        out[nm] = {"ms": round(ms, 4), "attempts": rar.ring_allreduce_ft(sets[0], plan, fws)["attempts"]}
    del fws, hws
    del sets, pristine
    torch.cuda.empty_cache()
    wb = inputs.WORKLOADS["bfp8"]
    xb = inputs.block_scaled(wb["n"], wb["count"])
    pristine = [torch.from_numpy(x).to("cuda:0") for x in xb]
    sets = make_sets(pristine, 1 + steps)
    cfg = rar.compress_cfg(unit_bytes=wb["unit_bytes"], schedule=rar.SCHED_STAGED)
    ws = torch.empty(rar.compressed_workspace_bytes(wb["n"], wb["count"], rar.F16, cfg), dtype=torch.uint8,
                     device="cuda:0")
    ms, k, _ = time_leg(lambda b: rar.ring_allreduce_compressed(b, cfg, ws), sets, 2, steps)
    Sb = wb["count"] * 2
    out["bfp8_allreduce_staged"] = {"ms": round(ms, 4), "busbw_GBs": round(busbw(Sb, wb["n"], ms), 1),
                                    "frac_of_roofline": round(2 * wb["n"] * Sb / (k * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    tr = pipeline_traffic("bfp8_allreduce_staged")
    out["bfp8_allreduce_staged"]["traffic_per_call"] = tr
    if tr:
        out["bfp8_allreduce_staged"]["frac_of_roofline_own_bytes"] = round(tr / (k * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)
    ms, k, _ = time_graph_leg(lambda b: rar.ring_allreduce_compressed(b, cfg, ws), sets, steps)
    out["bfp8_allreduce_staged_graph_replay"] = {
        "ms": round(ms, 4), "busbw_GBs": round(busbw(Sb, wb["n"], ms), 1),
        "frac_of_roofline": round(2 * wb["n"] * Sb / (k * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    del ws
    # standalone encode (K4) and decode-accumulate (K5) over one rank's 256 MiB
    x0 = sets[1][0]
    msg = torch.empty(rar.bfp_bytes(wb["count"], 128, 8), dtype=torch.uint8, device="cuda:0")
    mbytes = msg.numel()
    ms, k, _ = time_leg(lambda b: rar.bfp_compress(b[0], 128, 8, msg), sets, 2, steps)
    out["bfp8_compress_256MiB"] = {"ms": round(ms, 4), "bytes": Sb + mbytes,
                                   "frac_of_roofline": round((Sb + mbytes) / (k * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    ms, k, _ = time_leg(lambda b: rar.bfp_decompress_accumulate(msg, wb["count"], 128, 8, b[1]), sets, 2, steps)
    out["bfp8_decompress_accumulate_256MiB"] = {
        "ms": round(ms, 4), "bytes": mbytes + 2 * Sb,
        "frac_of_roofline": round((mbytes + 2 * Sb) / (k * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    del msg, x0
    # forwarding schedule: materialised messages, one decode+add+encode kernel per hop.
    # Its own traffic per element: hop 0 encode 2 + 1.008, N-1 forwarding hops
    # 1.008 + 2 + 1.008, allgather fan-out 1.008 + 2N (fp16, m = 8).
    cfg = rar.compress_cfg(unit_bytes=wb["unit_bytes"], schedule=rar.SCHED_FORWARD)
    ws = torch.empty(rar.compressed_workspace_bytes(wb["n"], wb["count"], rar.F16, cfg), dtype=torch.uint8,
                     device="cuda:0")
    ms, k, _ = time_leg(lambda b: rar.ring_allreduce_compressed(b, cfg, ws), sets, 2, steps)
    mb = 1.0 + 1.0 / 128
    own = wb["count"] * ((2 + mb) + (wb["n"] - 1) * (2 * mb + 2) + (mb + 2 * wb["n"]))
    out["bfp8_allreduce_forward"] = {
        "ms": round(ms, 4), "busbw_GBs": round(busbw(Sb, wb["n"], ms), 1),
        "frac_of_roofline": round(2 * wb["n"] * Sb / (k * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "own_bytes": int(own), "frac_of_roofline_own_bytes": round(own / (k * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    del ws
    # the same fused ring with per-rank error-feedback state (state read and
    # rewritten once per element per rank: 8 more bytes per element per rank)
    cfg = rar.compress_cfg(unit_bytes=wb["unit_bytes"], schedule=rar.SCHED_FUSED)
    ws = torch.empty(rar.compressed_workspace_bytes(wb["n"], wb["count"], rar.F16, cfg), dtype=torch.uint8,
                     device="cuda:0")
    state = [torch.zeros(wb["count"], dtype=torch.float32, device="cuda:0") for _ in range(wb["n"])]
    for nm, fb in (("bfp8_allreduce_fused_error_feedback", rar.FEEDBACK_ERROR),
                   ("bfp8_allreduce_fused_delta", rar.FEEDBACK_DELTA)):
        ms, k, _ = time_leg(lambda b: rar.ring_allreduce_compressed_state(b, state, fb, cfg, ws), sets, 2, steps)
        moved = 2 * wb["n"] * Sb + 2 * wb["n"] * wb["count"] * 4
        out[nm] = {"ms": round(ms, 4), "busbw_GBs": round(busbw(Sb, wb["n"], ms), 1),
                   "frac_of_roofline": round(moved / (k * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                   "algorithmic_bytes": moved}
    ck = COUNTER_KERNELS["bfp_ring_fold_state_f16_n8"]
    out["bfp8_allreduce_fused_error_feedback"]["traffic"] = counter_traffic("bfp_ring_fold_state_f16_n8",
                                                                            ck["sources"])
    if not args.no_cpu_baseline:
        import oracle
        sample = wb["count"] // 16
        log(f"[bench] stateful leg: oracle on a sample of T={sample} per rank")
        xs_s = inputs.block_scaled(wb["n"], sample, salt=1)
        dt, tot, core = oracle_runs(
            lambda: ([x.copy() for x in xs_s], [np.zeros(sample, dtype=np.float32) for _ in range(wb["n"])]),
            lambda a: oracle.ring_allreduce_compressed_state(a[0], a[1], oracle.FB_ERROR, block=128, mbits=8,
                                                             unit=wb["unit_bytes"] // 2), 3)
        del xs_s
        out["bfp8_allreduce_fused_error_feedback"]["cpu_baseline"] = {
            "value": round(busbw(sample * 2, wb["n"], dt * 1e3), 5), "unit": "GB/s", "cores": 1,
            "kind": "oracle",
            "sample": f"N={wb['n']}, T={sample} fp16 per rank with zero binary32 state (1/16 of the workload, "
                      f"same value recipe), median of 3 single-thread runs ({dt:.1f} s each, {tot:.1f} s in all) "
                      f"pinned to host core {core}"}
    del sets, pristine, ws, state
    torch.cuda.empty_cache()
    w5 = inputs.WORKLOADS["sparse_bfp4"]
    xsp = inputs.sparse_mix(w5["n"], w5["count"])
    pristine = [torch.from_numpy(x).to("cuda:0") for x in xsp]
    del xsp
    sets = make_sets(pristine, 1 + steps)
    cfg = rar.compress_cfg(method=rar.COMP_SPARSE_AUTO, mbits=w5["mbits"], unit_bytes=w5["unit_bytes"],
                           sparsity_threshold=w5["theta"], schedule=rar.SCHED_STAGED)
    ws = torch.empty(rar.compressed_workspace_bytes(w5["n"], w5["count"], rar.F16, cfg), dtype=torch.uint8,
                     device="cuda:0")
    ms, k, _ = time_leg(lambda b: rar.ring_allreduce_compressed(b, cfg, ws), sets, 2, steps)
    S5 = w5["count"] * 2
    sent, _ = rar.compressed_traffic(ws, w5["n"])
    out["sparse_bfp4_allreduce_staged"] = {"ms": round(ms, 4), "busbw_GBs": round(busbw(S5, w5["n"], ms), 1),
                                           "wire_bytes_rank0": sent[0],
                                           "frac_of_roofline": round(2 * w5["n"] * S5 / (k * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    tr = pipeline_traffic("sparse_bfp4_allreduce_staged")
    out["sparse_bfp4_allreduce_staged"]["traffic_per_call"] = tr
    if tr:
        out["sparse_bfp4_allreduce_staged"]["frac_of_roofline_own_bytes"] = round(
            tr / (k * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)
    ms, k, _ = time_graph_leg(lambda b: rar.ring_allreduce_compressed(b, cfg, ws), sets, steps)
    out["sparse_bfp4_allreduce_staged_graph_replay"] = {
        "ms": round(ms, 4), "busbw_GBs": round(busbw(S5, w5["n"], ms), 1),
        "frac_of_roofline": round(2 * w5["n"] * S5 / (k * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    del sets, pristine, ws
    torch.cuda.empty_cache()
    wk = inputs.WORKLOADS["buckets"]
    sizes = inputs.bucket_sizes(wk["ntensors"])
    th = inputs.bucket_tensors(wk["n"], sizes)
    # each rank's gradients in one region, regions a power of two apart (as a
    # gradient arena sits at the same address on every real GPU)
    arena, dev = rar.rank_tensors(wk["n"], sizes, torch.bfloat16, "cuda:0")
    for r in range(wk["n"]):
        for t, x in zip(th[r], dev[r]):
            x.copy_(torch.from_numpy(t.view(np.int16)).view(torch.bfloat16))
    del th
    ws = torch.empty(rar.bucketed_workspace_bytes(sizes, wk["n"], rar.BF16, wk["cap_bytes"]), dtype=torch.uint8,
                     device="cuda:0")
    # the gradient tensors are fixed, so the plan (pointer table and fold
    # descriptors) is prepared once, as a training loop would, and each timed
    # step launches the fold alone
    step = rar.BucketedAllreduce(dev, wk["cap_bytes"], ws)
    ms, k, _ = time_leg(lambda d: step(), [dev, dev], 1, min(steps, 5))
    S3 = sum(sizes) * 2
    nb, _ = rar.bucket_plan(sizes, rar.BF16, wk["cap_bytes"])
    out["buckets_bf16_allreduce"] = {"ms": round(ms, 4), "busbw_GBs": round(busbw(S3, wk["n"], ms), 1),
                                     "buckets": nb, "elements_per_rank": sum(sizes),
                                     "frac_of_roofline_fold_only_bytes": round(2 * wk["n"] * S3 / (k * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                                     "traffic": counter_traffic("bucket_fold_bf16_n16",
                                                                COUNTER_KERNELS["bucket_fold_bf16_n16"]["sources"])}
    del dev, arena, ws, step
    torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        import oracle
        k = int(np.searchsorted(np.cumsum(sizes), 32 << 20))  # the first tensors, up to 32M elements
        sub = sizes[:k]
        log(f"[bench] bucketed leg: oracle on the first {k} tensors")
        th_s = inputs.bucket_tensors(wk["n"], sub)
        dt, _, core = oracle_runs(lambda: th_s, lambda a: oracle.bucketed_allreduce(a, wk["cap_bytes"],
                                                                                   dt=oracle.BF16), 1)
        del th_s
        out["buckets_bf16_allreduce"]["cpu_baseline"] = {
            "value": round(busbw(sum(sub) * 2, wk["n"], dt * 1e3), 5), "unit": "GB/s", "cores": 1,
            "kind": "oracle",
            "sample": f"the workload's first {k} tensors ({sum(sub)} bf16 elements per rank, N={wk['n']}, "
                      f"same draws), one single-thread run ({dt:.1f} s) pinned to host core {core}"}
    # [P2] exercise: ring vs tree wall-clock on 4 ranks at 1 KB, 1 MB and 16 MB
    rvt = {}
    for nbytes in (1 << 10, 1 << 20, 16 << 20):
        cnt = nbytes // 4
        xf = inputs.gradient_like(4, cnt, salt=nbytes)
        pristine = [torch.from_numpy(x).to("cuda:0") for x in xf]
        sets = make_sets(pristine, 1 + steps)
        row = {}
        for nm, fn in (("ring_stepwise", lambda b: rar.ring_allreduce_ex(b, rar.ALGO_STEPWISE)),
                       ("tree_stepwise", lambda b: rar.tree_allreduce_ex(b, rar.ALGO_STEPWISE)),
                       ("ring_fused", lambda b: rar.ring_allreduce(b)),
                       ("tree_fused", lambda b: rar.tree_allreduce(b))):
            ms, k, _ = time_leg(fn, sets, 2, steps)
            row[nm + "_us"] = round(ms * 1e3, 2)
        rvt[f"{nbytes}B"] = row
        del sets, pristine
    out["ring_vs_tree_4ranks_fp32"] = rvt
    # ring_int: N=4, 1M integer-valued fp32 per rank (32 MiB moved per call), the
    # exact-sum parity case; small enough that the host's submission of a call
    # (binding, checks, launch) takes longer than the GPU's work.  Eager: calls
    # back to back as the host issues them.  Queued: the same calls enqueued
    # behind a GPU spin of about 2 ms, so they run back to back on the GPU and
    # the events give the GPU time per call.
    wi = inputs.WORKLOADS["ring_int"]
    xi = inputs.integers(wi["n"], wi["count"])
    pristine = [torch.from_numpy(x).to("cuda:0") for x in xi]
    sets = make_sets(pristine, 1 + 24)
    Si = wi["count"] * 4
    tl = time_leg(lambda b: rar.ring_allreduce(b), sets, 4, 24)
    stream = torch.cuda.current_stream()
    qs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(24)]
    torch.cuda.synchronize()
    torch.cuda._sleep(5_000_000)
    for i, (a, b) in enumerate(qs):
        a.record(stream)
        rar.ring_allreduce(sets[1 + i % 24])
        b.record(stream)
    torch.cuda.synchronize()
    qev = sorted(a.elapsed_time(b) for a, b in qs)
    qmed = qev[len(qev) // 2]
    out["ring_int_fp32_4x1M_fused"] = {
        "eager_us_per_call": round(tl[0] * 1e3, 2), "eager_event_us_median": round(tl.median_ms * 1e3, 2),
        "queued_event_us_median": round(qmed * 1e3, 2), "queued_event_us_min": round(qev[0] * 1e3, 2),
        "frac_of_roofline_queued": round(2 * wi["n"] * Si / (qmed * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    del sets, pristine
    torch.cuda.empty_cache()
    for name, fn, cnt in (("fp32_broadcast_fused", lambda b: rar.broadcast(b, 0), w5["bcast_count"]),
                          ("fp32_allgather_fused", lambda b: rar.allgather(b), w5["ag_shard"] * 8)):
        xf = inputs.filler(8, cnt)
        pristine = [torch.from_numpy(x).to("cuda:0") for x in xf]
        sets = make_sets(pristine, 1 + steps)
        ms, k, _ = time_leg(fn, sets, 2, steps)
        Sx = cnt * 4
        moved = 8 * Sx  # broadcast: read S once, write 7 S; allgather: read S (all shards), write 7 S
        bus = Sx / (ms * 1e-3) / 1e9 if "broadcast" in name else Sx * 7 / 8 / (ms * 1e-3) / 1e9
        out[name] = {"ms": round(ms, 4), "busbw_GBs": round(bus, 1),
                     "frac_of_roofline": round(moved / (k * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
        del sets, pristine
        torch.cuda.empty_cache()
    return out


def counters_run(reps=3):
    """Short launch sequence for hardware-counter passes: a plain copy of known
    size (broadcast over 2 ranks of 256 MiB fp32: 256 MiB read, 256 MiB
    written) that validates the counters, then the fused folds (fp32, BFP-8,
    BFP-8 with error feedback), the rank hash, the bucketed fold, the staged
    and pipelined compressed schedules."""
    import torch

    import ring_all_reduce_scatter_amd as rar
    from ring_all_reduce_scatter_amd import inputs

    cal = [torch.full((64 << 20,), float(r + 1), device="cuda:0") for r in range(2)]
    for _ in range(reps):
        rar.broadcast(cal, 0)
    del cal
    w = inputs.WORKLOADS["ring_grad"]
    bufs = [torch.from_numpy(x).to("cuda:0") for x in inputs.gradient_like(w["n"], w["count"])]
    for _ in range(reps):
        rar.ring_allreduce(bufs)
    del bufs
    wb = inputs.WORKLOADS["bfp8"]
    bufs = [torch.from_numpy(x).to("cuda:0") for x in inputs.block_scaled(wb["n"], wb["count"])]
    cfg = rar.compress_cfg(unit_bytes=wb["unit_bytes"])
    ws = torch.empty(rar.compressed_workspace_bytes(wb["n"], wb["count"], rar.F16, cfg), dtype=torch.uint8,
                     device="cuda:0")
    for _ in range(reps):
        rar.ring_allreduce_compressed(bufs, cfg, ws)
    state = [torch.zeros(wb["count"], dtype=torch.float32, device="cuda:0") for _ in range(wb["n"])]
    for _ in range(reps):
        rar.ring_allreduce_compressed_state(bufs, state, rar.FEEDBACK_ERROR, cfg, ws)
    del state, bufs
    w = inputs.WORKLOADS["ring_grad"]
    bufs = [torch.from_numpy(x).to("cuda:0") for x in inputs.gradient_like(w["n"], w["count"])]
    hws = torch.empty(rar.HASH_WORKSPACE_BYTES, dtype=torch.uint8, device="cuda:0")
    for _ in range(reps):
        rar.rank_hashes(bufs, hws)
    del bufs, hws
    # zero-copy bucketed allreduce (values do not change the bytes moved)
    wk = inputs.WORKLOADS["buckets"]
    sizes = inputs.bucket_sizes(wk["ntensors"])
    arena, dev = rar.rank_tensors(wk["n"], sizes, torch.bfloat16, "cuda:0")
    arena.normal_(0.0, 1e-3)
    ws = torch.empty(rar.bucketed_workspace_bytes(sizes, wk["n"], rar.BF16, wk["cap_bytes"]), dtype=torch.uint8,
                     device="cuda:0")
    step = rar.BucketedAllreduce(dev, wk["cap_bytes"], ws)
    for _ in range(reps):
        step()
    torch.cuda.synchronize()
    del arena, dev, ws, step
    log("[bench] counters run: folds, hash and buckets done")
    # the staged BFP-8 pipeline (its bytes do not depend on the values)
    wb = inputs.WORKLOADS["bfp8"]
    big = torch.empty(wb["n"] * wb["count"], dtype=torch.float16, device="cuda:0").normal_(0.0, 1e-3)
    bufs = [big[r * wb["count"]:(r + 1) * wb["count"]] for r in range(wb["n"])]
    cfg = rar.compress_cfg(unit_bytes=wb["unit_bytes"], schedule=rar.SCHED_STAGED)
    ws = torch.empty(rar.compressed_workspace_bytes(wb["n"], wb["count"], rar.F16, cfg), dtype=torch.uint8,
                     device="cuda:0")
    for _ in range(PIPELINE_COUNTERS["bfp8_allreduce_staged"]["calls"]):
        rar.ring_allreduce_compressed(bufs, cfg, ws)
    torch.cuda.synchronize()
    del big, bufs, ws
    log("[bench] counters run: staged BFP-8 done")
    # the staged sparse + BFP-4 pipeline on the workload's own zero pattern,
    # restored before every call (torch copies, not counted)
    w5 = inputs.WORKLOADS["sparse_bfp4"]
    pristine = [torch.from_numpy(x).to("cuda:0") for x in inputs.sparse_mix(w5["n"], w5["count"])]
    bufs = [p.clone() for p in pristine]
    cfg = rar.compress_cfg(method=rar.COMP_SPARSE_AUTO, mbits=w5["mbits"], unit_bytes=w5["unit_bytes"],
                           sparsity_threshold=w5["theta"], schedule=rar.SCHED_STAGED)
    ws = torch.empty(rar.compressed_workspace_bytes(w5["n"], w5["count"], rar.F16, cfg), dtype=torch.uint8,
                     device="cuda:0")
    for _ in range(PIPELINE_COUNTERS["sparse_bfp4_allreduce_staged"]["calls"]):
        for b, p in zip(bufs, pristine):
            b.copy_(p)
        rar.ring_allreduce_compressed(bufs, cfg, ws)
    torch.cuda.synchronize()
    del ws
    log("[bench] counters run: staged sparse done")
    # the same workload through the pipelined single-launch schedule
    cfg = rar.compress_cfg(method=rar.COMP_SPARSE_AUTO, mbits=w5["mbits"], unit_bytes=w5["unit_bytes"],
                           sparsity_threshold=w5["theta"], schedule=rar.SCHED_PIPELINED)
    ws = torch.empty(rar.compressed_workspace_bytes(w5["n"], w5["count"], rar.F16, cfg), dtype=torch.uint8,
                     device="cuda:0")
    for _ in range(PIPELINE_COUNTERS["sparse_bfp4_allreduce_pipelined"]["calls"]):
        for b, p in zip(bufs, pristine):
            b.copy_(p)
        rar.ring_allreduce_compressed(bufs, cfg, ws)
    torch.cuda.synchronize()
    del ws, bufs, pristine
    # the pipelined BFP-8 schedule on the bfp8 workload (4 MiB units)
    wb = inputs.WORKLOADS["bfp8"]
    bufs = [torch.from_numpy(x).to("cuda:0") for x in inputs.block_scaled(wb["n"], wb["count"])]
    cfg = rar.compress_cfg(unit_bytes=wb["unit_bytes"], schedule=rar.SCHED_PIPELINED)
    ws = torch.empty(rar.compressed_workspace_bytes(wb["n"], wb["count"], rar.F16, cfg), dtype=torch.uint8,
                     device="cuda:0")
    for _ in range(reps):
        rar.ring_allreduce_compressed(bufs, cfg, ws)
    torch.cuda.synchronize()
    log("[bench] counters run done")


def write_jsonl(path, line, f):
    """Per-leg records for the byte-counter log ([P2] exercise: per-rank byte
    counters written as JSON lines): the headline leg with every rank's
    logical bytes, the BFP-8 leg with its wire bytes, one record per extra leg."""
    stamp = time.strftime("%Y-%m-%dT%H:%M:%S")
    recs = [{"time": stamp, "leg": "fp32_allreduce_fused", "workload": line["config"]["workload"],
             "ms_per_step": line["ms_per_step"], "kernel_ms": line["kernel_ms"], "busbw_rank_GBs": line["value"],
             "roofline": line["roofline"], "sent_bytes_per_rank": f["bytes_per_rank"]["sent"],
             "recv_bytes_per_rank": f["bytes_per_rank"]["recv"]}]
    if "bfp8" in line:
        b = line["bfp8"]
        recs.append({"time": stamp, "leg": "bfp8_allreduce_fused", "workload": b["config"]["workload"],
                     "ms_per_step": b["ms_per_step"], "busbw_rank_GBs": b["value"], "roofline": b["roofline"],
                     "wire_bytes_rank0": b["wire_bytes_per_rank"]})
    for k, v in line.get("extra", {}).items():
        recs.append({"time": stamp, "leg": k, **v})
    with open(path, "a") as fh:
        for r in recs:
            fh.write(json.dumps(r) + "\n")


def _counter_values(path, counter, match):
    import csv
    vals = []
    with open(path, newline="") as f:
        for row in csv.DictReader(f):
            if row["Counter_Name"] == counter and match in row["Kernel_Name"]:
                vals.append(float(row["Counter_Value"]))
    return vals


def ingest_counters(csv_path):
    """Turn the rocprofv3 counter pass over `bench.py --counters` into
    profiles/counters.json: HBM bytes read = 32 x TCC_EA0_RDREQ_DRAM_32B and
    written = 32 x TCC_EA0_WRREQ_WRITE_DRAM_32B per dispatch (median over a
    kernel's dispatches), no scale factor.  The copy of known size is
    reported as a check of the counters."""
    import statistics
    rd, wr, r128, bub = PMC_COUNTERS

    def per_kernel(match):
        r = _counter_values(csv_path, rd, match)
        w = _counter_values(csv_path, wr, match)
        q = _counter_values(csv_path, r128, match)
        b = _counter_values(csv_path, bub, match)
        return r, w, q, b

    r, w, q, b = per_kernel(CALIBRATION["match"])
    cr, cw = 32 * statistics.median(r), 32 * statistics.median(w)
    out = {"_method": {
        "read_bytes": "32 x " + rd, "write_bytes": "32 x " + wr, "commands": PMC_COMMANDS,
        "check_copy": {"kernel": "copy_jobs_kernel (broadcast over 2 ranks, 256 MiB fp32)",
                       "bytes_each_way": CALIBRATION["bytes"], "read_bytes_measured": int(cr),
                       "write_bytes_measured": int(cw), "read_ratio": round(cr / CALIBRATION["bytes"], 5),
                       "write_ratio": round(cw / CALIBRATION["bytes"], 5),
                       "rdreq_128B": statistics.median(q), "tcc_bubble": statistics.median(b)}}}
    rows = [f"| copy check: `copy_jobs_kernel` 256 MiB each way | {len(r)} | {int(cr):,} | {int(cw):,} | "
            f"{int(cr + cw):,} | {2 * CALIBRATION['bytes']:,} | {(cr + cw) / (2 * CALIBRATION['bytes']):.4f} | "
            f"{statistics.median(q):,.0f} / {statistics.median(b):,.0f} |"]
    for key, k in COUNTER_KERNELS.items():
        r, w, q, b = per_kernel(k["match"])
        if not r or not w:
            continue
        rb, wb = int(32 * statistics.median(r)), int(32 * statistics.median(w))
        alg = _algorithmic(k)
        out[key] = {"kernel_match": k["match"], "workload": k["workload"], "dispatches": len(r),
                    "hbm_read_bytes_per_launch": rb, "hbm_write_bytes_per_launch": wb,
                    "hbm_bytes_per_launch": rb + wb, "algorithmic_bytes_per_launch": alg,
                    "rdreq_128B": statistics.median(q), "tcc_bubble": statistics.median(b),
                    "source_sha": source_sha(k["sources"]), "sources": k["sources"]}
        rows.append(f"| `{k['match']}` ({k['workload']}) | {len(r)} | {rb:,} | {wb:,} | {rb + wb:,} | {alg:,} | "
                    f"{(rb + wb) / alg:.4f} | {statistics.median(q):,.0f} / {statistics.median(b):,.0f} |")
    pipes = {}
    for key, pdef in PIPELINE_COUNTERS.items():
        rs = [v for m in pdef["matches"] for v in _counter_values(csv_path, rd, m)]
        ws_ = [v for m in pdef["matches"] for v in _counter_values(csv_path, wr, m)]
        if not rs:
            continue
        rb, wb = int(32 * sum(rs) / pdef["calls"]), int(32 * sum(ws_) / pdef["calls"])
        pipes[key] = {"workload": pdef["workload"], "kernels": pdef["matches"], "calls": pdef["calls"],
                      "dispatches": len(rs), "hbm_read_bytes_per_call": rb, "hbm_write_bytes_per_call": wb,
                      "hbm_bytes_per_call": rb + wb, "source_sha": source_sha(pdef["sources"]),
                      "sources": pdef["sources"]}
        rows.append(f"| {pdef['workload']} (all {len(rs)} dispatches of {pdef['calls']} calls, per call) | "
                    f"{len(rs)} | {rb:,} | {wb:,} | {rb + wb:,} | - | - | - |")
    out["pipelines"] = pipes
    with open(os.path.join(ROOT, "profiles", "counters.json"), "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print("| kernel (workload) | dispatches | HBM read bytes | HBM write bytes | HBM bytes | algorithmic bytes | "
          "ratio | 128-byte read requests / TCC_BUBBLE |")
    print("|---|---|---|---|---|---|---|---|")
    print("\n".join(rows))


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--max-sets", type=int, default=24, help="device input sets per leg (2 GiB each)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--skip-bfp8", action="store_true")
    ap.add_argument("--extra", action="store_true", help="also time stepwise, staged and other collectives")
    ap.add_argument("--counters", action="store_true",
                    help="only run the short launch sequence used for rocprofv3 --pmc passes")
    ap.add_argument("--jsonl", metavar="PATH",
                    help="also append one JSON record per leg (timing, bandwidth, roofline, per-rank bytes)")
    ap.add_argument("--ingest-counters", metavar="PMC_CSV",
                    help="(no GPU) write profiles/counters.json from the rocprofv3 --pmc pass over --counters")
    args = ap.parse_args()
    if args.ingest_counters:
        ingest_counters(args.ingest_counters)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: the N simulated ranks share one MI355X's HBM, so --gpus "
              f"{args.gpus} is not supported", file=sys.stderr)
        sys.exit(2)
    if args.steps < 1:
        print("--steps must be >= 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import ring_all_reduce_scatter_amd as rar
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    rar.lib()
    if args.counters:
        counters_run()
        return

    f = fp32_leg(args)
    line = {
        "metric": METRIC,
        "value": round(f["busbw"], 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(f["ms"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded N(0,1e-3) gradients, 1% outliers x100)",
        "config": {"workload": f"ring allreduce, N={f['n']} simulated ranks on one GPU, T={f['count']} fp32 per rank "
                               f"(256 MiB), fused schedule", "n_ranks": f["n"], "count_per_rank": f["count"],
                   "schedule": "fused"},
        "busbw_aggregate_GBs": round(f["busbw"] * f["n"], 1),
        "pct_hbm_peak": round(100 * f["roofline"]["frac"], 2),
        "kernel_ms": round(f["kern_ms"], 4),
        "kernel_ms_median": round(f["kern_median_ms"], 4),
        "kernel_ms_min": round(f["kern_min_ms"], 4),
        "roofline": f["roofline"],
        "cpu_baseline": f["cpu_baseline"],
        "parity": f["parity_first_timed_output"],
        "bytes_per_rank_sent": f["bytes_per_rank"]["sent"][0],
    }
    cp = copy_peak()
    line["copy_peak"] = cp
    line["roofline"]["frac_of_copy_peak"] = round(line["roofline"]["achieved"] / cp["value"], 4)
    if not args.skip_bfp8:
        b = bfp8_leg(args)
        b["roofline"]["frac_of_copy_peak"] = round(b["roofline"]["achieved"] / cp["value"], 4)
        line["bfp8_pipelined"] = {"metric": b["metric"], "config": {**b["config"], "schedule": "pipelined"},
                                  **b.pop("pipelined")}
        line["bfp8"] = b
        line["sparse_bfp4"] = sparse_leg(args)
    if args.extra:
        line["extra"] = extra_legs(args)
    if args.jsonl:
        write_jsonl(args.jsonl, line, f)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
