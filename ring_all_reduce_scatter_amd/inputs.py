"""Seeded synthetic inputs for the ring all-reduce workloads.

This module only draws numbers: it holds none of the collective's arithmetic,
so both the GPU library's tests and the CPU oracle can be fed from it.  Every
generator is deterministic in its seed; values are produced on the host as
numpy arrays (bfloat16 data as uint16 bit patterns).

Workloads (sizes per rank; N simulated ranks):
  ring_int      N=4,  T=1,048,576 fp32, integers uniform in {-8..8}
  ring_grad     N=8,  T=64M fp32, N(0, sigma=1e-3) with 1% of elements x100
  buckets       N=16, bf16, 200 tensors of floor(2^U(10,24)) elements,
                N(0, 1e-3), fused into 25 MiB buckets
  bfp8          N=8,  T=128M fp16, x = s_b * N(0, 1e-3) with one scale
                s_b = 2^U(-12, 0) per 128-element block shared by all ranks
  sparse_bfp4   N=8,  T=64M fp16; ranks 0..N/2-1 keep each element with
                probability 0.05 (else exact zero), ranks N/2.. dense;
                values N(0, 1e-3); plus a 16M fp32 broadcast and 16M fp32
                allgather shards
Gradients are drawn in float32 (standard normal times sigma) and rounded to
the buffer dtype with round-to-nearest-even.  A binary64 draw would be a
different random stream of the same distribution; the binary32 one halves
the host memory and time of the 8 x 128M workloads, and the buffers keep at
most 24 significant bits either way.
"""
from __future__ import annotations

import numpy as np

SEED = 1234

# workload id -> static description (sizes per rank)
WORKLOADS = {
    "ring_int": dict(wid=1, n=4, count=1 << 20, dtype="f32"),
    "ring_grad": dict(wid=2, n=8, count=64 << 20, dtype="f32"),
    "buckets": dict(wid=3, n=16, ntensors=200, dtype="bf16", cap_bytes=25 << 20),
    "bfp8": dict(wid=4, n=8, count=128 << 20, dtype="f16", block=128, mbits=8, unit_bytes=4 << 20),
    "sparse_bfp4": dict(wid=5, n=8, count=64 << 20, dtype="f16", block=128, mbits=4,
                        unit_bytes=4 << 20, theta=0.5, bcast_count=16 << 20, ag_shard=16 << 20),
}


def rng(wid: int, *stream: int) -> np.random.Generator:
    return np.random.default_rng([SEED, wid, *stream])


def _to_bf16_bits(x32: np.ndarray) -> np.ndarray:
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def cast(x32: np.ndarray, dtype: str) -> np.ndarray:
    """Round float32 draws to the buffer dtype (RNE)."""
    if dtype == "f32":
        return np.ascontiguousarray(x32, dtype=np.float32)
    if dtype == "f16":
        return x32.astype(np.float16)
    if dtype == "bf16":
        return _to_bf16_bits(x32)
    raise ValueError(dtype)


def integers(n: int, count: int, lo: int = -8, hi: int = 8, dtype: str = "f32", wid: int = 1,
             salt: int = 0) -> list[np.ndarray]:
    """Integer-valued floats uniform in {lo..hi}: every partial sum is exact."""
    out = []
    for r in range(n):
        g = rng(wid, salt, r)
        out.append(cast(g.integers(lo, hi + 1, size=count).astype(np.float32), dtype))
    return out


def gradient_like(n: int, count: int, sigma: float = 1e-3, outlier_p: float = 0.01,
                  outlier_scale: float = 100.0, dtype: str = "f32", wid: int = 2,
                  salt: int = 0) -> list[np.ndarray]:
    """N(0, sigma) with an independent Bernoulli(outlier_p) x outlier_scale per element."""
    out = []
    for r in range(n):
        g = rng(wid, salt, r)
        x = g.standard_normal(count, dtype=np.float32)
        x *= np.float32(sigma)
        if outlier_p > 0:
            m = g.random(count, dtype=np.float32) < np.float32(outlier_p)
            x[m] *= np.float32(outlier_scale)
        out.append(cast(x, dtype))
    return out


def block_scaled(n: int, count: int, block: int = 128, sigma: float = 1e-3, lo_exp: float = -12.0,
                 hi_exp: float = 0.0, dtype: str = "f16", wid: int = 4, salt: int = 0) -> list[np.ndarray]:
    """x = s_b * N(0, sigma); s_b = 2^U(lo_exp, hi_exp) per block, the same on every rank."""
    nb = (count + block - 1) // block
    scale = np.exp2(rng(wid, salt, 1_000_000).uniform(lo_exp, hi_exp, size=nb)).astype(np.float32)
    per_elem = np.repeat(scale, block)[:count]
    out = []
    for r in range(n):
        g = rng(wid, salt, r)
        x = g.standard_normal(count, dtype=np.float32)
        x *= np.float32(sigma)
        x *= per_elem
        out.append(cast(x, dtype))
    return out


def sparse_mix(n: int, count: int, sparse_ranks: int | None = None, density: float = 0.05,
               sigma: float = 1e-3, dtype: str = "f16", wid: int = 5, salt: int = 0) -> list[np.ndarray]:
    """Ranks 0..sparse_ranks-1 keep each element with probability `density`
    (others exactly +0); the remaining ranks are dense N(0, sigma)."""
    if sparse_ranks is None:
        sparse_ranks = n // 2
    out = []
    for r in range(n):
        g = rng(wid, salt, r)
        x = g.standard_normal(count, dtype=np.float32)
        x *= np.float32(sigma)
        if r < sparse_ranks:
            keep = g.random(count, dtype=np.float32) < np.float32(density)
            x = np.where(keep, x, np.float32(0.0)).astype(np.float32)
        out.append(cast(x, dtype))
    return out


def bucket_sizes(ntensors: int = 200, lo_exp: float = 10.0, hi_exp: float = 24.0, wid: int = 3,
                 salt: int = 0) -> list[int]:
    """Tensor sizes floor(2^U(lo_exp, hi_exp)) elements (log-uniform).  The
    workload's draw (salt 0) comes from default_rng([1234, 3]): 200 tensors,
    234,101,211 elements, 22 buckets of at most 25 MiB in bf16."""
    g = rng(wid) if salt == 0 else rng(wid, salt, 999)
    u = g.uniform(lo_exp, hi_exp, size=ntensors)
    return [int(v) for v in np.floor(np.exp2(u))]


def bucket_tensors(n: int, sizes: list[int], sigma: float = 1e-3, dtype: str = "bf16", wid: int = 3,
                   salt: int = 0) -> list[list[np.ndarray]]:
    """tensors[r][t]: rank r's gradient tensor t, N(0, sigma)."""
    out = []
    for r in range(n):
        g = rng(wid, salt, r)
        flat = g.standard_normal(int(sum(sizes)), dtype=np.float32)
        flat *= np.float32(sigma)
        flat = cast(flat, dtype)
        ts, off = [], 0
        for s in sizes:
            ts.append(flat[off:off + s].copy())
            off += s
        out.append(ts)
    return out


def filler(n: int, count: int, dtype: str = "f32", wid: int = 5, salt: int = 77) -> list[np.ndarray]:
    """Values for buffers that a collective is expected to overwrite, distinct
    per rank so that a missed write shows."""
    return [cast(rng(wid, salt, r).uniform(-1.0, 1.0, size=count).astype(np.float32), dtype)
            for r in range(n)]
