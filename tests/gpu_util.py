"""Helpers for the GPU parity tests: host numpy <-> device torch tensors and
bit-level comparison.  bfloat16 data is carried on the host as uint16 bits."""
import numpy as np

DT_NAMES = {"f32": 0, "f16": 1, "bf16": 2}


def torch_dtype(dt: str):
    import torch
    return {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[dt]


def to_dev(arrs, dt: str):
    import torch
    out = []
    for a in arrs:
        a = np.ascontiguousarray(a)
        if dt == "bf16":
            t = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16)
        else:
            t = torch.from_numpy(a)
        out.append(t.to("cuda:0"))
    return out


def to_host(tensors, dt: str):
    import torch
    out = []
    for t in tensors:
        c = t.detach().cpu()
        if dt == "bf16":
            out.append(c.view(torch.int16).numpy().view(np.uint16).copy())
        else:
            out.append(c.numpy().copy())
    return out


def bits(a: np.ndarray) -> np.ndarray:
    return a.view(np.uint32) if a.dtype == np.float32 else a.view(np.uint16)


def assert_bits_equal(got: np.ndarray, ref: np.ndarray, what: str = "") -> None:
    g, r = bits(got), bits(ref)
    if g.shape != r.shape:
        raise AssertionError(f"{what}: shape {g.shape} != {r.shape}")
    bad = np.flatnonzero(g != r)
    if bad.size:
        i = int(bad[0])
        raise AssertionError(f"{what}: {bad.size} of {g.size} elements differ; first at {i}: "
                             f"got {got[i]!r} (0x{int(g[i]):x}) expected {ref[i]!r} (0x{int(r[i]):x})")


def as_f64(a: np.ndarray, dt: str) -> np.ndarray:
    if dt == "bf16":
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def nan_mask(a: np.ndarray, dt: str) -> np.ndarray:
    return np.isnan(as_f64(a, dt))
