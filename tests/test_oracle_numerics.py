"""Pins for the oracle's number formats and its accumulate (CPU only).

The oracle writes its binary16 / bfloat16 conversions from the IEEE-754
format definition.  Here they are pinned to library routines that are
independent of it: numpy's float16 conversions and torch's bfloat16
conversions, both round-to-nearest-even.  The fp16/bf16 accumulate
(widen to binary32, add, round back) is pinned to the correctly rounded
sum computed in binary64 and rounded once by numpy / torch.
"""
import numpy as np
import pytest
import torch


def _all_f16_codes():
    return np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)


def test_f16_decode_all_codes(orc):
    codes = _all_f16_codes()
    got = orc.convert(codes.view(np.float16), orc.F16, orc.F32)
    ref = codes.view(np.float16).astype(np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def _f32_probe_values(seed=7, n=400_000):
    g = np.random.default_rng(seed)
    f16_vals = _all_f16_codes().view(np.float16).astype(np.float64)
    f16_vals = f16_vals[np.isfinite(f16_vals)]
    srt = np.unique(f16_vals)
    mids = (srt[:-1] + srt[1:]) / 2.0  # exact ties between neighbours
    mids32 = mids.astype(np.float32)
    up = np.nextafter(mids32, np.float32(np.inf))
    dn = np.nextafter(mids32, np.float32(-np.inf))
    rnd_bits = g.integers(0, 1 << 32, size=n, dtype=np.uint64).astype(np.uint32).view(np.float32)
    rnd_small = (g.standard_normal(n) * np.exp2(g.uniform(-30, 17, n))).astype(np.float32)
    specials = np.array([0.0, -0.0, np.inf, -np.inf, 65504.0, 65519.996, 65520.0, 65536.0,
                         2.0 ** -24, 2.0 ** -25, 3 * 2.0 ** -26, 2.0 ** -14, 2.0 ** -15,
                         1e-30, -1e-30, 3.4e38], dtype=np.float32)
    return np.concatenate([f16_vals.astype(np.float32), mids32, up, dn, rnd_bits, rnd_small, specials])


def test_f16_encode_matches_numpy(orc):
    x = _f32_probe_values()
    got = orc.convert(x, orc.F32, orc.F16)
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint16), ref[~nan].view(np.uint16))


def test_bf16_decode_all_codes(orc):
    codes = _all_f16_codes()
    got = orc.convert(codes, orc.BF16, orc.F32)
    ref = torch.from_numpy(codes.view(np.int16).copy()).view(torch.bfloat16).float().numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def test_bf16_encode_matches_torch(orc):
    g = np.random.default_rng(11)
    bf = torch.from_numpy(_all_f16_codes().view(np.int16).copy()).view(torch.bfloat16).float().numpy()
    bf = bf[np.isfinite(bf)].astype(np.float64)
    srt = np.unique(bf)
    mids = ((srt[:-1] + srt[1:]) / 2.0).astype(np.float32)  # bf16 ties are exact in binary32
    x = np.concatenate([
        mids, np.nextafter(mids, np.float32(np.inf)), np.nextafter(mids, np.float32(-np.inf)),
        g.integers(0, 1 << 32, size=400_000, dtype=np.uint64).astype(np.uint32).view(np.float32),
        np.array([0.0, -0.0, np.inf, -np.inf, 3.3895314e38, 3.4028235e38, 1e-40, -1e-45], dtype=np.float32),
    ])
    got = orc.convert(x, orc.F32, orc.BF16)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    nan = np.isnan(x)
    assert np.array_equal(got[~nan], ref[~nan])
    # NaN stays NaN
    back = orc.convert(got[nan], orc.BF16, orc.F32)
    assert np.all(np.isnan(back))


def _pairs_via_ring(orc, a, b, dt):
    """a (+) b as the oracle's own ring computes it: with N=2 ranks every
    element is local + received exactly once."""
    bufs = [np.ascontiguousarray(a).copy(), np.ascontiguousarray(b).copy()]
    orc.ring_allreduce(bufs, dt=dt)
    assert np.array_equal(bufs[0].view(np.uint16), bufs[1].view(np.uint16))
    return bufs[0]


def test_f16_accumulate_is_correctly_rounded_add(orc):
    """widen-add-narrow in binary32 == one rounding of the exact sum (the
    double-rounding result for 24 >= 2*11+2), including subnormals."""
    g = np.random.default_rng(3)
    n = 1 << 19
    codes_a = g.integers(0, 1 << 16, size=n, dtype=np.uint32).astype(np.uint16)
    codes_b = g.integers(0, 1 << 16, size=n, dtype=np.uint32).astype(np.uint16)
    # plus near-cancelling and same-binade pairs, where ties are common
    a2 = (g.standard_normal(n) * 4).astype(np.float16)
    b2 = (-(a2.astype(np.float32)) * (1 + g.standard_normal(n).astype(np.float32) * 1e-3)).astype(np.float16)
    a = np.concatenate([codes_a.view(np.float16), a2])
    b = np.concatenate([codes_b.view(np.float16), b2])
    fin = np.isfinite(a) & np.isfinite(b)
    a, b = a[fin], b[fin]
    got = _pairs_via_ring(orc, a, b, orc.F16)
    with np.errstate(over="ignore"):
        exact = a.astype(np.float64) + b.astype(np.float64)  # exact: fp16 pairs need < 53 bits
        ref = exact.astype(np.float16)
    nz = exact != 0
    assert np.array_equal(got[nz].view(np.uint16), ref[nz].view(np.uint16))
    assert np.all(got[~nz] == 0)


def test_f16_accumulate_exhaustive(orc):
    """Every pair of finite binary16 codes (2^32 pairs, in batches of 64 first
    operands): the oracle's accumulate equals the exact sum rounded once to
    binary16 (numpy's binary64 -> binary16 conversion, round-to-nearest-even);
    exact zeros come out as a zero of either sign.  The batches run on a
    thread pool (the oracle is plain C without global state, and ctypes and
    numpy release the GIL), about 40 s on 8 cores."""
    import os
    from concurrent.futures import ThreadPoolExecutor

    codes = _all_f16_codes()
    finite = codes[np.isfinite(codes.view(np.float16))]
    b64 = finite.view(np.float16).astype(np.float64)
    per = 64

    def batch(i):
        ac = finite[i:i + per]
        a = np.repeat(ac, finite.size)
        b = np.tile(finite, ac.size)
        got = _pairs_via_ring(orc, a.view(np.float16), b.view(np.float16), orc.F16)
        with np.errstate(over="ignore"):
            exact = (np.repeat(ac.view(np.float16).astype(np.float64), finite.size)
                     + np.tile(b64, ac.size))  # exact: binary16 pairs need < 53 bits
            ref = exact.astype(np.float16)
        nz = exact != 0
        gu, ru = got.view(np.uint16)[nz], ref.view(np.uint16)[nz]
        if not np.array_equal(gu, ru):
            k = np.flatnonzero(gu != ru)[0]
            return (f"pair {a[nz][k]:#06x} + {b[nz][k]:#06x}: got {gu[k]:#06x}, expected {ru[k]:#06x}")
        if not np.all(got[~nz].astype(np.float32) == 0):
            return f"a non-zero result for an exact zero sum in the batch from {ac[0]:#06x}"
        return None

    orc.lib()  # load once before the threads
    with ThreadPoolExecutor(max_workers=max(1, min(8, os.cpu_count() or 1))) as ex:
        errors = [e for e in ex.map(batch, range(0, finite.size, per)) if e]
    assert not errors, errors[:3]


def test_bf16_accumulate_is_correctly_rounded_add(orc):
    g = np.random.default_rng(5)
    n = 1 << 18
    ea = g.integers(-100, 100, size=n)
    # exponent gap <= 15 keeps the exact sum representable in binary32, so
    # torch's binary32 -> bfloat16 rounding is the single correct rounding
    eb = ea + g.integers(-15, 16, size=n)
    fa = (g.uniform(1, 2, n) * np.exp2(ea) * g.choice([-1, 1], n)).astype(np.float32)
    fb = (g.uniform(1, 2, n) * np.exp2(eb) * g.choice([-1, 1], n)).astype(np.float32)
    a = torch.from_numpy(fa).to(torch.bfloat16)
    b = torch.from_numpy(fb).to(torch.bfloat16)
    exact = a.double() + b.double()
    assert torch.equal(exact.float().double(), exact)
    ref = exact.float().to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    ab = a.view(torch.int16).numpy().view(np.uint16).copy()
    bb = b.view(torch.int16).numpy().view(np.uint16).copy()
    got = _pairs_via_ring(orc, ab, bb, orc.BF16)
    nz = exact.numpy() != 0
    assert np.array_equal(got[nz], ref[nz])


def test_f32_accumulate_is_ieee_add(orc):
    g = np.random.default_rng(9)
    n = 1 << 18
    a = g.integers(0, 1 << 32, size=n, dtype=np.uint64).astype(np.uint32).view(np.float32)
    b = (a * g.uniform(-2, 2, n).astype(np.float32)).astype(np.float32)
    fin = np.isfinite(a) & np.isfinite(b)
    a, b = a[fin], b[fin]
    got = _pairs_via_ring(orc, a, b, orc.F32)
    with np.errstate(over="ignore"):
        ref = (a + b).astype(np.float32)  # numpy binary32 add, RNE
    same = (got.view(np.uint32) == ref.view(np.uint32)) | (np.isnan(got) & np.isnan(ref))
    assert same.all()


def test_subnormal_f32_survives(orc):
    x = np.array([1e-45, 2e-45, -3e-44, 1.1754942e-38], dtype=np.float32)
    y = np.array([1e-45, 1e-45, 1e-45, 1e-45], dtype=np.float32)
    got = _pairs_via_ring(orc, x, y, orc.F32)
    assert np.array_equal(got, (x + y).astype(np.float32))
    assert got[0] != 0.0
