"""Buffers past the 32-bit limits: more than 2^31 elements and more than
4 GiB per rank, so every element index and byte offset of the kernels needs
64 bits.  Inputs are integer-valued (filled on the device from a closed
form), so the allreduce must equal the exact sum whatever the order; the
BFP ring with 8-bit mantissas is exact on them too (every partial sum of two
ranks is an integer below 2^5 in magnitude, and the block step is at most
2^(4-6) = 1/4).  The rank hash of an 8 GiB buffer is compared with the oracle's."""
import numpy as np
import pytest
import torch

import oracle
import ring_all_reduce_scatter_amd as rar

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

PIECE = 1 << 28


def _fill(buf, rank):
    """x_r[i] = ((7 i + 3 r) mod 17) - 8, written piece by piece."""
    n = buf.numel()
    for lo in range(0, n, PIECE):
        hi = min(n, lo + PIECE)
        i = torch.arange(lo, hi, dtype=torch.int64, device=buf.device)
        buf[lo:hi] = ((7 * i + 3 * rank) % 17 - 8).to(buf.dtype)
        del i


def _check_exact_sum(bufs):
    n = len(bufs)
    count = bufs[0].numel()
    for lo in range(0, count, PIECE):
        hi = min(count, lo + PIECE)
        i = torch.arange(lo, hi, dtype=torch.int64, device=bufs[0].device)
        want = sum((7 * i + 3 * r) % 17 - 8 for r in range(n)).to(bufs[0].dtype)
        for r in range(n):
            if not torch.equal(bufs[r][lo:hi], want):
                bad = torch.nonzero(bufs[r][lo:hi] != want)[0].item() + lo
                raise AssertionError(f"rank {r} element {bad}: {bufs[r][bad].item()} != exact sum")
        del i, want


@pytest.fixture(scope="module")
def big_f32():
    count = (1 << 31) + (1 << 20) + 77  # 8.004 GiB per rank
    bufs = [torch.empty(count, dtype=torch.float32, device="cuda:0") for _ in range(2)]
    yield bufs
    del bufs
    torch.cuda.empty_cache()


@pytest.mark.parametrize("algo", [rar.ALGO_FUSED, rar.ALGO_STEPWISE])
def test_allreduce_beyond_4gib_is_exact(big_f32, algo):
    for r, b in enumerate(big_f32):
        _fill(b, r)
    rar.ring_allreduce_ex(big_f32, algo)
    _check_exact_sum(big_f32)
    S = big_f32[0].numel() * 4  # with two ranks each sends one chunk per pass: S bytes in all
    assert rar.last_traffic(2) == ([S, S], [S, S])


def test_rank_hash_beyond_4gib_matches_oracle(big_f32):
    for r, b in enumerate(big_f32):
        _fill(b, r)
    ws = torch.empty(rar.HASH_WORKSPACE_BYTES, dtype=torch.uint8, device="cuda:0")
    h = rar.rank_hashes(big_f32, ws)
    assert h[0] != h[1]
    host = big_f32[1].cpu().numpy()
    assert h[1] == oracle.hash64(host)


def test_bfp_ring_beyond_2g_elements_is_exact():
    count = (1 << 31) + 4099  # fp16: element indices past 2^31, byte offsets past 4 GiB
    bufs = [torch.empty(count, dtype=torch.float16, device="cuda:0") for _ in range(2)]
    for r, b in enumerate(bufs):
        _fill(b, r)
    cfg = rar.compress_cfg(mbits=8)
    ws = torch.empty(rar.compressed_workspace_bytes(2, count, rar.F16, cfg), dtype=torch.uint8, device="cuda:0")
    rar.ring_allreduce_compressed(bufs, cfg, ws)
    _check_exact_sum(bufs)
    del bufs
    torch.cuda.empty_cache()
