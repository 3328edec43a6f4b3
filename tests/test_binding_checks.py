"""The Python binding refuses buffers the kernels would overrun, before any
launch: non-contiguous views, messages or destinations too small for the
element count, hash lengths past a buffer, a workspace too small to hold the
byte counters.  CPU only: every call here must raise ValueError from the
binding's own checks, which run before a device pointer is taken (so host
tensors reach them and no GPU is needed)."""
import pytest
import torch

import ring_all_reduce_scatter_amd as rar


def _raises(fn, match):
    with pytest.raises(ValueError, match=match):
        fn()


def test_bfp_compress_checks_message_size_and_layout():
    src = torch.zeros(1000, dtype=torch.float16)
    need = rar.bfp_bytes(1000, 128, 8)
    _raises(lambda: rar.bfp_compress(src, 128, 8, torch.zeros(need - 1, dtype=torch.uint8)), "bytes")
    _raises(lambda: rar.bfp_compress(src[::2], 128, 8, torch.zeros(need, dtype=torch.uint8)), "contiguous")
    _raises(lambda: rar.bfp_compress(src, 128, 8, torch.zeros(2 * need, dtype=torch.uint8)[::2]), "contiguous")
    # big enough and contiguous: only the host-tensor check is left
    _raises(lambda: rar.bfp_compress(src, 128, 8, torch.zeros(need, dtype=torch.uint8)), "GPU tensor")


@pytest.mark.parametrize("fn", [rar.bfp_decompress, rar.bfp_decompress_accumulate])
def test_bfp_decode_checks_count_and_message(fn):
    acc = torch.zeros(4096, dtype=torch.float32)
    msg = torch.zeros(rar.bfp_bytes(4096, 128, 4), dtype=torch.uint8)
    _raises(lambda: fn(msg, 4097, 128, 4, acc), "outside")
    _raises(lambda: fn(msg, -1, 128, 4, acc), "outside")
    _raises(lambda: fn(msg[:-1], 4096, 128, 4, acc), "bytes")
    _raises(lambda: fn(msg, 4096, 128, 8, acc), "bytes")  # an 8-bit message of 4096 is larger
    _raises(lambda: fn(msg, 4096, 128, 4, torch.zeros(8192)[::2]), "contiguous")
    _raises(lambda: fn(msg, 4096, 128, 4, acc), "GPU tensor")
    _raises(lambda: fn(msg, 100, 128, 4, acc), "GPU tensor")  # a prefix of the destination is fine


def test_rank_hashes_checks_length():
    bufs = [torch.zeros(64, dtype=torch.float32) for _ in range(2)]
    ws = torch.zeros(rar.HASH_WORKSPACE_BYTES, dtype=torch.uint8)
    _raises(lambda: rar.rank_hashes(bufs, ws, nbytes=257), "outside")
    _raises(lambda: rar.rank_hashes(bufs, ws, nbytes=-1), "outside")
    _raises(lambda: rar.rank_hashes([torch.zeros(128)[::2]] * 2, ws), "contiguous")
    _raises(lambda: rar.rank_hashes(bufs, ws, nbytes=256), "GPU tensor")


def test_compressed_traffic_checks_workspace_size():
    _raises(lambda: rar.compressed_traffic(torch.zeros(rar.TRAFFIC_BYTES - 1, dtype=torch.uint8), 2), "bytes")
    _raises(lambda: rar.compressed_traffic(torch.zeros(2 * rar.TRAFFIC_BYTES, dtype=torch.uint8)[::2], 2),
            "contiguous")
    _raises(lambda: rar.compressed_traffic(torch.zeros(rar.TRAFFIC_BYTES, dtype=torch.uint8), 2), "GPU tensor")


def test_compressed_allreduce_refuses_strided_workspace():
    bufs = [torch.zeros(256, dtype=torch.float16) for _ in range(2)]
    ws = torch.zeros(4096, dtype=torch.uint8)[::2]
    _raises(lambda: rar.ring_allreduce_compressed(bufs, rar.compress_cfg(), ws), "contiguous")
