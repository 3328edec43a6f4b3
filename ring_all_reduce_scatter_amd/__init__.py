"""MI355X ring all-reduce family: Python binding over the C-ABI library librar.so.

Importing the package does not load the library; the first call does, and
raises RuntimeError if the library has not been built.
"""
from ._binding import (  # noqa: F401
    ALGO_FUSED, ALGO_STEPWISE, ALLREDUCE_RING, ALLREDUCE_TREE, TREE_THRESHOLD_DEFAULT, allreduce_auto,
    tree_allreduce, tree_allreduce_ex, BF16, COMP_BFP, COMP_NONE, COMP_SPARSE_AUTO, F16, F32, MAX_RANKS,
    OP_ALLGATHER, OP_ALLREDUCE, OP_BROADCAST, SCHED_FUSED, SCHED_STAGED, SCHED_FORWARD, SCHED_PIPELINED, CompressCfg, RarError, ag_step,
    allgather, allgather_ex, bfp_bytes, bfp_compress, bfp_decompress, bfp_decompress_accumulate, broadcast,
    broadcast_ex, bucket_plan, bucketed_allreduce, bucketed_workspace_bytes, chunk_len, compress_cfg,
    compress_cfg_default, compressed_chunk_len, compressed_traffic, compressed_workspace_bytes, dtype_code,
    last_traffic, lib, reduce_scatter, reduce_scatter_ex, ring_allreduce, ring_allreduce_compressed,
    ring_allreduce_ex, rs_step, status_string, version, FEEDBACK_DELTA, FEEDBACK_ERROR,
    ring_allreduce_compressed_state, EABORT, HASH_WORKSPACE_BYTES, Fault, FtReport, ft_workspace_bytes,
    rank_hashes, ring_allreduce_ft, shared_state_sync, BucketedAllreduce, rank_tensors, TRAFFIC_BYTES,
    ring_allreduce_compressed_noalloc, NOALLOC_SCRATCH_BYTES,
)
