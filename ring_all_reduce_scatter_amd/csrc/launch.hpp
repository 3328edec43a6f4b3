// Host-side launchers of the gfx950 kernels (internal to librar.so).
// Every launcher enqueues asynchronously on `stream` and returns a
// hipError_t from hipGetLastError() after the launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.hpp"

namespace rar {

// -------------------------------------------------------------- launch status
// Result of the launch just enqueued on `stream`.  With RAR_DEBUG_SYNC set to
// a value other than 0 in the environment, the stream is also synchronised
// so an execution error surfaces at the call that caused it (a debugging
// aid: it serialises every call and must not be used under graph capture).
hipError_t launch_status(hipStream_t stream);

// -------------------------------------------------------------- residency control
// Streaming kernels keep most HBM efficiency with about 64 KiB of loads in
// flight per CU; at full occupancy the memory controllers see too many
// outstanding requests and throughput drops (measured on MI355X: the fp32
// N=8 fold moves 5.7 TB/s at 8 workgroups per CU, 6.1 TB/s at 1).  A launch
// caps its workgroups per CU by reserving dynamic LDS it does not use:
// residency_lds(w) is just over 1/(w+1) of the CU's LDS, so w workgroups fit
// and w+1 do not.  0 = no cap.
size_t residency_lds(int wgs_per_cu);
// Workgroups per CU for a fused fold of dtype dt over n ranks (0 = no cap).
int fold_wgs_per_cu(int dt, int n);
// Consecutive tiles of one chunk that consecutive fused-fold workgroups take
// (1 = chunk fastest), for a chunk of `tiles` tiles.
uint64_t fold_tile_group(int dt, int n, uint64_t tiles);

// -------------------------------------------------------------- ring (ring_kernels.hip)

// Fused ring fold over all chunks: chunk c of every element position gets
// the fold of ranks c+1, ..., c+N-1, c (mod N); stored to every rank
// (store_all) or to the owner c only (reduce-scatter).
hipError_t launch_ring_fold(const RankPtrs& bufs, int n, uint64_t count, uint64_t L, int dt,
                            bool store_all, hipStream_t stream);

// One reduce-scatter step s: rank r <- rank r (+) rank r-1 on chunk (r-s-1) mod N.
hipError_t launch_rs_step(const RankPtrs& bufs, int n, uint64_t count, uint64_t L, int dt, int s,
                          hipStream_t stream);

// Tree allreduce: fused (all ranks in registers, binomial order) for the
// rank counts tree_fold_supported() accepts; pairwise whole-buffer adds for
// the stepwise rounds.
struct PairJobs {
  int8_t src[kMaxRanks];
  int8_t dst[kMaxRanks];
  int npairs;
};
bool tree_fold_supported(int n);
hipError_t launch_tree_fold(const RankPtrs& bufs, int n, uint64_t count, int dt, hipStream_t stream);
hipError_t launch_pair_add(const RankPtrs& bufs, const PairJobs& pairs, uint64_t count, int dt, hipStream_t stream);

// Byte-range copies from one rank buffer to a set of rank buffers, at the
// same offset in each.  Up to kMaxRanks jobs per launch.
struct CopyJobs {
  RankPtrs ptrs;
  uint64_t lo[kMaxRanks];       // byte offset of the range
  uint64_t len[kMaxRanks];      // bytes (a multiple of 2)
  uint64_t dstmask[kMaxRanks];  // bit d set: write rank d
  int8_t src[kMaxRanks];        // source rank
  int njobs;
};
hipError_t launch_copy_jobs(const CopyJobs& jobs, hipStream_t stream);

// -------------------------------------------------------------- BFP (bfp_kernels.hip)

// One contiguous message job: `len` elements at `data` <-> message at `msg`.
struct BfpJobs {
  const char* src[kMaxRanks];  // encode: elements to encode
  char* dst[kMaxRanks];        // decode: elements to write / accumulate into
  uint8_t* msg[kMaxRanks];     // message base (exponents, then mantissas)
  uint64_t len[kMaxRanks];     // elements
  int njobs;
};

hipError_t launch_bfp_encode(const BfpJobs& jobs, int dt, int block, int mbits, hipStream_t stream);

// Forwarding hop jobs: out <- encode(local (+) decode(in)), or encode(local)
// when in is NULL; `len` elements each.
struct FwdJobs {
  const uint8_t* in[kMaxRanks];
  const char* local[kMaxRanks];
  uint8_t* out[kMaxRanks];
  uint64_t len[kMaxRanks];
  int njobs;
};
hipError_t launch_bfp_forward(const FwdJobs& jobs, int dt, int block, int mbits, hipStream_t stream);
// accumulate: dst <- dst (+) decoded; otherwise dst <- decoded.
hipError_t launch_bfp_decode(const BfpJobs& jobs, int dt, int block, int mbits, bool accumulate,
                             hipStream_t stream);
// Decode each job's message once and store it to the same element range of
// every rank in `fan` (allgather of the compressed ring).
hipError_t launch_bfp_decode_fanout(const BfpJobs& jobs, const RankPtrs& fan, int nfan,
                                    uint64_t elem_off[kMaxRanks], int dt, int block, int mbits,
                                    hipStream_t stream);

// Pipelined compressed ring, one launch: every message (hop h = 1..N of
// chunk c, unit u) is stored to slots + (((h-1)*n + c)*upc + u)*slot and
// loaded back by its receiver; hop N is the owner's allgather message, whose
// decode goes to every rank.  A workgroup carries one tile through the hops.
hipError_t launch_bfp_pipe(const RankPtrs& bufs, int n, uint64_t count, uint64_t L, uint64_t U, uint64_t upc,
                           uint64_t slot, uint8_t* slots, int dt, int block, int mbits, hipStream_t stream);

// Fused compressed ring fold: per block, the RS hop chain with an encode /
// decode per hop kept in registers, then the allgather encode / decode;
// the result is stored to every rank.
hipError_t launch_bfp_ring_fold(const RankPtrs& bufs, int n, uint64_t count, uint64_t L, int dt,
                                int block, int mbits, hipStream_t stream);

// -------------------------------------------------------------- sparse-or-BFP (sparse_kernels.hip)

// Messages of the SPARSE_AUTO compressed ring (one per pipeline unit).
struct CompJobs {
  const char* src[kMaxRanks];  // unit data to encode
  uint8_t* msg[kMaxRanks];     // message: 16-byte header + payload
  uint32_t* tiles[kMaxRanks];  // scratch: per-tile non-zero counts, then offsets
  uint64_t len[kMaxRanks];     // elements in the unit
  int8_t from[kMaxRanks];      // first sender charged in the byte counters
  int8_t hops[kMaxRanks];      // links the message crosses (1, or N-1 in the allgather)
  int njobs;
  int nranks;
};

// Tiles (2048 elements) per unit: the scratch needs 2 * this many uint32.
uint64_t comp_tiles_per_unit(uint64_t unit_elems);
// count -> plan (threshold, header, byte counters) -> write; traffic points
// at u64 sent[kMaxRanks] followed by recv[kMaxRanks] in device memory.
// counted: the per-tile non-zero counts are already in jobs.tiles (written
// by the decode that produced the data), so the count pass is skipped.
hipError_t launch_comp_encode(const CompJobs& jobs, int dt, int block, int mbits, float theta, uint64_t* traffic,
                              bool counted, hipStream_t stream);
// dst <- dst (+) decoded message (job dst / msg / len).
// Receiver side: dst <- dst (+) decode(msg), per 2048-element tile; when
// counts[j] is set, the tile's non-zero count after the add goes to
// counts[j][tile] (the count the next encode of dst needs).
struct CompAccJobs {
  uint8_t* msg[kMaxRanks];
  char* dst[kMaxRanks];
  uint64_t len[kMaxRanks];
  uint32_t* counts[kMaxRanks];
  int njobs;
};
hipError_t launch_comp_decode_acc(const CompAccJobs& jobs, int dt, int block, int mbits, hipStream_t stream);
// Pipelined SPARSE_AUTO ring in one cooperative launch (sparse_pipe_kernels.hip):
// messages of hop h = 1..N of (chunk c, unit u) at slots + (((h-1)*n + c)*upc
// + u)*slot.  flags: sparse_pipe_flag_words() words of device memory for the
// per-(hop, unit) arrival words, per-tile counts and the abort word (all
// cleared by the launch itself); traffic: u64 sent[64], recv[64] (cleared
// too).  Returns hipErrorCooperativeLaunchTooLarge, before enqueuing
// anything, when one unit's tiles cannot all be resident at once.
uint64_t sparse_pipe_tiles_per_unit(uint64_t unit_elems, int dt);
uint64_t sparse_pipe_flag_words(int n, uint64_t upc, uint64_t U, int dt);
bool sparse_pipe_fits(int n, uint64_t upc, uint64_t U, int dt, int block);
hipError_t launch_sparse_pipe(const RankPtrs& bufs, int n, uint64_t count, uint64_t L, uint64_t U, uint64_t upc,
                              uint64_t slot, uint8_t* slots, uint64_t* flags, uint64_t nflag_words,
                              uint64_t* traffic, int dt, int block, int mbits, float theta, hipStream_t stream);
// Store each decoded message to elem_off[j] of every rank in `fan`.
hipError_t launch_comp_decode_fanout(const BfpJobs& jobs, const RankPtrs& fan, int nfan, const uint64_t* elem_off,
                                     int dt, int block, int mbits, hipStream_t stream);

// -------------------------------------------------------------- buckets (bucket_kernels.hip)

// Segment copies: dst[0, bytes) <- src[0, bytes), then dst[bytes, zero_to) <- 0.
// src and dst 16-byte aligned, bytes a multiple of 2, zero_to - bytes < 16.
struct SegJobs {
  const char* src[kMaxRanks];
  char* dst[kMaxRanks];
  uint64_t bytes[kMaxRanks];
  uint64_t zero_to[kMaxRanks];
  int njobs;
};
hipError_t launch_seg_copy(const SegJobs& jobs, hipStream_t stream);

// Elements per workgroup tile of the zero-copy bucket fold.
uint64_t bucket_fold_tile_elems(int dt);
// The fold tiles each run (the elements one tensor shares with one chunk)
// from the run's first element rounded down to a multiple of kRunAlign
// elements of its tensor.
constexpr uint64_t kRunAlign = 64;
// Bytes of one fold workgroup's descriptor: 16 of header, 8 per rank,
// rounded up to 16.
uint64_t bucket_desc_stride(int n);
// Descriptors of the grid fold workgroups (bucket_desc_stride(n) bytes each
// at dev_desc), from the device table (layout in bucket_kernels.hip).
hipError_t launch_bucket_desc(const uint64_t* dev_table, void* dev_desc, int n, uint64_t ntensors, uint64_t grid,
                              int dt, hipStream_t stream);
// All buckets in one launch, in place on the tensors, from the descriptors;
// grid = total workgroups.
hipError_t launch_bucket_fold(const void* dev_desc, int n, uint64_t grid, int dt, hipStream_t stream);

// Fused compressed ring with per-rank binary32 state (feedback 1 = error
// feedback, 2 = delta coding); state.p[r] holds count floats.
hipError_t launch_bfp_ring_fold_state(const RankPtrs& bufs, const RankPtrs& state, int n, uint64_t count, uint64_t L,
                                      int dt, int block, int mbits, int feedback, hipStream_t stream);

// Writes nvals host values into device memory, stream-ordered: the values
// travel as kernel arguments (3.5 KiB per launch), so the host array may be
// reused as soon as the call returns.
hipError_t launch_fill_u64(uint64_t* dst, const uint64_t* host_vals, int nvals, hipStream_t stream);

// -------------------------------------------------------------- hash (hash_kernels.hip)

// acc[y] = sum over the 64-bit words of bufs.p[y] (y < n) of the hash's
// per-word terms (accumulators cleared first, stream-ordered).  The caller
// finishes each rank's hash as mix64(acc[y] xor nbytes).
hipError_t launch_rank_hash(const RankPtrs& bufs, int n, uint64_t nbytes, uint64_t* acc, hipStream_t stream);

// Output function of the splitmix64 generator (Steele, Lea and Flood,
// "Fast splittable pseudorandom number generators", OOPSLA 2014).
__host__ __device__ inline uint64_t hash_mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

__host__ __device__ inline uint64_t bfp_exp_bytes(uint64_t count, int block) {
  uint64_t nb = (count + (uint64_t)block - 1) / (uint64_t)block;
  return (nb + 15) / 16 * 16;
}
__host__ __device__ inline uint64_t bfp_msg_bytes(uint64_t count, int block, int mbits) {
  return bfp_exp_bytes(count, block) + (mbits > 4 ? count : (count + 1) / 2);
}

}  // namespace rar
