/*
 * rar.h -- C-ABI of the MI355X ring all-reduce library (librar.so).
 *
 * N simulated data-parallel ranks live in one GPU's HBM: rank r's tensor is
 * the device buffer bufs[r].  Every collective works on the array of N rank
 * buffers at once and does one GPU's share of the ring's work at its real
 * shape.
 *
 * Sources (page title, section):
 *  [P2] "从零实现集合通信" (collective ops from scratch): two-pass ring
 *       allreduce (reduce-scatter then allgather over T/N chunks), the
 *       per-primitive byte table, broadcast over a log2(N) tree, allgather by
 *       N-1 rotations, reduce_scatter as the first half of the allreduce,
 *       bucketing gradients into ~25 MB buckets (production patterns).
 *  [P4] "CCCL通信压缩库：突破LLM训练通信墙的工程实践": section 2.1 layered
 *       compression (sparse value+index when sparsity exceeds a threshold;
 *       block floating point with a shared exponent per block of e.g. 128
 *       elements and 8- or 4-bit mantissas; operator-aware choice), section
 *       2.2 chunked compress -> communicate -> decompress -> reduce pipeline on
 *       separate streams synchronised by events, section 3.3 configuration
 *       (compression type, sparsity threshold, collective filter, 1-4 MB
 *       chunks), section 4.3 (compressed staging buffers cost memory),
 *       section 5 (error feedback).
 *  [P1] "Prime Intellect 发布 PCCL 分布式训练通信库", section "PCCL 模型":
 *       a shared state checked by hash and re-sent to peers off the
 *       majority; a collective cut short by a failing peer is retried on the
 *       remaining peers.
 *
 * Conventions for every call:
 *  - Device pointers are HIP device addresses, 16-byte aligned.  Host arrays
 *    (the `bufs` pointer table, counts, configs, outputs of *_traffic) are
 *    read or written during the call only and may be reused on return.
 *  - `stream` is a hipStream_t (NULL = the default stream).  Work is enqueued
 *    asynchronously and is stream-ordered: buffers must stay alive until the
 *    stream has executed it.  The few calls that return device results to
 *    the host (byte counters of the compressed calls, hashes, the
 *    fault-tolerant ring) say so and synchronise the stream; every other
 *    call can be captured in a HIP graph.  The library allocates no device memory; where
 *    scratch is needed the caller passes a workspace.
 *  - Errors in the arguments are reported synchronously, before anything is
 *    enqueued, by a nonzero rar_status; nothing is modified then.  A failed
 *    kernel launch returns RAR_EHIP.  No call aborts or throws.
 *  - count == 0 and nranks == 1 are valid and leave the buffers unchanged;
 *    with count == 0 the buffer pointers are not inspected (NULL is fine).
 *  - Element types: RAR_F32 (binary32), RAR_F16 (binary16), RAR_BF16
 *    (bfloat16).  The reduce op is SUM.  fp32 adds are IEEE binary32
 *    round-to-nearest-even with subnormals kept; fp16/bf16 adds widen both
 *    operands to binary32, add, and round back to nearest-even.  No FMA
 *    contraction, no reassociation.
 *  - Chunk rule: chunk c of a T-element buffer is [c*L, min((c+1)*L, T)) with
 *    L = rar_chunk_len(T, N) = roundup(ceil(T/N), 128); trailing chunks may be
 *    short or empty.  This fixes each element's summation order, so results
 *    are deterministic and identical across schedules.
 */
#ifndef RAR_H
#define RAR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define RAR_MAX_RANKS 64

typedef enum rar_status {
  RAR_OK = 0,
  RAR_EINVAL = 1,     /* bad size, rank count, root, step, block, mbits, config */
  RAR_EDTYPE = 2,     /* unknown element type */
  RAR_EALIGN = 3,     /* a device pointer is not 16-byte aligned */
  RAR_EWORKSPACE = 4, /* workspace missing or smaller than required */
  RAR_EHIP = 5,       /* the HIP runtime reported an error (launch, event, stream) */
  RAR_ENOTSUP = 6,    /* valid request that this library does not implement */
  RAR_EOVERLAP = 7,   /* two rank buffers overlap, a workspace overlaps a rank
                         buffer, two tensors of the bucketed call overlap, or a
                         buffer is NULL */
  RAR_EABORT = 8      /* fault-tolerant ring: every member failed */
} rar_status;

typedef enum rar_dtype { RAR_F32 = 0, RAR_F16 = 1, RAR_BF16 = 2 } rar_dtype;

/* Schedules.  Both give bit-identical results.
 * FUSED: one launch; each chunk's ring-ordered fold is kept in registers and
 *        stored once per rank (reads N*S, writes N*S bytes of HBM).
 * STEPWISE: one launch per ring step, every step materialised in the rank
 *        buffers exactly as the ring's sends and receives would leave them. */
typedef enum rar_algo { RAR_ALGO_FUSED = 0, RAR_ALGO_STEPWISE = 1 } rar_algo;

/* Elements per chunk for a T-element buffer split over N ranks
 * (roundup(ceil(T/N), 128)); 0 if nranks is out of range. */
size_t rar_chunk_len(size_t count, int nranks);

/* ---------------------------------------------------------------------- */
/* Uncompressed collectives ([P2] two-pass ring and byte table).           */
/* bufs: host array of nranks device pointers, each to `count` elements.  */
/* ---------------------------------------------------------------------- */

/* Ring allreduce, in place: afterwards every rank holds the same sum.
 * Chunk c's sum is the fold, in ring order, of ranks c+1, c+2, ..., c+N-1, c
 * (mod N): the order the reduce-scatter steps produce.  FUSED schedule. */
int rar_ring_allreduce(void* const* bufs, int nranks, size_t count, int dtype, void* stream);
int rar_ring_allreduce_ex(void* const* bufs, int nranks, size_t count, int dtype, int algo,
                          void* stream);

/* Reduce-scatter, in place: afterwards chunk r of rank r holds the full sum
 * of chunk r.  Other chunks are left unspecified (FUSED leaves them as they
 * were; STEPWISE leaves the ring's partial sums). */
int rar_reduce_scatter(void* const* bufs, int nranks, size_t count, int dtype, void* stream);
int rar_reduce_scatter_ex(void* const* bufs, int nranks, size_t count, int dtype, int algo,
                          void* stream);

/* Allgather, in place: each buffer holds N shards of count/N elements
 * (count must be divisible by nranks); rank r's own shard is shard r.
 * Afterwards every buffer holds all N shards.  STEPWISE = N-1 rotations. */
int rar_allgather(void* const* bufs, int nranks, size_t count, int dtype, void* stream);
int rar_allgather_ex(void* const* bufs, int nranks, size_t count, int dtype, int algo,
                     void* stream);

/* Broadcast of bufs[root] to every rank.  STEPWISE = binomial tree: in round
 * k every rank at distance < 2^k from the root sends to distance + 2^k
 * (ceil(log2 N) rounds); FUSED = one read of the root, N-1 writes. */
int rar_broadcast(void* const* bufs, int nranks, size_t count, int dtype, int root, void* stream);
int rar_broadcast_ex(void* const* bufs, int nranks, size_t count, int dtype, int root, int algo,
                     void* stream);

/* Single ring steps (the schedule's building blocks), step = 1..N-1.
 * RS step s: every rank r adds chunk (r-s-1) mod N received from rank
 * (r-1) mod N into its own copy (local + received).
 * AG step s: every rank r stores chunk (r-s) mod N received from rank
 * (r-1) mod N.  Running RS steps 1..N-1 then AG steps 1..N-1 equals
 * rar_ring_allreduce. */
int rar_rs_step(void* const* bufs, int nranks, size_t count, int dtype, int step, void* stream);
int rar_ag_step(void* const* bufs, int nranks, size_t count, int dtype, int step, void* stream);

/* ---------------------------------------------------------------------- */
/* Tree allreduce and size-based selection ([P2] ring-vs-tree table and   */
/* production patterns: the tree has depth log2 N and wins for small      */
/* messages or high-latency links; the ring wins for large ones).         */
/* ---------------------------------------------------------------------- */

/* Binomial tree rooted at rank 0: in the reduce round with distance span
 * (1, 2, 4, ...) rank rel (rel % 2span == 0, rel + span < N) adds rank
 * rel+span's buffer into its own (local + received); then the binomial
 * broadcast from rank 0.  Every rank ends with rank 0's sum, e.g. for N = 8
 * ((x0+x1)+(x2+x3))+((x4+x5)+(x6+x7)).  FUSED runs in one launch for
 * N in 2..8 and 16 (other N run the STEPWISE rounds); STEPWISE launches one
 * pairwise-add per reduce round and one copy per broadcast round.
 * Per-rank bytes: rank 0 receives and sends ceil(log2 N) * T. */
int rar_tree_allreduce(void* const* bufs, int nranks, size_t count, int dtype, void* stream);
int rar_tree_allreduce_ex(void* const* bufs, int nranks, size_t count, int dtype, int algo,
                          void* stream);

enum { RAR_ALLREDUCE_RING = 0, RAR_ALLREDUCE_TREE = 1 };
#define RAR_TREE_THRESHOLD_DEFAULT (1u << 20) /* 1 MiB per rank, the crossover [P2] quotes */

/* Tree below threshold_bytes per rank (0 = RAR_TREE_THRESHOLD_DEFAULT),
 * ring otherwise; *chosen (if not NULL) receives RAR_ALLREDUCE_RING or
 * RAR_ALLREDUCE_TREE.  The two orders round differently, so results can
 * differ in the last bits between the two sides of the threshold. */
int rar_allreduce_auto(void* const* bufs, int nranks, size_t count, int dtype,
                       size_t threshold_bytes, int* chosen, void* stream);

/* Logical bytes each rank sent and received in the last collective issued
 * by the calling host thread (uncompressed calls; the counters of the
 * compressed allreduce are read with rar_compressed_traffic).  sent/recv:
 * host arrays of at least nranks entries.  Matches [P2]'s byte table:
 * allreduce 2T(N-1)/N, reduce-scatter and allgather T(N-1)/N, broadcast T
 * received per non-root rank (bytes; exact when chunks are equal). */
int rar_last_traffic(uint64_t* sent, uint64_t* recv, int nranks);

/* ---------------------------------------------------------------------- */
/* Block floating point ([P4] section 2.1, numeric-precision layer).       */
/* A block of `block` consecutive elements (power of two, 16..512; 128 on  */
/* the pages) shares E, the biased binary32 exponent of its largest        */
/* magnitude; with e = max(E,1) - 127 each element is stored as            */
/*   q = clamp(round_half_even(x * 2^(m-2-e)), -(2^(m-1)-1), 2^(m-1)-1)    */
/* and stands for q * 2^(e+2-m).  m = mbits (2..8) counts the sign bit.    */
/* Per element |decoded - x| <= 2^-(m-1) * max|x over the block|.          */
/* Blocks holding Inf or NaN get E = 255 and decode to NaN.                */
/* Message layout: uint8 E[nblocks] zero-padded to a multiple of 16 bytes, */
/* then the mantissas: one int8 per element for m > 4, else two's-         */
/* complement nibbles (element 2j in bits 3:0, element 2j+1 in bits 7:4,   */
/* an odd tail's high nibble zero).  The last block may be partial.        */
/* ---------------------------------------------------------------------- */

/* Bytes of a message for `count` elements; 0 if block/mbits are invalid. */
size_t rar_bfp_bytes(size_t count, int block, int mbits);

/* Encode src (count elements of src_dtype) into dst (rar_bfp_bytes bytes). */
int rar_bfp_compress(const void* src, int src_dtype, size_t count, int block, int mbits, void* dst,
                     void* stream);

/* acc[i] <- acc[i] (+) decoded[i]: binary32 add of the exact decoded value,
 * rounded to acc_dtype. */
int rar_bfp_decompress_accumulate(const void* src, size_t count, int block, int mbits, void* acc,
                                  int acc_dtype, void* stream);

/* dst[i] <- decoded[i] rounded to dst_dtype. */
int rar_bfp_decompress(const void* src, size_t count, int block, int mbits, void* dst,
                       int dst_dtype, void* stream);

/* ---------------------------------------------------------------------- */
/* Compression-coupled ring allreduce ([P4] sections 2.1-2.2, 3.3, 4.3).   */
/* ---------------------------------------------------------------------- */

typedef enum rar_comp {
  RAR_COMP_NONE = 0,        /* plain ring allreduce */
  RAR_COMP_BFP = 1,         /* every message block floating point */
  RAR_COMP_SPARSE_AUTO = 2  /* per message: values + uint32 indices when
                               zeros > threshold * len, else BFP */
} rar_comp;

enum { RAR_OP_ALLREDUCE = 1u, RAR_OP_ALLGATHER = 2u, RAR_OP_BROADCAST = 4u };

typedef enum rar_sched {
  RAR_SCHED_FUSED = 0,   /* one launch, per-block hop chain in registers (BFP only) */
  RAR_SCHED_STAGED = 1,  /* messages materialised per pipeline unit; encode and
                            decode on two streams ordered by events */
  RAR_SCHED_FORWARD = 2, /* messages materialised per unit (BFP only); hop by
                            hop, every receiver decodes, adds its own copy and
                            encodes its next message in one kernel, without
                            writing the partial sum back; one launch per hop */
  RAR_SCHED_PIPELINED = 3 /* messages materialised per (hop, chunk, unit), all
                            kept in the workspace; one launch in which each
                            tile of a unit runs through the hops in ring
                            order: the sender stores its message, the
                            receiver loads it back, decodes, adds its own
                            copy and encodes the next; tiles at different
                            hops overlap.  Message h (1..N) of chunk c is
                            sent by rank (c+h) mod N; message N is the
                            owner's allgather message.  Slot of (h, c, u):
                            workspace + 1024 + (((h-1)*N + c) *
                            units_per_chunk + u) * slot, with slot the
                            unit's largest message (BFP: rar_bfp_bytes;
                            SPARSE_AUTO: 16 + BFP rounded up to 16, then
                            room for the all-non-zero sparse body, where a
                            sparse message's body starts) rounded up to
                            256.
                            SPARSE_AUTO: block 128 only (other blocks run
                            STAGED); the tiles of a unit decide its format
                            together, so one launch holds whole units on
                            the chip at once (cooperative launch); a unit
                            too large for that returns RAR_ENOTSUP before
                            anything is enqueued */
} rar_sched;

typedef struct rar_compress_cfg {
  int method;                /* rar_comp */
  int block;                 /* elements per BFP block: power of two, 16..512 */
  int mbits;                 /* mantissa bits incl. sign, 2..8 */
  float sparsity_threshold;  /* SPARSE_AUTO: sparse iff zeros > threshold * len */
  size_t unit_bytes;         /* pipeline unit, bytes of the uncompressed dtype;
                                unit_bytes/elem_size must be a multiple of block */
  unsigned collective_mask;  /* RAR_OP_* bits allowed to compress; without
                                RAR_OP_ALLREDUCE the call runs uncompressed */
  int schedule;              /* rar_sched */
} rar_compress_cfg;

/* Fill cfg with the pages' starting point: BFP, block 128, 8 bits,
 * threshold 0.5, 4 MiB units, allreduce only, fused schedule. */
void rar_compress_cfg_default(rar_compress_cfg* cfg);

/* Chunk length of the compressed ring: roundup(ceil(T/N), max(128, block)). */
size_t rar_compressed_chunk_len(size_t count, int nranks, int block);

/* Device workspace bytes the compressed allreduce needs (0 on bad args). */
size_t rar_compressed_workspace_bytes(int nranks, size_t count, int dtype,
                                      const rar_compress_cfg* cfg);

/* In-place compressed ring allreduce.  Reduce-scatter hop s: the sender
 * (rank r-1) encodes its current partial of chunk (r-s-1) mod N one unit at
 * a time, rank r decodes each message and adds it to its own copy.
 * Allgather: the owner encodes each finished unit once, the bytes travel
 * unchanged, and every rank (owner included) stores the decoded unit, so all
 * ranks end bit-identical.  Deterministic: the same inputs always give the
 * same bits, whatever the schedule.  The wire byte counters are left in the
 * workspace (see rar_compressed_traffic). */
int rar_ring_allreduce_compressed(void* const* bufs, int nranks, size_t count, int dtype,
                                  const rar_compress_cfg* cfg, void* workspace, size_t ws_bytes,
                                  void* stream);

/* Size of the library's own scratch array for the allocation-free variant
 * below: 32 MiB of device memory per GPU the library runs on, held from the
 * first such call on that GPU until the process ends. */
#define RAR_NOALLOC_SCRATCH_BYTES (32u << 20)

/* rar_ring_allreduce_compressed for callers that cannot allocate device
 * memory or pass a workspace: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc.  Same arguments and results,
 * bit for bit, as rar_ring_allreduce_compressed without the workspace: the
 * message slots and byte counters live in a file-scope device array of
 * RAR_NOALLOC_SCRATCH_BYTES in the library (its address is looked up once
 * per device on the first call there).  The call allocates nothing.
 * Returns RAR_EWORKSPACE when rar_compressed_workspace_bytes for these
 * arguments exceeds RAR_NOALLOC_SCRATCH_BYTES (the fused schedule needs
 * 1 KiB at any size; the staged and forwarding schedules hold one or two
 * messages per (rank, unit)).  Every call on a GPU shares that GPU's array
 * and leaves its contents behind, so calls that overlap in time on one GPU
 * (concurrent streams, or threads) race and give undefined results; calls
 * ordered on one stream are safe.  The byte counters it writes are not
 * readable by the caller. */
int rar_ring_allreduce_compressed_noalloc(void* const* bufs, int nranks, size_t count, int dtype,
                                          const rar_compress_cfg* cfg, void* stream);

/* Stateful compression for the fused BFP ring ([P4] section 2.1, the
 * differential encoding layer; section 5, error feedback as the remedy for
 * the accuracy loss of lossy compression). */
typedef enum rar_feedback {
  RAR_FEEDBACK_ERROR = 1,  /* encode v = p + e; keep e = v - decode(msg) */
  RAR_FEEDBACK_DELTA = 2   /* encode v = p - ref; ref += decode(msg); the
                              receiver takes ref, the sender's reconstruction */
} rar_feedback;

/* rar_ring_allreduce_compressed with per-rank state.  state[r] holds count
 * binary32 values owned by rank r (device memory, 16-byte aligned, zero
 * before the first call, kept by the caller between calls; neither the state
 * buffers nor the rank buffers may overlap).  Each rank encodes each element
 * exactly once per call: in the reduce-scatter as the sender of its partial,
 * in the allgather as the owner of its chunk, and that encode reads and
 * rewrites the rank's state element.  With error feedback the receiver takes
 * decode(msg); with delta coding it takes the sender's running
 * reconstruction ref.  In every other respect (order, rounding, message
 * bytes) the call is the fused BFP ring: with all-zero state and feedback
 * ERROR its first result equals rar_ring_allreduce_compressed's.
 * cfg must select RAR_COMP_BFP, RAR_SCHED_FUSED and include
 * RAR_OP_ALLREDUCE (else RAR_ENOTSUP); the workspace is the one
 * rar_compressed_workspace_bytes sizes for cfg, and receives the wire byte
 * counters.  With nranks == 1 nothing travels and nothing is encoded:
 * buffer and state are left as they are. */
int rar_ring_allreduce_compressed_state(void* const* bufs, void* const* state, int nranks, size_t count,
                                        int dtype, int feedback, const rar_compress_cfg* cfg,
                                        void* workspace, size_t ws_bytes, void* stream);

/* Wire bytes each rank sent and received in the last compressed allreduce
 * that used this workspace.  Synchronises `stream` first. */
int rar_compressed_traffic(const void* workspace, int nranks, uint64_t* sent, uint64_t* recv,
                           void* stream);

/* ---------------------------------------------------------------------- */
/* Shared state and fault tolerance ([P1] "Prime Intellect 发布 PCCL 分布式  */
/* 训练通信库", section "PCCL 模型": peers check a shared state by hash and  */
/* re-send it to peers off the majority; a collective interrupted by a    */
/* failing peer is retried on the peers that remain).                     */
/* ---------------------------------------------------------------------- */

/* Device workspace the hash calls need: 64 accumulators. */
#define RAR_HASH_WORKSPACE_BYTES 512

/* hashes[r] = 64-bit hash of the first nbytes bytes of bufs[r].  The bytes
 * are read as little-endian 64-bit words w_0 .. w_{W-1} (the last one
 * zero-padded); h = sum_i mix64(w_i + (i+1) * 0x9E3779B97F4A7C15) mod 2^64
 * and the hash is mix64(h xor nbytes), mix64 being the splitmix64 output
 * function.  Not cryptographic: it detects divergence, not tampering.
 * Buffers: 16-byte aligned, may overlap (they are only read).  workspace:
 * RAR_HASH_WORKSPACE_BYTES of device memory, 16-byte aligned.  Synchronises
 * `stream` to return the hashes. */
int rar_rank_hashes(void* const* bufs, int nranks, size_t nbytes, void* workspace, size_t ws_bytes,
                    uint64_t* hashes, void* stream);

/* Shared-state check and re-send.  The majority hash is the one held by the
 * most ranks (a tie goes to the hash of the lowest rank among the tied
 * ones); the lowest rank holding it sends its nbytes bytes to every rank
 * whose hash differs.  *resent = number of ranks overwritten; hashes (may be
 * NULL) receives the hashes before the re-send.  rar_last_traffic reports
 * nbytes per re-sent rank.  Buffers must not overlap.  Synchronises
 * `stream` once (the source is chosen on the host), then enqueues the
 * copies on it. */
int rar_shared_state_sync(void* const* bufs, int nranks, size_t nbytes, void* workspace, size_t ws_bytes,
                          int* resent, uint64_t* hashes, void* stream);

/* A failure injected from the host before step `step` of a pass (steps
 * 1 .. 2(M-1) of a pass over M members, reduce-scatter steps first).
 * stall_ms = 0: `rank` is gone, and the check before the step finds it at
 * once.  stall_ms > 0: `rank` stops answering for that long; see the
 * deadline of rar_ring_allreduce_ft. */
typedef struct rar_fault {
  int rank;
  int step;
  int stall_ms;
} rar_fault;

enum { RAR_FT_ALIVE = 0, RAR_FT_GONE = 1, RAR_FT_DEADLINE = 2 };

typedef struct rar_ft_report {
  int attempts;                     /* passes started (1 when no member failed) */
  int nsurvivors;                   /* members of the pass that completed */
  int survivors[RAR_MAX_RANKS];     /* their ranks, ascending */
  int dead_attempt[RAR_MAX_RANKS];  /* pass in which rank r was found failed, 0 = never */
  int dead_step[RAR_MAX_RANKS];     /* step before which it was found failed */
  int dead_reason[RAR_MAX_RANKS];   /* RAR_FT_ALIVE / _GONE / _DEADLINE */
  long long waited_ms;              /* time the scheduler spent waiting on stalled members */
  uint64_t hash[RAR_MAX_RANKS];     /* rar_rank_hashes of every rank's final buffer */
} rar_ft_report;

/* Device workspace of rar_ring_allreduce_ft: one snapshot of every rank's
 * buffer plus the hash accumulators. */
size_t rar_ft_workspace_bytes(int nranks, size_t count, int dtype);

/* Ring allreduce that survives failing members ([P1] retry on the
 * remaining peers; [P2] exercise: a receive deadline turns a stuck rank
 * into an error instead of a hang).  The ring runs step by step from the
 * host (the stepwise schedule).  Before each step the host checks the
 * members against the fault list: a fault fires the first time a pass
 * reaches its step while its rank is still a member.  A gone member is
 * found at once.  A stalled member is waited for: with deadline_ms > 0 it is
 * declared failed after deadline_ms if its stall is longer, otherwise the
 * step goes ahead once it answers; deadline_ms <= 0 waits out every stall.
 * Members are checked together, so the wait before a step is the largest
 * one its faults cause (the host thread sleeps that long).  A pass that
 * meets a failed member is abandoned: every rank's buffer is restored from
 * the snapshot taken on entry, the failed ranks leave the ring, and a new
 * pass runs over the survivors (ascending rank order, the ring closing over
 * the gaps, chunk length rar_chunk_len(count, M)).  On return the survivors
 * hold the ring allreduce of their inputs, failed ranks hold their inputs,
 * and report->hash lets the caller confirm the survivors agree.
 * rar_last_traffic counts every step that ran, abandoned ones included.
 * Returns RAR_OK when a pass completed, RAR_EABORT when every rank failed
 * (all buffers restored).  Faults: 0 <= rank < nranks, step >= 1,
 * stall_ms >= 0, at most 256.  Synchronises `stream` (for the hashes). */
int rar_ring_allreduce_ft(void* const* bufs, int nranks, size_t count, int dtype, const rar_fault* faults,
                          int nfaults, int deadline_ms, void* workspace, size_t ws_bytes, rar_ft_report* report,
                          void* stream);

/* ---------------------------------------------------------------------- */
/* Gradient bucketing ([P2] production patterns: fuse small gradients     */
/* into ~25 MB buckets, one allreduce per bucket).                        */
/* ---------------------------------------------------------------------- */

/* Greedy plan in tensor order: a bucket is closed when the next tensor
 * would push it past cap_bytes; a tensor larger than the cap travels alone.
 * bucket_of[t] receives tensor t's bucket.  Returns the bucket count. */
size_t rar_bucket_plan(const size_t* counts, size_t ntensors, int dtype, size_t cap_bytes,
                       int* bucket_of);

/* Workspace for rar_bucketed_allreduce(_ex) and rar_bucketed_prepare (0 on
 * bad args).
 * FUSED: the launch table, 8 * (3 + nbuckets*(1 + nranks) + 4*nruns +
 * nranks*ntensors) bytes rounded up to 256, then roundup(16 + 8*nranks, 16)
 * bytes of descriptor per workgroup of the fold launch, rounded up to 256.
 * A run is the elements [a, b) of a tensor that lie in one chunk of its
 * bucket (chunk length L = roundup(ceil(P/nranks), 128) for a bucket of P
 * padded elements) and has ceil((b - floor(a/64)*64) / tile) tiles, tile =
 * 2048 elements for f32 and bf16, 4096 for f16; a bucket takes nranks
 * times the largest tile count of its chunks' runs (summed per chunk)
 * workgroups.
 * STEPWISE: nranks flat buffers of the largest padded bucket. */
size_t rar_bucketed_workspace_bytes(const size_t* counts, size_t ntensors, int nranks, int dtype,
                                    size_t cap_bytes);
size_t rar_bucketed_workspace_bytes_ex(const size_t* counts, size_t ntensors, int nranks, int dtype,
                                       size_t cap_bytes, int algo);

/* tensors: host array of nranks*ntensors device pointers, rank-major
 * (tensors[r*ntensors + t] is rank r's tensor t of counts[t] elements; the N
 * copies of a tensor must not overlap).  Buckets follow rar_bucket_plan; in a
 * bucket the tensors are laid end to end, each starting on a 16-byte
 * boundary with a zero gap after it, and the bucket is ring-allreduced with
 * the chunk rule on that flat layout.
 * FUSED (rar_bucketed_allreduce): one launch folds every bucket straight
 * from and into the tensors (no packing; workspace holds the launch table).
 * STEPWISE: each bucket is packed into flat per-rank buffers in the
 * workspace, allreduced, and unpacked.  Both give the same bits. */
int rar_bucketed_allreduce(void* const* tensors, const size_t* counts, size_t ntensors,
                           int nranks, int dtype, size_t cap_bytes, void* workspace,
                           size_t ws_bytes, void* stream);
int rar_bucketed_allreduce_ex(void* const* tensors, const size_t* counts, size_t ntensors,
                              int nranks, int dtype, size_t cap_bytes, int algo, void* workspace,
                              size_t ws_bytes, void* stream);

/* A bucketed allreduce prepared once and launched many times (a training
 * loop reduces the same gradient tensors every step).  Plain data owned by
 * the caller; filled by rar_bucketed_prepare. */
typedef struct {
  void* workspace;                /* the prepared workspace */
  uint64_t desc_offset;           /* bytes from workspace to the fold descriptors */
  uint64_t grid;                  /* fold workgroups (0: nothing to launch) */
  uint64_t ntensors;
  int nranks;
  int dtype;
  uint64_t sent[RAR_MAX_RANKS];   /* byte counters of one call (rar_last_traffic) */
  uint64_t recv[RAR_MAX_RANKS];
} rar_bucketed_plan;

/* FUSED bucketed allreduce in two parts.  rar_bucketed_prepare checks the
 * arguments as rar_bucketed_allreduce does, writes the launch table and the
 * per-workgroup descriptors (the N ranks' addresses of each tile) into the
 * workspace with work enqueued on `stream`, and fills *plan; the tensors'
 * values are not read.  rar_bucketed_launch enqueues the fold alone: every
 * bucket allreduced in place, the same bits as rar_bucketed_allreduce, and
 * rar_last_traffic reports the plan's byte counters.  Between the two, and
 * for as long as the plan is launched, the tensors must keep their
 * addresses and sizes and nothing may write the workspace; launches on a
 * stream other than the preparing one must be ordered after the
 * preparation by the caller.  RAR_EINVAL for a NULL plan or one whose
 * fields are out of range. */
int rar_bucketed_prepare(void* const* tensors, const size_t* counts, size_t ntensors, int nranks,
                         int dtype, size_t cap_bytes, void* workspace, size_t ws_bytes,
                         rar_bucketed_plan* plan, void* stream);
int rar_bucketed_launch(const rar_bucketed_plan* plan, void* stream);

/* ---------------------------------------------------------------------- */

/* Static description of a status code. */
const char* rar_status_string(int status);

/* Library version string. */
const char* rar_version(void);

#ifdef __cplusplus
}
#endif

#endif /* RAR_H */
