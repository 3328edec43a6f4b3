// C-ABI of librar.so: argument checking, the ring's chunk scheduler, byte
// accounting, the staged and forwarding compressed schedules, the tree,
// bucket, stateful and fault-tolerant entry points.  Kernels live in
// ring_kernels.hip, bfp_kernels.hip, sparse_kernels.hip, bucket_kernels.hip
// and hash_kernels.hip; this file only plans, checks and launches.
//
// Ring schedule (page "从零实现集合通信", two-pass ring allreduce section):
// reduce-scatter step s = 1..N-1: rank r receives chunk (r-s-1) mod N from
// rank r-1 and adds it to its copy; allgather step s: rank r receives chunk
// (r-s) mod N.  Byte table of the same page: allreduce 2T(N-1)/N per rank,
// reduce-scatter and allgather T(N-1)/N, broadcast T.
//
// Compressed pipeline (page "CCCL通信压缩库：突破LLM训练通信墙的工程实践",
// section 2.2): chunks are cut into units; unit u is compressed on one
// stream, and after an event the receiver's decompress + reduce of unit u
// runs on a second stream while unit u+1 is being compressed.
#include <algorithm>
#include <chrono>
#include <cstring>
#include <mutex>
#include <thread>
#include <vector>

#include "launch.hpp"
#include "rar.h"

using namespace rar;

namespace {

constexpr size_t kTrafficBytes = 2 * RAR_MAX_RANKS * sizeof(uint64_t);
constexpr size_t kAlign = 256;
constexpr int kMaxEvents = 64;

struct Traffic {
  int n = 0;
  uint64_t sent[RAR_MAX_RANKS] = {};
  uint64_t recv[RAR_MAX_RANKS] = {};
  void reset(int nr) {
    n = nr;
    std::memset(sent, 0, sizeof sent);
    std::memset(recv, 0, sizeof recv);
  }
  void add(int from, int to, uint64_t bytes) {
    sent[from] += bytes;
    recv[to] += bytes;
  }
};

thread_local Traffic g_last;

size_t es_of(int dt) { return dt == RAR_F32 ? 4 : 2; }
bool dt_ok(int dt) { return dt == RAR_F32 || dt == RAR_F16 || dt == RAR_BF16; }
size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }
int modn(int a, int n) { return ((a % n) + n) % n; }

size_t chunk_len_aligned(size_t count, int n, size_t align) {
  if (n < 1 || n > RAR_MAX_RANKS) return 0;
  return round_up((count + (size_t)n - 1) / (size_t)n, align);
}

void chunk_range(size_t count, size_t L, int c, size_t* lo, size_t* hi) {
  size_t a = (size_t)c * L, b = a + L;
  *lo = std::min(a, count);
  *hi = std::min(b, count);
}

int hip_rc(hipError_t e) { return e == hipSuccess ? RAR_OK : RAR_EHIP; }

// N distinct, non-null, 16-byte aligned, non-overlapping buffers of `bytes`.
// Zero-byte buffers touch no memory, so any pointer (NULL included) is fine.
int check_bufs(void* const* bufs, int n, int dt, size_t bytes) {
  if (n < 1 || n > RAR_MAX_RANKS) return RAR_EINVAL;
  if (!dt_ok(dt)) return RAR_EDTYPE;
  if (!bufs) return RAR_EOVERLAP;
  if (bytes == 0) return RAR_OK;
  std::vector<uintptr_t> a((size_t)n);
  for (int r = 0; r < n; ++r) {
    if (!bufs[r]) return RAR_EOVERLAP;
    if ((uintptr_t)bufs[r] & 15u) return RAR_EALIGN;
    a[(size_t)r] = (uintptr_t)bufs[r];
  }
  std::sort(a.begin(), a.end());
  for (int r = 0; r + 1 < n; ++r) {
    if (a[(size_t)r] == a[(size_t)r + 1] && bytes > 0) return RAR_EOVERLAP;
    if (a[(size_t)r + 1] - a[(size_t)r] < bytes) return RAR_EOVERLAP;
  }
  return RAR_OK;
}

// bufs (n buffers of `bytes`) and state (n buffers of `sbytes`): every
// pointer non-null and 16-byte aligned, no two of the 2n ranges overlapping.
int check_state_bufs(void* const* bufs, void* const* state, int n, size_t bytes, size_t sbytes) {
  if (!state) return RAR_EOVERLAP;
  if (bytes == 0) return RAR_OK;
  std::vector<std::pair<uintptr_t, size_t>> a;
  for (int r = 0; r < n; ++r) {
    if (!state[r]) return RAR_EOVERLAP;
    if ((uintptr_t)state[r] & 15u) return RAR_EALIGN;
    a.emplace_back((uintptr_t)bufs[r], bytes);
    a.emplace_back((uintptr_t)state[r], sbytes);
  }
  std::sort(a.begin(), a.end());
  for (size_t i = 0; i + 1 < a.size(); ++i)
    if (a[i + 1].first - a[i].first < a[i].second) return RAR_EOVERLAP;
  return RAR_OK;
}

// No two of the byte ranges [p, p + len) overlap; empty ranges are ignored.
int check_disjoint(std::vector<std::pair<uintptr_t, size_t>>& a) {
  a.erase(std::remove_if(a.begin(), a.end(), [](const std::pair<uintptr_t, size_t>& x) { return x.second == 0; }),
          a.end());
  std::sort(a.begin(), a.end());
  for (size_t i = 0; i + 1 < a.size(); ++i)
    if (a[i + 1].first - a[i].first < a[i].second) return RAR_EOVERLAP;
  return RAR_OK;
}

// The workspace's used bytes clear of every rank buffer (and state buffer).
int check_ws_clear(void* const* bufs, void* const* state, int n, size_t bytes, size_t sbytes, const void* ws,
                   size_t ws_used) {
  std::vector<std::pair<uintptr_t, size_t>> a;
  for (int r = 0; r < n; ++r) {
    a.emplace_back((uintptr_t)bufs[r], bytes);
    if (state) a.emplace_back((uintptr_t)state[r], sbytes);
  }
  a.emplace_back((uintptr_t)ws, ws_used);
  return check_disjoint(a);
}

RankPtrs make_ptrs(void* const* bufs, int n) {
  RankPtrs p{};
  for (int r = 0; r < n; ++r) p.p[r] = (char*)bufs[r];
  return p;
}

// Ring traffic of one pass: rank r sends chunk (r-s+shift) mod N at step s.
void ring_pass_traffic(Traffic& t, int n, size_t count, size_t L, size_t es, int shift) {
  for (int s = 1; s <= n - 1; ++s)
    for (int r = 0; r < n; ++r) {
      size_t lo, hi;
      chunk_range(count, L, modn(r - s + shift, n), &lo, &hi);
      t.add(r, (r + 1) % n, (uint64_t)(hi - lo) * es);
    }
}

void tree_traffic(Traffic& t, int n, int root, uint64_t bytes) {
  for (int span = 1; span < n; span *= 2)
    for (int rel = 0; rel < span && rel + span < n; ++rel) t.add((root + rel) % n, (root + rel + span) % n, bytes);
}

// ------------------------------------------------------------------ uncompressed steps

int run_rs_step(const RankPtrs& p, int n, size_t count, size_t L, int dt, int s, hipStream_t st) {
  return hip_rc(launch_rs_step(p, n, count, L, dt, s, st));
}

int run_ag_step(const RankPtrs& p, int n, size_t count, size_t L, size_t es, int s, hipStream_t st) {
  CopyJobs jobs{};
  jobs.ptrs = p;
  int j = 0;
  for (int r = 0; r < n; ++r) {
    size_t lo, hi;
    chunk_range(count, L, modn(r - s, n), &lo, &hi);
    if (hi == lo) continue;
    jobs.lo[j] = lo * es;
    jobs.len[j] = (hi - lo) * es;
    jobs.dstmask[j] = 1ull << r;
    jobs.src[j] = (int8_t)modn(r - 1, n);
    ++j;
  }
  jobs.njobs = j;
  return hip_rc(launch_copy_jobs(jobs, st));
}

int allreduce_impl(void* const* bufs, int n, size_t count, int dt, int algo, bool full,
                   hipStream_t st) {
  const size_t es = es_of(dt);
  int rc = check_bufs(bufs, n, dt, count * es);
  if (rc) return rc;
  if (algo != RAR_ALGO_FUSED && algo != RAR_ALGO_STEPWISE) return RAR_EINVAL;
  const size_t L = chunk_len_aligned(count, n, 128);
  g_last.reset(n);
  ring_pass_traffic(g_last, n, count, L, es, 0);
  if (full) ring_pass_traffic(g_last, n, count, L, es, 1);
  if (n == 1 || count == 0) return RAR_OK;
  RankPtrs p = make_ptrs(bufs, n);
  if (algo == RAR_ALGO_FUSED) return hip_rc(launch_ring_fold(p, n, count, L, dt, full, st));
  for (int s = 1; s <= n - 1; ++s)
    if ((rc = run_rs_step(p, n, count, L, dt, s, st))) return rc;
  if (full)
    for (int s = 1; s <= n - 1; ++s)
      if ((rc = run_ag_step(p, n, count, L, es, s, st))) return rc;
  return RAR_OK;
}

// ------------------------------------------------------------------ per-device pipeline state

struct DevCtx {
  bool ready = false;
  hipStream_t side = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
  hipEvent_t evE[kMaxEvents] = {}, evD[kMaxEvents] = {};
};

std::mutex g_ctx_mu;
DevCtx g_ctx[64];

int get_ctx(DevCtx** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return RAR_EHIP;
  DevCtx& c = g_ctx[dev];
  if (!c.ready) {
    if (hipStreamCreateWithFlags(&c.side, hipStreamNonBlocking) != hipSuccess) return RAR_EHIP;
    if (hipEventCreateWithFlags(&c.fork, hipEventDisableTiming) != hipSuccess) return RAR_EHIP;
    if (hipEventCreateWithFlags(&c.join, hipEventDisableTiming) != hipSuccess) return RAR_EHIP;
    for (int i = 0; i < kMaxEvents; ++i) {
      if (hipEventCreateWithFlags(&c.evE[i], hipEventDisableTiming) != hipSuccess) return RAR_EHIP;
      if (hipEventCreateWithFlags(&c.evD[i], hipEventDisableTiming) != hipSuccess) return RAR_EHIP;
    }
    c.ready = true;
  }
  *out = &c;
  return RAR_OK;
}

// ------------------------------------------------------------------ compressed allreduce

struct CompPlan {
  int n, dt, method, block, mbits, sched;
  size_t count, es, L, U, upc, slot;
  float theta;
};

int cfg_check(const rar_compress_cfg* cfg, int dt, CompPlan* pl) {
  if (!cfg) return RAR_EINVAL;
  if (cfg->method < RAR_COMP_NONE || cfg->method > RAR_COMP_SPARSE_AUTO) return RAR_EINVAL;
  if (cfg->mbits < 2 || cfg->mbits > 8) return RAR_EINVAL;
  if (cfg->block < 16 || cfg->block > 512 || (cfg->block & (cfg->block - 1))) return RAR_EINVAL;
  if (cfg->schedule != RAR_SCHED_FUSED && cfg->schedule != RAR_SCHED_STAGED && cfg->schedule != RAR_SCHED_FORWARD &&
      cfg->schedule != RAR_SCHED_PIPELINED)
    return RAR_EINVAL;
  const size_t es = es_of(dt);
  if (cfg->unit_bytes == 0 || cfg->unit_bytes % es) return RAR_EINVAL;
  const size_t U = cfg->unit_bytes / es;
  if (U % (size_t)cfg->block || U > 0xffffffffull) return RAR_EINVAL;
  if (!(cfg->sparsity_threshold >= 0.0f && cfg->sparsity_threshold <= 1.0f)) return RAR_EINVAL;
  pl->method = cfg->method;
  pl->block = cfg->block;
  pl->mbits = cfg->mbits;
  // SPARSE_AUTO runs staged, or pipelined with 128-element blocks (the fused
  // and forwarding schedules are BFP-only)
  pl->sched = cfg->method == RAR_COMP_BFP
                  ? cfg->schedule
                  : (cfg->schedule == RAR_SCHED_PIPELINED && cfg->block == 128 ? RAR_SCHED_PIPELINED
                                                                               : RAR_SCHED_STAGED);
  pl->U = U;
  pl->es = es;
  pl->theta = cfg->sparsity_threshold;
  return RAR_OK;
}

void plan_sizes(CompPlan* pl, int n, size_t count, int dt) {
  pl->n = n;
  pl->count = count;
  pl->dt = dt;
  pl->L = chunk_len_aligned(count, n, (size_t)std::max(128, pl->block));
  pl->upc = pl->L ? (pl->L + pl->U - 1) / pl->U : 0;
  size_t slot = bfp_msg_bytes(pl->U, pl->block, pl->mbits);
  if (pl->method == RAR_COMP_SPARSE_AUTO) {
    const size_t body_max = round_up(pl->U * pl->es, 16) + 4 * pl->U;  // all non-zero
    // pipelined: a sparse message's body follows the BFP area in its slot
    slot = pl->sched == RAR_SCHED_PIPELINED ? 16 + round_up(slot, 16) + body_max : std::max(16 + slot, 16 + body_max);
  }
  pl->slot = round_up(slot, kAlign);
}

size_t slots_offset() { return round_up(kTrafficBytes, kAlign); }
size_t tiles_offset(const CompPlan& pl) { return slots_offset() + (size_t)pl.n * pl.upc * pl.slot; }
size_t tiles_per_slot(const CompPlan& pl) { return 2 * (size_t)comp_tiles_per_unit(pl.U); }

size_t workspace_need(const CompPlan& pl) {
  if (pl.method == RAR_COMP_NONE || pl.sched == RAR_SCHED_FUSED) return kTrafficBytes;
  if (pl.sched == RAR_SCHED_FORWARD) return slots_offset() + 2 * (size_t)pl.n * pl.upc * pl.slot;
  if (pl.sched == RAR_SCHED_PIPELINED) {
    const size_t slots = slots_offset() + (size_t)pl.n * pl.n * pl.upc * pl.slot;
    if (pl.method != RAR_COMP_SPARSE_AUTO) return slots;
    return slots + 8 * (size_t)sparse_pipe_flag_words(pl.n, pl.upc, pl.U, pl.dt);
  }
  size_t need = tiles_offset(pl);
  if (pl.method == RAR_COMP_SPARSE_AUTO) need += (size_t)pl.n * pl.upc * tiles_per_slot(pl) * sizeof(uint32_t);
  return need;
}

int write_traffic(const Traffic& t, void* ws, hipStream_t st) {
  uint64_t vals[2 * RAR_MAX_RANKS] = {};
  for (int r = 0; r < t.n; ++r) {
    vals[r] = t.sent[r];
    vals[RAR_MAX_RANKS + r] = t.recv[r];
  }
  return hip_rc(launch_fill_u64((uint64_t*)ws, vals, 2 * RAR_MAX_RANKS, st));
}

// Staged BFP ring: messages materialised per (sender, unit) in the workspace.
int staged_bfp(const CompPlan& pl, void* const* bufs, char* ws, Traffic& tr, hipStream_t st) {
  DevCtx* ctx = nullptr;
  std::lock_guard<std::mutex> lock(g_ctx_mu);
  int rc = get_ctx(&ctx);
  if (rc) return rc;
  const int n = pl.n;
  char* slots = ws + slots_offset();
  auto slot = [&](int rank, size_t u) { return (uint8_t*)(slots + ((size_t)rank * pl.upc + u) * pl.slot); };
  hipStream_t E = st, D = ctx->side;
  if (hipEventRecord(ctx->fork, E) != hipSuccess || hipStreamWaitEvent(D, ctx->fork, 0) != hipSuccess)
    return RAR_EHIP;
  // reduce-scatter hops
  for (int s = 1; s <= n - 1; ++s) {
    for (size_t u = 0; u < pl.upc; ++u) {
      BfpJobs enc{}, dec{};
      int j = 0;
      for (int r = 0; r < n; ++r) {
        const int src = modn(r - 1, n), c = modn(r - s - 1, n);
        size_t lo, hi;
        chunk_range(pl.count, pl.L, c, &lo, &hi);
        const size_t ulo = lo + u * pl.U;
        if (ulo >= hi) continue;
        const size_t len = std::min(pl.U, hi - ulo);
        enc.src[j] = (const char*)bufs[src] + ulo * pl.es;
        enc.msg[j] = slot(src, u);
        enc.len[j] = len;
        dec.dst[j] = (char*)bufs[r] + ulo * pl.es;
        dec.msg[j] = slot(src, u);
        dec.len[j] = len;
        tr.add(src, r, bfp_msg_bytes(len, pl.block, pl.mbits));
        ++j;
      }
      if (!j) continue;
      enc.njobs = dec.njobs = j;
      hipEvent_t eE = ctx->evE[u % kMaxEvents], eD = ctx->evD[u % kMaxEvents];
      if (s > 1 && hipStreamWaitEvent(E, eD, 0) != hipSuccess) return RAR_EHIP;
      if ((rc = hip_rc(launch_bfp_encode(enc, pl.dt, pl.block, pl.mbits, E)))) return rc;
      if (hipEventRecord(eE, E) != hipSuccess || hipStreamWaitEvent(D, eE, 0) != hipSuccess) return RAR_EHIP;
      if ((rc = hip_rc(launch_bfp_decode(dec, pl.dt, pl.block, pl.mbits, true, D)))) return rc;
      if (hipEventRecord(eD, D) != hipSuccess) return RAR_EHIP;
    }
  }
  // allgather: each owner encodes its finished unit once; every rank stores
  // the decoded unit (the relayed bytes are the owner's message unchanged)
  RankPtrs fan = make_ptrs(bufs, n);
  for (size_t u = 0; u < pl.upc; ++u) {
    BfpJobs enc{};
    uint64_t off[kMaxRanks] = {};
    int j = 0;
    for (int c = 0; c < n; ++c) {
      size_t lo, hi;
      chunk_range(pl.count, pl.L, c, &lo, &hi);
      const size_t ulo = lo + u * pl.U;
      if (ulo >= hi) continue;
      const size_t len = std::min(pl.U, hi - ulo);
      enc.src[j] = (const char*)bufs[c] + ulo * pl.es;
      enc.msg[j] = slot(c, u);
      enc.len[j] = len;
      off[j] = ulo;
      const uint64_t bytes = bfp_msg_bytes(len, pl.block, pl.mbits);
      for (int s = 1; s <= n - 1; ++s) tr.add(modn(c + s - 1, n), modn(c + s, n), bytes);
      ++j;
    }
    if (!j) continue;
    enc.njobs = j;
    hipEvent_t eE = ctx->evE[u % kMaxEvents], eD = ctx->evD[u % kMaxEvents];
    if (hipStreamWaitEvent(E, eD, 0) != hipSuccess) return RAR_EHIP;
    if ((rc = hip_rc(launch_bfp_encode(enc, pl.dt, pl.block, pl.mbits, E)))) return rc;
    if (hipEventRecord(eE, E) != hipSuccess || hipStreamWaitEvent(D, eE, 0) != hipSuccess) return RAR_EHIP;
    if ((rc = hip_rc(launch_bfp_decode_fanout(enc, fan, n, off, pl.dt, pl.block, pl.mbits, D)))) return rc;
    if (hipEventRecord(eD, D) != hipSuccess) return RAR_EHIP;
  }
  if (hipEventRecord(ctx->join, D) != hipSuccess || hipStreamWaitEvent(E, ctx->join, 0) != hipSuccess)
    return RAR_EHIP;
  return RAR_OK;
}

// Staged SPARSE_AUTO ring: each unit message is sparse or BFP by the
// threshold rule; sizes (and so the byte counters) are decided on the device.
int staged_sparse(const CompPlan& pl, void* const* bufs, char* ws, hipStream_t st) {
  DevCtx* ctx = nullptr;
  std::lock_guard<std::mutex> lock(g_ctx_mu);
  int rc = get_ctx(&ctx);
  if (rc) return rc;
  const int n = pl.n;
  char* slots = ws + slots_offset();
  uint32_t* tiles = (uint32_t*)(ws + tiles_offset(pl));
  const size_t tps = tiles_per_slot(pl);
  auto slot = [&](int rank, size_t u) { return (uint8_t*)(slots + ((size_t)rank * pl.upc + u) * pl.slot); };
  auto scratch = [&](int rank, size_t u) { return tiles + ((size_t)rank * pl.upc + u) * tps; };
  uint64_t* traffic = (uint64_t*)ws;
  hipStream_t E = st, D = ctx->side;
  const uint64_t zeros[2 * RAR_MAX_RANKS] = {};
  if ((rc = hip_rc(launch_fill_u64(traffic, zeros, 2 * RAR_MAX_RANKS, E)))) return rc;
  if (hipEventRecord(ctx->fork, E) != hipSuccess || hipStreamWaitEvent(D, ctx->fork, 0) != hipSuccess)
    return RAR_EHIP;
  for (int s = 1; s <= n - 1; ++s) {
    for (size_t u = 0; u < pl.upc; ++u) {
      CompJobs enc{};
      CompAccJobs dec{};
      int j = 0;
      for (int r = 0; r < n; ++r) {
        const int src = modn(r - 1, n), c = modn(r - s - 1, n);
        size_t lo, hi;
        chunk_range(pl.count, pl.L, c, &lo, &hi);
        const size_t ulo = lo + u * pl.U;
        if (ulo >= hi) continue;
        const size_t len = std::min(pl.U, hi - ulo);
        enc.src[j] = (const char*)bufs[src] + ulo * pl.es;
        enc.msg[j] = slot(src, u);
        enc.tiles[j] = scratch(src, u);
        enc.len[j] = len;
        enc.from[j] = (int8_t)src;
        enc.hops[j] = 1;
        dec.dst[j] = (char*)bufs[r] + ulo * pl.es;
        dec.msg[j] = slot(src, u);
        dec.len[j] = len;
        dec.counts[j] = scratch(r, u);  // r encodes this partial next (or, at s = N-1, as the owner)
        ++j;
      }
      if (!j) continue;
      enc.njobs = dec.njobs = j;
      enc.nranks = n;
      hipEvent_t eE = ctx->evE[u % kMaxEvents], eD = ctx->evD[u % kMaxEvents];
      if (s > 1 && hipStreamWaitEvent(E, eD, 0) != hipSuccess) return RAR_EHIP;
      // from step 2 on, the sender's tile counts came with the decode that made its partial
      if ((rc = hip_rc(launch_comp_encode(enc, pl.dt, pl.block, pl.mbits, pl.theta, traffic, s > 1, E)))) return rc;
      if (hipEventRecord(eE, E) != hipSuccess || hipStreamWaitEvent(D, eE, 0) != hipSuccess) return RAR_EHIP;
      if ((rc = hip_rc(launch_comp_decode_acc(dec, pl.dt, pl.block, pl.mbits, D)))) return rc;
      if (hipEventRecord(eD, D) != hipSuccess) return RAR_EHIP;
    }
  }
  RankPtrs fan = make_ptrs(bufs, n);
  for (size_t u = 0; u < pl.upc; ++u) {
    CompJobs enc{};
    BfpJobs dec{};
    uint64_t off[kMaxRanks] = {};
    int j = 0;
    for (int c = 0; c < n; ++c) {
      size_t lo, hi;
      chunk_range(pl.count, pl.L, c, &lo, &hi);
      const size_t ulo = lo + u * pl.U;
      if (ulo >= hi) continue;
      const size_t len = std::min(pl.U, hi - ulo);
      enc.src[j] = (const char*)bufs[c] + ulo * pl.es;
      enc.msg[j] = slot(c, u);
      enc.tiles[j] = scratch(c, u);
      enc.len[j] = len;
      enc.from[j] = (int8_t)c;
      enc.hops[j] = (int8_t)(n - 1);
      dec.msg[j] = slot(c, u);
      dec.len[j] = len;
      off[j] = ulo;
      ++j;
    }
    if (!j) continue;
    enc.njobs = dec.njobs = j;
    enc.nranks = n;
    hipEvent_t eE = ctx->evE[u % kMaxEvents], eD = ctx->evD[u % kMaxEvents];
    if (hipStreamWaitEvent(E, eD, 0) != hipSuccess) return RAR_EHIP;
    // the owner's counts came with the last reduce-scatter decode
    if ((rc = hip_rc(launch_comp_encode(enc, pl.dt, pl.block, pl.mbits, pl.theta, traffic, true, E)))) return rc;
    if (hipEventRecord(eE, E) != hipSuccess || hipStreamWaitEvent(D, eE, 0) != hipSuccess) return RAR_EHIP;
    if ((rc = hip_rc(launch_comp_decode_fanout(dec, fan, n, off, pl.dt, pl.block, pl.mbits, D)))) return rc;
    if (hipEventRecord(eD, D) != hipSuccess) return RAR_EHIP;
  }
  if (hipEventRecord(ctx->join, D) != hipSuccess || hipStreamWaitEvent(E, ctx->join, 0) != hipSuccess)
    return RAR_EHIP;
  return RAR_OK;
}

// Forwarding BFP ring: message slots [parity][rank][unit] in the workspace.
// Hop 0: every rank q encodes its own chunk (q-1) mod N, the one it sends at
// reduce-scatter step 1.  Hop s = 1..N-1: receiver r decodes rank r-1's
// message of chunk (r-s-1) mod N, adds its own copy and encodes the sum as
// its next message (at s = N-1 r owns the chunk and the message is the
// allgather's).  Then every rank stores the owners' messages decoded.
int forward_bfp(const CompPlan& pl, void* const* bufs, char* ws, hipStream_t st) {
  const int n = pl.n;
  char* slots = ws + slots_offset();
  auto slot = [&](int parity, int rank, size_t u) {
    return (uint8_t*)(slots + (((size_t)parity * n + rank) * pl.upc + u) * pl.slot);
  };
  int rc;
  FwdJobs jobs{};
  auto flush = [&]() -> int {
    if (jobs.njobs == 0) return RAR_OK;
    const int r = hip_rc(launch_bfp_forward(jobs, pl.dt, pl.block, pl.mbits, st));
    jobs.njobs = 0;
    return r;
  };
  for (int s = 0; s <= n - 1; ++s) {
    for (int r = 0; r < n; ++r) {
      const int c = modn(r - s - 1, n);
      size_t lo, hi;
      chunk_range(pl.count, pl.L, c, &lo, &hi);
      for (size_t u = 0; u < pl.upc; ++u) {
        const size_t ulo = lo + u * pl.U;
        if (ulo >= hi) break;
        const int j = jobs.njobs++;
        jobs.in[j] = s == 0 ? nullptr : slot((s - 1) & 1, modn(r - 1, n), u);
        jobs.local[j] = (const char*)bufs[r] + ulo * pl.es;
        jobs.out[j] = slot(s & 1, r, u);
        jobs.len[j] = std::min(pl.U, hi - ulo);
        if (jobs.njobs == kMaxRanks && (rc = flush())) return rc;
      }
    }
    if ((rc = flush())) return rc;  // hop s+1 reads what hop s wrote: stream order separates them
  }
  RankPtrs fan = make_ptrs(bufs, n);
  BfpJobs ag{};
  uint64_t off[kMaxRanks] = {};
  auto flush_ag = [&]() -> int {
    if (ag.njobs == 0) return RAR_OK;
    const int r = hip_rc(launch_bfp_decode_fanout(ag, fan, n, off, pl.dt, pl.block, pl.mbits, st));
    ag.njobs = 0;
    return r;
  };
  for (int c = 0; c < n; ++c) {
    size_t lo, hi;
    chunk_range(pl.count, pl.L, c, &lo, &hi);
    for (size_t u = 0; u < pl.upc; ++u) {
      const size_t ulo = lo + u * pl.U;
      if (ulo >= hi) break;
      const int j = ag.njobs++;
      ag.msg[j] = slot((n - 1) & 1, c, u);
      ag.len[j] = std::min(pl.U, hi - ulo);
      off[j] = ulo;
      if (ag.njobs == kMaxRanks && (rc = flush_ag())) return rc;
    }
  }
  return flush_ag();
}

void fused_bfp_traffic(const CompPlan& pl, Traffic& tr) {
  const int n = pl.n;
  for (int s = 1; s <= n - 1; ++s)
    for (int r = 0; r < n; ++r) {
      size_t lo, hi;
      chunk_range(pl.count, pl.L, modn(r - s - 1, n), &lo, &hi);
      for (size_t u = lo; u < hi; u += pl.U)
        tr.add(modn(r - 1, n), r, bfp_msg_bytes(std::min(pl.U, hi - u), pl.block, pl.mbits));
    }
  for (int c = 0; c < n; ++c) {
    size_t lo, hi;
    chunk_range(pl.count, pl.L, c, &lo, &hi);
    for (size_t u = lo; u < hi; u += pl.U) {
      const uint64_t bytes = bfp_msg_bytes(std::min(pl.U, hi - u), pl.block, pl.mbits);
      for (int s = 1; s <= n - 1; ++s) tr.add(modn(c + s - 1, n), modn(c + s, n), bytes);
    }
  }
}

}  // namespace

// ====================================================================== C ABI

extern "C" {

size_t rar_chunk_len(size_t count, int nranks) { return chunk_len_aligned(count, nranks, 128); }

int rar_ring_allreduce_ex(void* const* bufs, int nranks, size_t count, int dtype, int algo, void* stream) {
  return allreduce_impl(bufs, nranks, count, dtype, algo, true, (hipStream_t)stream);
}

int rar_ring_allreduce(void* const* bufs, int nranks, size_t count, int dtype, void* stream) {
  return rar_ring_allreduce_ex(bufs, nranks, count, dtype, RAR_ALGO_FUSED, stream);
}

int rar_reduce_scatter_ex(void* const* bufs, int nranks, size_t count, int dtype, int algo, void* stream) {
  return allreduce_impl(bufs, nranks, count, dtype, algo, false, (hipStream_t)stream);
}

int rar_reduce_scatter(void* const* bufs, int nranks, size_t count, int dtype, void* stream) {
  return rar_reduce_scatter_ex(bufs, nranks, count, dtype, RAR_ALGO_FUSED, stream);
}

int rar_rs_step(void* const* bufs, int nranks, size_t count, int dtype, int step, void* stream) {
  int rc = check_bufs(bufs, nranks, dtype, count * es_of(dtype));
  if (rc) return rc;
  if (step < 1 || step > nranks - 1) return RAR_EINVAL;
  const size_t L = chunk_len_aligned(count, nranks, 128);
  g_last.reset(nranks);
  for (int r = 0; r < nranks; ++r) {
    size_t lo, hi;
    chunk_range(count, L, modn(r - step, nranks), &lo, &hi);
    g_last.add(r, (r + 1) % nranks, (uint64_t)(hi - lo) * es_of(dtype));
  }
  if (count == 0) return RAR_OK;
  return run_rs_step(make_ptrs(bufs, nranks), nranks, count, L, dtype, step, (hipStream_t)stream);
}

int rar_ag_step(void* const* bufs, int nranks, size_t count, int dtype, int step, void* stream) {
  int rc = check_bufs(bufs, nranks, dtype, count * es_of(dtype));
  if (rc) return rc;
  if (step < 1 || step > nranks - 1) return RAR_EINVAL;
  const size_t L = chunk_len_aligned(count, nranks, 128);
  g_last.reset(nranks);
  for (int r = 0; r < nranks; ++r) {
    size_t lo, hi;
    chunk_range(count, L, modn(r - step + 1, nranks), &lo, &hi);
    g_last.add(r, (r + 1) % nranks, (uint64_t)(hi - lo) * es_of(dtype));
  }
  if (count == 0) return RAR_OK;
  return run_ag_step(make_ptrs(bufs, nranks), nranks, count, L, es_of(dtype), step, (hipStream_t)stream);
}

int rar_allgather_ex(void* const* bufs, int nranks, size_t count, int dtype, int algo, void* stream) {
  const size_t es = es_of(dtype);
  int rc = check_bufs(bufs, nranks, dtype, count * es);
  if (rc) return rc;
  if (count % (size_t)nranks) return RAR_EINVAL;
  if (algo != RAR_ALGO_FUSED && algo != RAR_ALGO_STEPWISE) return RAR_EINVAL;
  const size_t shard = count / (size_t)nranks;
  g_last.reset(nranks);
  ring_pass_traffic(g_last, nranks, count, shard, es, 1);
  if (nranks == 1 || count == 0) return RAR_OK;
  RankPtrs p = make_ptrs(bufs, nranks);
  hipStream_t st = (hipStream_t)stream;
  if (algo == RAR_ALGO_STEPWISE) {
    for (int s = 1; s <= nranks - 1; ++s)
      if ((rc = run_ag_step(p, nranks, count, shard, es, s, st))) return rc;
    return RAR_OK;
  }
  CopyJobs jobs{};
  jobs.ptrs = p;
  const uint64_t all = nranks == 64 ? ~0ull : ((1ull << nranks) - 1);
  for (int c = 0; c < nranks; ++c) {
    jobs.lo[c] = (uint64_t)c * shard * es;
    jobs.len[c] = shard * es;
    jobs.dstmask[c] = all & ~(1ull << c);
    jobs.src[c] = (int8_t)c;
  }
  jobs.njobs = nranks;
  return hip_rc(launch_copy_jobs(jobs, st));
}

int rar_allgather(void* const* bufs, int nranks, size_t count, int dtype, void* stream) {
  return rar_allgather_ex(bufs, nranks, count, dtype, RAR_ALGO_FUSED, stream);
}

int rar_broadcast_ex(void* const* bufs, int nranks, size_t count, int dtype, int root, int algo,
                     void* stream) {
  const size_t es = es_of(dtype);
  int rc = check_bufs(bufs, nranks, dtype, count * es);
  if (rc) return rc;
  if (root < 0 || root >= nranks) return RAR_EINVAL;
  if (algo != RAR_ALGO_FUSED && algo != RAR_ALGO_STEPWISE) return RAR_EINVAL;
  g_last.reset(nranks);
  tree_traffic(g_last, nranks, root, (uint64_t)count * es);
  if (nranks == 1 || count == 0) return RAR_OK;
  RankPtrs p = make_ptrs(bufs, nranks);
  hipStream_t st = (hipStream_t)stream;
  if (algo == RAR_ALGO_FUSED) {
    CopyJobs jobs{};
    jobs.ptrs = p;
    const uint64_t all = nranks == 64 ? ~0ull : ((1ull << nranks) - 1);
    jobs.lo[0] = 0;
    jobs.len[0] = count * es;
    jobs.dstmask[0] = all & ~(1ull << root);
    jobs.src[0] = (int8_t)root;
    jobs.njobs = 1;
    return hip_rc(launch_copy_jobs(jobs, st));
  }
  for (int span = 1; span < nranks; span *= 2) {
    CopyJobs jobs{};
    jobs.ptrs = p;
    int j = 0;
    for (int rel = 0; rel < span && rel + span < nranks; ++rel) {
      jobs.lo[j] = 0;
      jobs.len[j] = count * es;
      jobs.dstmask[j] = 1ull << ((root + rel + span) % nranks);
      jobs.src[j] = (int8_t)((root + rel) % nranks);
      ++j;
    }
    jobs.njobs = j;
    if ((rc = hip_rc(launch_copy_jobs(jobs, st)))) return rc;
  }
  return RAR_OK;
}

int rar_broadcast(void* const* bufs, int nranks, size_t count, int dtype, int root, void* stream) {
  return rar_broadcast_ex(bufs, nranks, count, dtype, root, RAR_ALGO_FUSED, stream);
}

// ------------------------------------------------------------------ tree allreduce

static int tree_broadcast_rounds(const RankPtrs& p, int nranks, size_t bytes, hipStream_t st) {
  for (int span = 1; span < nranks; span *= 2) {
    CopyJobs jobs{};
    jobs.ptrs = p;
    int j = 0;
    for (int rel = 0; rel < span && rel + span < nranks; ++rel) {
      jobs.lo[j] = 0;
      jobs.len[j] = bytes;
      jobs.dstmask[j] = 1ull << (rel + span);
      jobs.src[j] = (int8_t)rel;
      ++j;
    }
    jobs.njobs = j;
    int rc = hip_rc(launch_copy_jobs(jobs, st));
    if (rc) return rc;
  }
  return RAR_OK;
}

int rar_tree_allreduce_ex(void* const* bufs, int nranks, size_t count, int dtype, int algo, void* stream) {
  const size_t es = es_of(dtype);
  int rc = check_bufs(bufs, nranks, dtype, count * es);
  if (rc) return rc;
  if (algo != RAR_ALGO_FUSED && algo != RAR_ALGO_STEPWISE) return RAR_EINVAL;
  g_last.reset(nranks);
  for (int span = 1; span < nranks; span *= 2)
    for (int rel = 0; rel + span < nranks; rel += 2 * span) g_last.add(rel + span, rel, (uint64_t)count * es);
  tree_traffic(g_last, nranks, 0, (uint64_t)count * es);
  if (nranks == 1 || count == 0) return RAR_OK;
  RankPtrs p = make_ptrs(bufs, nranks);
  hipStream_t st = (hipStream_t)stream;
  if (algo == RAR_ALGO_FUSED && tree_fold_supported(nranks))
    return hip_rc(launch_tree_fold(p, nranks, count, dtype, st));
  for (int span = 1; span < nranks; span *= 2) {
    PairJobs pairs{};
    for (int rel = 0; rel + span < nranks; rel += 2 * span) {
      pairs.dst[pairs.npairs] = (int8_t)rel;
      pairs.src[pairs.npairs] = (int8_t)(rel + span);
      ++pairs.npairs;
    }
    if ((rc = hip_rc(launch_pair_add(p, pairs, count, dtype, st)))) return rc;
  }
  return tree_broadcast_rounds(p, nranks, count * es, st);
}

int rar_tree_allreduce(void* const* bufs, int nranks, size_t count, int dtype, void* stream) {
  return rar_tree_allreduce_ex(bufs, nranks, count, dtype, RAR_ALGO_FUSED, stream);
}

int rar_allreduce_auto(void* const* bufs, int nranks, size_t count, int dtype, size_t threshold_bytes,
                       int* chosen, void* stream) {
  if (!dt_ok(dtype)) return RAR_EDTYPE;
  const size_t thr = threshold_bytes ? threshold_bytes : (size_t)RAR_TREE_THRESHOLD_DEFAULT;
  const int tree = count * es_of(dtype) < thr;
  const int rc = tree ? rar_tree_allreduce(bufs, nranks, count, dtype, stream)
                      : rar_ring_allreduce(bufs, nranks, count, dtype, stream);
  if (rc == RAR_OK && chosen) *chosen = tree ? RAR_ALLREDUCE_TREE : RAR_ALLREDUCE_RING;
  return rc;
}

int rar_last_traffic(uint64_t* sent, uint64_t* recv, int nranks) {
  if (!sent || !recv || nranks < 1 || nranks > RAR_MAX_RANKS) return RAR_EINVAL;
  for (int r = 0; r < nranks; ++r) {
    sent[r] = r < g_last.n ? g_last.sent[r] : 0;
    recv[r] = r < g_last.n ? g_last.recv[r] : 0;
  }
  return RAR_OK;
}

// ------------------------------------------------------------------ BFP

size_t rar_bfp_bytes(size_t count, int block, int mbits) {
  if (mbits < 2 || mbits > 8 || block < 16 || block > 512 || (block & (block - 1))) return 0;
  return bfp_msg_bytes(count, block, mbits);
}

static int bfp_args(const void* a, const void* b, int dt, int block, int mbits) {
  if (!a || !b) return RAR_EINVAL;
  if (!dt_ok(dt)) return RAR_EDTYPE;
  if (rar_bfp_bytes(1, block, mbits) == 0) return RAR_EINVAL;
  if (((uintptr_t)a & 15u) || ((uintptr_t)b & 15u)) return RAR_EALIGN;
  return RAR_OK;
}

int rar_bfp_compress(const void* src, int src_dtype, size_t count, int block, int mbits, void* dst,
                     void* stream) {
  int rc = bfp_args(src, dst, src_dtype, block, mbits);
  if (rc) return rc;
  if (count == 0) return RAR_OK;
  BfpJobs jobs{};
  jobs.src[0] = (const char*)src;
  jobs.msg[0] = (uint8_t*)dst;
  jobs.len[0] = count;
  jobs.njobs = 1;
  return hip_rc(launch_bfp_encode(jobs, src_dtype, block, mbits, (hipStream_t)stream));
}

static int bfp_decode_entry(const void* src, size_t count, int block, int mbits, void* dst, int dt,
                            bool acc, void* stream) {
  int rc = bfp_args(src, dst, dt, block, mbits);
  if (rc) return rc;
  if (count == 0) return RAR_OK;
  BfpJobs jobs{};
  jobs.msg[0] = (uint8_t*)src;
  jobs.dst[0] = (char*)dst;
  jobs.len[0] = count;
  jobs.njobs = 1;
  return hip_rc(launch_bfp_decode(jobs, dt, block, mbits, acc, (hipStream_t)stream));
}

int rar_bfp_decompress_accumulate(const void* src, size_t count, int block, int mbits, void* acc,
                                  int acc_dtype, void* stream) {
  return bfp_decode_entry(src, count, block, mbits, acc, acc_dtype, true, stream);
}

int rar_bfp_decompress(const void* src, size_t count, int block, int mbits, void* dst, int dst_dtype,
                       void* stream) {
  return bfp_decode_entry(src, count, block, mbits, dst, dst_dtype, false, stream);
}

// ------------------------------------------------------------------ compressed allreduce

void rar_compress_cfg_default(rar_compress_cfg* cfg) {
  if (!cfg) return;
  cfg->method = RAR_COMP_BFP;
  cfg->block = 128;
  cfg->mbits = 8;
  cfg->sparsity_threshold = 0.5f;
  cfg->unit_bytes = (size_t)4 << 20;
  cfg->collective_mask = RAR_OP_ALLREDUCE;
  cfg->schedule = RAR_SCHED_FUSED;
}

size_t rar_compressed_chunk_len(size_t count, int nranks, int block) {
  if (block < 16 || block > 512 || (block & (block - 1))) return 0;
  return chunk_len_aligned(count, nranks, (size_t)std::max(128, block));
}

size_t rar_compressed_workspace_bytes(int nranks, size_t count, int dtype, const rar_compress_cfg* cfg) {
  if (nranks < 1 || nranks > RAR_MAX_RANKS || !dt_ok(dtype)) return 0;
  CompPlan pl{};
  if (cfg_check(cfg, dtype, &pl)) return 0;
  if (!(cfg->collective_mask & RAR_OP_ALLREDUCE)) pl.method = RAR_COMP_NONE;
  plan_sizes(&pl, nranks, count, dtype);
  return workspace_need(pl);
}

}  // extern "C"

namespace {

// Checks and plan of a compressed allreduce, up to (not including) the
// workspace.  The caller then checks the workspace it will use.
int compressed_plan(void* const* bufs, int nranks, size_t count, int dtype, const rar_compress_cfg* cfg,
                    CompPlan* pl) {
  int rc = check_bufs(bufs, nranks, dtype, count * es_of(dtype));
  if (rc) return rc;
  if ((rc = cfg_check(cfg, dtype, pl))) return rc;
  if (!(cfg->collective_mask & RAR_OP_ALLREDUCE)) pl->method = RAR_COMP_NONE;
  plan_sizes(pl, nranks, count, dtype);
  return RAR_OK;
}

int compressed_run(const CompPlan& pl, void* const* bufs, void* workspace, hipStream_t st);

// File-scope scratch of the allocation-free compressed allreduce.  In host
// code `scratch` names a host-side stand-in, not device memory: its device
// address is looked up once per device with hipGetSymbolAddress and only
// that address is handed to kernels.
static __device__ __align__(256) unsigned char scratch[RAR_NOALLOC_SCRATCH_BYTES];

std::mutex g_scratch_mu;
void* g_scratch_ptr[64] = {};

int scratch_of_current_device(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return RAR_EHIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return RAR_EHIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return RAR_OK;
}

}  // namespace

extern "C" {

int rar_ring_allreduce_compressed_noalloc(void* const* bufs, int nranks, size_t count, int dtype,
                                          const rar_compress_cfg* cfg, void* stream) {
  CompPlan pl{};
  int rc = compressed_plan(bufs, nranks, count, dtype, cfg, &pl);
  if (rc) return rc;
  if (workspace_need(pl) > (size_t)RAR_NOALLOC_SCRATCH_BYTES) return RAR_EWORKSPACE;
  void* ws = nullptr;
  if ((rc = scratch_of_current_device(&ws))) return rc;
  // the stream and events of the staged schedules are made here, not mid-call
  if (pl.method != RAR_COMP_NONE && pl.sched == RAR_SCHED_STAGED) {
    DevCtx* ctx = nullptr;
    std::lock_guard<std::mutex> lock(g_ctx_mu);
    if ((rc = get_ctx(&ctx))) return rc;
  }
  return compressed_run(pl, bufs, ws, (hipStream_t)stream);
}

int rar_ring_allreduce_compressed(void* const* bufs, int nranks, size_t count, int dtype,
                                  const rar_compress_cfg* cfg, void* workspace, size_t ws_bytes,
                                  void* stream) {
  CompPlan pl{};
  int rc = compressed_plan(bufs, nranks, count, dtype, cfg, &pl);
  if (rc) return rc;
  if (!workspace || ws_bytes < workspace_need(pl)) return RAR_EWORKSPACE;
  if ((uintptr_t)workspace & 15u) return RAR_EALIGN;
  if ((rc = check_ws_clear(bufs, nullptr, nranks, count * es_of(dtype), 0, workspace, workspace_need(pl))))
    return rc;
  return compressed_run(pl, bufs, workspace, (hipStream_t)stream);
}

}  // extern "C"

namespace {

int compressed_run(const CompPlan& pl, void* const* bufs, void* workspace, hipStream_t st) {
  const int nranks = pl.n, dtype = pl.dt;
  const size_t count = pl.count;
  int rc;
  Traffic tr;
  tr.reset(nranks);
  if (pl.method == RAR_COMP_NONE) {
    if ((rc = allreduce_impl(bufs, nranks, count, dtype, RAR_ALGO_FUSED, true, st))) return rc;
    return write_traffic(g_last, workspace, st);
  }
  if (pl.method == RAR_COMP_SPARSE_AUTO) {
    if (nranks == 1 || count == 0) return write_traffic(tr, workspace, st);
    if (pl.sched == RAR_SCHED_PIPELINED) {
      char* ws = (char*)workspace;
      const size_t flags_off = slots_offset() + (size_t)pl.n * pl.n * pl.upc * pl.slot;
      const hipError_t e = launch_sparse_pipe(make_ptrs(bufs, nranks), nranks, count, pl.L, pl.U, pl.upc, pl.slot,
                                              (uint8_t*)ws + slots_offset(), (uint64_t*)(ws + flags_off),
                                              sparse_pipe_flag_words(pl.n, pl.upc, pl.U, pl.dt), (uint64_t*)ws, dtype,
                                              pl.block, pl.mbits, pl.theta, st);
      return e == hipErrorCooperativeLaunchTooLarge ? RAR_ENOTSUP : hip_rc(e);
    }
    return staged_sparse(pl, bufs, (char*)workspace, st);
  }
  if (nranks > 1 && count > 0) {
    if (pl.sched == RAR_SCHED_FUSED) {
      fused_bfp_traffic(pl, tr);
      if ((rc = hip_rc(launch_bfp_ring_fold(make_ptrs(bufs, nranks), nranks, count, pl.L, dtype, pl.block,
                                            pl.mbits, st))))
        return rc;
    } else if (pl.sched == RAR_SCHED_FORWARD) {
      fused_bfp_traffic(pl, tr);
      if ((rc = forward_bfp(pl, bufs, (char*)workspace, st))) return rc;
    } else if (pl.sched == RAR_SCHED_PIPELINED) {
      fused_bfp_traffic(pl, tr);
      if ((rc = hip_rc(launch_bfp_pipe(make_ptrs(bufs, nranks), nranks, count, pl.L, pl.U, pl.upc, pl.slot,
                                       (uint8_t*)workspace + slots_offset(), dtype, pl.block, pl.mbits, st))))
        return rc;
    } else {
      if ((rc = staged_bfp(pl, bufs, (char*)workspace, tr, st))) return rc;
    }
  }
  return write_traffic(tr, workspace, st);
}

}  // namespace

extern "C" {

int rar_ring_allreduce_compressed_state(void* const* bufs, void* const* state, int nranks, size_t count, int dtype,
                                        int feedback, const rar_compress_cfg* cfg, void* workspace, size_t ws_bytes,
                                        void* stream) {
  const size_t es = es_of(dtype);
  int rc = check_bufs(bufs, nranks, dtype, count * es);
  if (rc) return rc;
  if (feedback != RAR_FEEDBACK_ERROR && feedback != RAR_FEEDBACK_DELTA) return RAR_EINVAL;
  CompPlan pl{};
  if ((rc = cfg_check(cfg, dtype, &pl))) return rc;
  if (cfg->method != RAR_COMP_BFP || cfg->schedule != RAR_SCHED_FUSED || !(cfg->collective_mask & RAR_OP_ALLREDUCE))
    return RAR_ENOTSUP;
  if ((rc = check_state_bufs(bufs, state, nranks, count * es, count * sizeof(float)))) return rc;
  plan_sizes(&pl, nranks, count, dtype);
  if (!workspace || ws_bytes < workspace_need(pl)) return RAR_EWORKSPACE;
  if ((uintptr_t)workspace & 15u) return RAR_EALIGN;
  if ((rc = check_ws_clear(bufs, state, nranks, count * es, count * sizeof(float), workspace, workspace_need(pl))))
    return rc;
  hipStream_t st = (hipStream_t)stream;
  Traffic tr;
  tr.reset(nranks);
  if (nranks > 1 && count > 0) {
    fused_bfp_traffic(pl, tr);
    if ((rc = hip_rc(launch_bfp_ring_fold_state(make_ptrs(bufs, nranks), make_ptrs(state, nranks), nranks, count,
                                                 pl.L, dtype, pl.block, pl.mbits, feedback, st))))
      return rc;
  }
  return write_traffic(tr, workspace, st);
}

int rar_compressed_traffic(const void* workspace, int nranks, uint64_t* sent, uint64_t* recv, void* stream) {
  if (!workspace || !sent || !recv || nranks < 1 || nranks > RAR_MAX_RANKS) return RAR_EINVAL;
  if (hipStreamSynchronize((hipStream_t)stream) != hipSuccess) return RAR_EHIP;
  uint64_t vals[2 * RAR_MAX_RANKS];
  if (hipMemcpy(vals, workspace, sizeof vals, hipMemcpyDeviceToHost) != hipSuccess) return RAR_EHIP;
  for (int r = 0; r < nranks; ++r) {
    sent[r] = vals[r];
    recv[r] = vals[RAR_MAX_RANKS + r];
  }
  return RAR_OK;
}

// ------------------------------------------------------------------ shared state, faults

int rar_rank_hashes(void* const* bufs, int nranks, size_t nbytes, void* workspace, size_t ws_bytes,
                    uint64_t* hashes, void* stream) {
  if (nranks < 1 || nranks > RAR_MAX_RANKS || !bufs || !hashes) return RAR_EINVAL;
  if (!workspace || ws_bytes < RAR_HASH_WORKSPACE_BYTES) return RAR_EWORKSPACE;
  if ((uintptr_t)workspace & 15u) return RAR_EALIGN;
  for (int r = 0; r < nranks && nbytes; ++r) {
    if (!bufs[r]) return RAR_EOVERLAP;
    if ((uintptr_t)bufs[r] & 15u) return RAR_EALIGN;
  }
  hipStream_t st = (hipStream_t)stream;
  uint64_t acc[RAR_MAX_RANKS] = {};
  if (nbytes) {
    if (hip_rc(launch_rank_hash(make_ptrs(bufs, nranks), nranks, nbytes, (uint64_t*)workspace, st))) return RAR_EHIP;
    if (hipStreamSynchronize(st) != hipSuccess) return RAR_EHIP;
    if (hipMemcpy(acc, workspace, sizeof(uint64_t) * (size_t)nranks, hipMemcpyDeviceToHost) != hipSuccess)
      return RAR_EHIP;
  }
  for (int r = 0; r < nranks; ++r) hashes[r] = hash_mix64(acc[r] ^ (uint64_t)nbytes);
  return RAR_OK;
}

int rar_shared_state_sync(void* const* bufs, int nranks, size_t nbytes, void* workspace, size_t ws_bytes,
                          int* resent, uint64_t* hashes, void* stream) {
  if (!resent) return RAR_EINVAL;
  int rc = check_bufs(bufs, nranks, RAR_F32, nbytes);  // byte buffers: the element type plays no part
  if (rc) return rc;
  uint64_t h[RAR_MAX_RANKS];
  if ((rc = rar_rank_hashes(bufs, nranks, nbytes, workspace, ws_bytes, h, stream))) return rc;
  if (hashes)
    for (int r = 0; r < nranks; ++r) hashes[r] = h[r];
  int src = 0, best = 0;
  for (int r = 0; r < nranks; ++r) {
    int votes = 0;
    for (int q = 0; q < nranks; ++q) votes += h[q] == h[r];
    if (votes > best) {
      best = votes;
      src = r;
    }
  }
  Traffic tr;
  tr.reset(nranks);
  int moved = 0;
  for (int r = 0; r < nranks; ++r) {
    if (h[r] == h[src]) continue;
    if (hipMemcpyAsync(bufs[r], bufs[src], nbytes, hipMemcpyDeviceToDevice, (hipStream_t)stream) != hipSuccess)
      return RAR_EHIP;
    tr.add(src, r, (uint64_t)nbytes);
    ++moved;
  }
  g_last = tr;
  *resent = moved;
  return RAR_OK;
}

size_t rar_ft_workspace_bytes(int nranks, size_t count, int dtype) {
  if (nranks < 1 || nranks > RAR_MAX_RANKS || !dt_ok(dtype)) return 0;
  return RAR_HASH_WORKSPACE_BYTES + (size_t)nranks * round_up(count * es_of(dtype), kAlign);
}

int rar_ring_allreduce_ft(void* const* bufs, int nranks, size_t count, int dtype, const rar_fault* faults,
                          int nfaults, int deadline_ms, void* workspace, size_t ws_bytes, rar_ft_report* report,
                          void* stream) {
  const size_t es = es_of(dtype);
  int rc = check_bufs(bufs, nranks, dtype, count * es);
  if (rc) return rc;
  if (!report || nfaults < 0 || nfaults > 256 || (nfaults && !faults)) return RAR_EINVAL;
  for (int i = 0; i < nfaults; ++i)
    if (faults[i].rank < 0 || faults[i].rank >= nranks || faults[i].step < 1 || faults[i].stall_ms < 0)
      return RAR_EINVAL;
  if (!workspace || ws_bytes < rar_ft_workspace_bytes(nranks, count, dtype)) return RAR_EWORKSPACE;
  if ((uintptr_t)workspace & 15u) return RAR_EALIGN;
  if ((rc = check_ws_clear(bufs, nullptr, nranks, count * es, 0, workspace,
                           rar_ft_workspace_bytes(nranks, count, dtype))))
    return rc;
  hipStream_t st = (hipStream_t)stream;
  const size_t bytes = count * es, slot = round_up(bytes, kAlign);
  char* snap = (char*)workspace + RAR_HASH_WORKSPACE_BYTES;
  auto copy_all = [&](bool to_snapshot) -> int {
    for (int r = 0; r < nranks && bytes; ++r) {
      void* dst = to_snapshot ? (void*)(snap + (size_t)r * slot) : bufs[r];
      const void* src = to_snapshot ? (const void*)bufs[r] : (const void*)(snap + (size_t)r * slot);
      if (hipMemcpyAsync(dst, src, bytes, hipMemcpyDeviceToDevice, st) != hipSuccess) return RAR_EHIP;
    }
    return RAR_OK;
  };
  if ((rc = copy_all(true))) return rc;
  bool alive[RAR_MAX_RANKS];
  std::vector<char> fired((size_t)nfaults, 0);
  std::memset(report, 0, sizeof *report);
  for (int r = 0; r < nranks; ++r) alive[r] = true;
  Traffic tr;
  tr.reset(nranks);
  int attempt = 0, m = 0, members[RAR_MAX_RANKS];
  for (;;) {
    ++attempt;
    m = 0;
    RankPtrs sub{};
    for (int r = 0; r < nranks; ++r)
      if (alive[r]) {
        sub.p[m] = (char*)bufs[r];
        members[m++] = r;
      }
    if (m == 0) {  // no pass can start
      --attempt;
      break;
    }
    const size_t L = chunk_len_aligned(count, m, 128);
    bool aborted = false;
    for (int g = 1; g <= 2 * (m - 1); ++g) {
      // liveness check of the members before step g
      long long wait = 0;
      for (int i = 0; i < nfaults; ++i) {
        if (fired[(size_t)i] || faults[i].step != g) continue;
        fired[(size_t)i] = 1;
        const int k = faults[i].rank, stall = faults[i].stall_ms;
        if (!alive[k]) continue;
        if (stall > 0 && (deadline_ms <= 0 || stall <= deadline_ms)) {  // answers again in time
          wait = std::max<long long>(wait, stall);
          continue;
        }
        if (stall > 0) wait = std::max<long long>(wait, deadline_ms);
        alive[k] = false;
        report->dead_attempt[k] = attempt;
        report->dead_step[k] = g;
        report->dead_reason[k] = stall > 0 ? RAR_FT_DEADLINE : RAR_FT_GONE;
        aborted = true;
      }
      if (wait > 0) {
        std::this_thread::sleep_for(std::chrono::milliseconds(wait));
        report->waited_ms += wait;
      }
      if (aborted) break;
      const bool rs = g <= m - 1;
      const int s = rs ? g : g - (m - 1);
      for (int j = 0; j < m; ++j) {  // member j sends chunk (j-s) (RS) or (j-s+1) (AG) to member j+1
        size_t lo, hi;
        chunk_range(count, L, modn(rs ? j - s : j - s + 1, m), &lo, &hi);
        tr.add(members[j], members[(j + 1) % m], (uint64_t)(hi - lo) * es);
      }
      if (count == 0) continue;
      if ((rc = rs ? run_rs_step(sub, m, count, L, dtype, s, st) : run_ag_step(sub, m, count, L, es, s, st)))
        return rc;
    }
    if (!aborted) break;
    if ((rc = copy_all(false))) return rc;
  }
  g_last = tr;
  report->attempts = attempt;
  report->nsurvivors = m;
  for (int j = 0; j < m; ++j) report->survivors[j] = members[j];
  if ((rc = rar_rank_hashes(bufs, nranks, bytes, workspace, ws_bytes, report->hash, stream))) return rc;
  return m == 0 ? RAR_EABORT : RAR_OK;
}

// ------------------------------------------------------------------ bucketing

size_t rar_bucket_plan(const size_t* counts, size_t ntensors, int dtype, size_t cap_bytes, int* bucket_of) {
  if (!dt_ok(dtype) || (ntensors && (!counts || !bucket_of))) return 0;
  const size_t es = es_of(dtype);
  size_t nb = 0, cur = 0;
  bool open = false;
  for (size_t t = 0; t < ntensors; ++t) {
    const size_t b = counts[t] * es;
    if (b > cap_bytes) {  // an oversize tensor travels alone
      if (open) ++nb;
      bucket_of[t] = (int)nb++;
      open = false;
      cur = 0;
      continue;
    }
    if (open && cur + b > cap_bytes) {
      ++nb;
      open = false;
      cur = 0;
    }
    bucket_of[t] = (int)nb;
    cur += b;
    open = true;
  }
  return nb + (open ? 1 : 0);
}

static size_t padded_elems(size_t count, size_t es) { return round_up(count * es, 16) / es; }

static size_t bucket_flat_bytes(const size_t* counts, size_t nt, int dtype, size_t cap, std::vector<int>& plan,
                                size_t* nb_out) {
  const size_t es = es_of(dtype);
  plan.assign(nt ? nt : 1, 0);
  const size_t nb = rar_bucket_plan(counts, nt, dtype, cap, plan.data());
  size_t maxb = 0, cur = 0;
  for (size_t t = 0; t < nt; ++t) {
    if (t > 0 && plan[t] != plan[t - 1]) cur = 0;
    cur += padded_elems(counts[t], es) * es;
    maxb = std::max(maxb, cur);
  }
  *nb_out = nb;
  return round_up(maxb, kAlign);
}

// Zero-copy plan: table words (see bucket_kernels.hip) and the launch grid.
// A run is the elements [a, b) of tensor t that lie in chunk c of its
// bucket; the fold tiles it from a rounded down to kRunAlign.  A bucket
// takes N times its largest chunk's tile count workgroups, in the order
// bucket_desc_kernel gives them (XCD-major when N is a multiple of 8, else
// chunk fastest).
static void bucket_table(const size_t* counts, size_t nt, int n, int dtype, size_t cap, void* const* tensors,
                         std::vector<uint64_t>& tab, uint64_t* grid, Traffic* tr) {
  const size_t es = es_of(dtype);
  std::vector<int> plan(nt ? nt : 1, 0);
  const size_t nb = rar_bucket_plan(counts, nt, dtype, cap, plan.data());
  const uint64_t tile = bucket_fold_tile_elems(dtype);
  struct Run {
    uint64_t t, a, b, before;
  };
  std::vector<Run> runs;
  std::vector<uint64_t> crun((size_t)nb * n + 1, 0), start(nb + 1, 0);
  uint64_t wg = 0;
  size_t t = 0;
  for (size_t bk = 0; bk < nb; ++bk) {
    const size_t t0 = t;
    uint64_t total = 0;
    while (t < nt && plan[t] == (int)bk) total += padded_elems(counts[t++], es);
    const uint64_t L = chunk_len_aligned(total, n, 128);
    std::vector<uint64_t> tiles((size_t)n, 0);  // per chunk, so far
    uint64_t off = 0;
    int cprev = -1;
    for (size_t k = t0; k < t; ++k) {
      const uint64_t end = off + counts[k];
      for (uint64_t pos = off; pos < end;) {
        const uint64_t c = pos / L, stop = std::min<uint64_t>(end, (c + 1) * L);
        while (cprev < (int)c) crun[bk * n + (size_t)++cprev] = runs.size();  // chunks cprev+1 .. c start here
        const uint64_t a = pos - off, b = stop - off;
        runs.push_back(Run{k, a, b, tiles[c]});
        tiles[c] += (b - a / kRunAlign * kRunAlign + tile - 1) / tile;
        pos = stop;
      }
      off += padded_elems(counts[k], es);
    }
    while (cprev < n - 1) crun[bk * n + (size_t)++cprev] = runs.size();
    start[bk] = wg;
    wg += (uint64_t)n * *std::max_element(tiles.begin(), tiles.end());
    if (tr) ring_pass_traffic(*tr, n, total, L, es, 0), ring_pass_traffic(*tr, n, total, L, es, 1);
  }
  start[nb] = wg;
  crun[(size_t)nb * n] = runs.size();
  const size_t nr = runs.size();
  tab.assign(3 + nb + (size_t)nb * n + 4 * nr + (size_t)n * nt, 0);
  tab[0] = nb;
  std::copy(start.begin(), start.end(), tab.begin() + 1);
  std::copy(crun.begin(), crun.end(), tab.begin() + 2 + nb);
  uint64_t* run = &tab[3 + nb + (size_t)nb * n];
  uint64_t* ptr = run + 4 * nr;
  for (size_t j = 0; j < nr; ++j) {
    run[4 * j] = runs[j].t;
    run[4 * j + 1] = runs[j].a;
    run[4 * j + 2] = runs[j].b;
    run[4 * j + 3] = runs[j].before;
  }
  if (tensors)
    for (int r = 0; r < n; ++r)
      for (size_t k = 0; k < nt; ++k) ptr[(size_t)r * nt + k] = (uint64_t)(uintptr_t)tensors[(size_t)r * nt + k];
  *grid = wg;
}

size_t rar_bucketed_workspace_bytes_ex(const size_t* counts, size_t ntensors, int nranks, int dtype,
                                       size_t cap_bytes, int algo) {
  if (nranks < 1 || nranks > RAR_MAX_RANKS || !dt_ok(dtype) || (ntensors && !counts)) return 0;
  if (algo == RAR_ALGO_FUSED) {
    // launch table, then one descriptor per workgroup
    std::vector<uint64_t> tab;
    uint64_t grid = 0;
    bucket_table(counts, ntensors, nranks, dtype, cap_bytes, nullptr, tab, &grid, nullptr);
    return round_up(tab.size() * sizeof(uint64_t), kAlign) +
           round_up((size_t)grid * (size_t)bucket_desc_stride(nranks), kAlign);
  }
  if (algo != RAR_ALGO_STEPWISE) return 0;
  std::vector<int> plan;
  size_t nb = 0;
  const size_t per = bucket_flat_bytes(counts, ntensors, dtype, cap_bytes, plan, &nb);
  return std::max<size_t>((size_t)nranks * per, 16);
}

size_t rar_bucketed_workspace_bytes(const size_t* counts, size_t ntensors, int nranks, int dtype,
                                    size_t cap_bytes) {
  return rar_bucketed_workspace_bytes_ex(counts, ntensors, nranks, dtype, cap_bytes, RAR_ALGO_FUSED);
}

// Pack each bucket into flat per-rank buffers, fused ring allreduce, unpack.
static int bucketed_packed(void* const* tensors, const size_t* counts, size_t ntensors, int nranks, int dtype,
                           size_t cap_bytes, void* workspace, hipStream_t st) {
  const size_t es = es_of(dtype);
  std::vector<int> plan;
  size_t nb = 0;
  const size_t per = bucket_flat_bytes(counts, ntensors, dtype, cap_bytes, plan, &nb);
  Traffic total;
  total.reset(nranks);
  void* flat[RAR_MAX_RANKS];
  for (int r = 0; r < nranks; ++r) flat[r] = (char*)workspace + (size_t)r * per;
  size_t t0 = 0;
  int rc = RAR_OK;
  for (size_t b = 0; b < nb; ++b) {
    size_t t1 = t0, elems = 0;
    std::vector<size_t> off;
    while (t1 < ntensors && plan[t1] == (int)b) {
      off.push_back(elems);
      elems += padded_elems(counts[t1++], es);
    }
    SegJobs jobs{};
    auto flush = [&]() -> int {
      if (!jobs.njobs) return RAR_OK;
      int r2 = hip_rc(launch_seg_copy(jobs, st));
      jobs = SegJobs{};
      return r2;
    };
    for (int r = 0; r < nranks; ++r)
      for (size_t t = t0; t < t1; ++t) {
        jobs.src[jobs.njobs] = (const char*)tensors[(size_t)r * ntensors + t];
        jobs.dst[jobs.njobs] = (char*)flat[r] + off[t - t0] * es;
        jobs.bytes[jobs.njobs] = counts[t] * es;
        jobs.zero_to[jobs.njobs] = padded_elems(counts[t], es) * es;
        if (++jobs.njobs == kMaxRanks && (rc = flush())) return rc;
      }
    if ((rc = flush())) return rc;
    if ((rc = allreduce_impl(flat, nranks, elems, dtype, RAR_ALGO_FUSED, true, st))) return rc;
    for (int r = 0; r < nranks; ++r) {
      total.sent[r] += g_last.sent[r];
      total.recv[r] += g_last.recv[r];
    }
    for (int r = 0; r < nranks; ++r)
      for (size_t t = t0; t < t1; ++t) {
        jobs.src[jobs.njobs] = (const char*)flat[r] + off[t - t0] * es;
        jobs.dst[jobs.njobs] = (char*)tensors[(size_t)r * ntensors + t];
        jobs.bytes[jobs.njobs] = counts[t] * es;
        jobs.zero_to[jobs.njobs] = counts[t] * es;
        if (++jobs.njobs == kMaxRanks && (rc = flush())) return rc;
      }
    if ((rc = flush())) return rc;
    t0 = t1;
  }
  g_last = total;
  return RAR_OK;
}

// Argument checks of the bucketed calls (both algorithms).
static int bucketed_check(void* const* tensors, const size_t* counts, size_t ntensors, int nranks, int dtype,
                          size_t cap_bytes, int algo, void* workspace, size_t ws_bytes) {
  if (nranks < 1 || nranks > RAR_MAX_RANKS) return RAR_EINVAL;
  if (!dt_ok(dtype)) return RAR_EDTYPE;
  if (algo != RAR_ALGO_FUSED && algo != RAR_ALGO_STEPWISE) return RAR_EINVAL;
  if (ntensors && (!tensors || !counts)) return RAR_EINVAL;
  const size_t es = es_of(dtype);
  // tensor t of every rank: non-null, aligned, and no two copies overlap
  for (size_t t = 0; t < ntensors; ++t) {
    if (counts[t] == 0) continue;
    std::vector<void*> copies((size_t)nranks);
    for (int r = 0; r < nranks; ++r) copies[(size_t)r] = tensors[(size_t)r * ntensors + t];
    const int rc = check_bufs(copies.data(), nranks, dtype, counts[t] * es);
    if (rc) return rc;
  }
  const size_t need = rar_bucketed_workspace_bytes_ex(counts, ntensors, nranks, dtype, cap_bytes, algo);
  if (!workspace || ws_bytes < need) return RAR_EWORKSPACE;
  if ((uintptr_t)workspace & 15u) return RAR_EALIGN;
  // every tensor of every rank and the workspace: pairwise disjoint
  std::vector<std::pair<uintptr_t, size_t>> a;
  a.reserve((size_t)nranks * ntensors + 1);
  for (int r = 0; r < nranks; ++r)
    for (size_t t = 0; t < ntensors; ++t) a.emplace_back((uintptr_t)tensors[(size_t)r * ntensors + t], counts[t] * es);
  a.emplace_back((uintptr_t)workspace, need);
  return check_disjoint(a);
}

int rar_bucketed_prepare(void* const* tensors, const size_t* counts, size_t ntensors, int nranks, int dtype,
                         size_t cap_bytes, void* workspace, size_t ws_bytes, rar_bucketed_plan* plan,
                         void* stream) {
  if (!plan) return RAR_EINVAL;
  int rc = bucketed_check(tensors, counts, ntensors, nranks, dtype, cap_bytes, RAR_ALGO_FUSED, workspace, ws_bytes);
  if (rc) return rc;
  hipStream_t st = (hipStream_t)stream;
  std::vector<uint64_t> tab;
  uint64_t grid = 0;
  Traffic tr;
  tr.reset(nranks);
  bucket_table(counts, ntensors, nranks, dtype, cap_bytes, tensors, tab, &grid, &tr);
  rar_bucketed_plan p{};
  p.workspace = workspace;
  p.desc_offset = round_up(tab.size() * sizeof(uint64_t), kAlign);
  p.grid = nranks == 1 ? 0 : grid;  // one rank: nothing to reduce
  p.ntensors = ntensors;
  p.nranks = nranks;
  p.dtype = dtype;
  for (int r = 0; r < nranks; ++r) {
    p.sent[r] = tr.sent[r];
    p.recv[r] = tr.recv[r];
  }
  if (p.grid) {
    if ((rc = hip_rc(launch_fill_u64((uint64_t*)workspace, tab.data(), (int)tab.size(), st)))) return rc;
    char* desc = (char*)workspace + p.desc_offset;
    if ((rc = hip_rc(launch_bucket_desc((const uint64_t*)workspace, desc, nranks, ntensors, grid, dtype, st))))
      return rc;
  }
  *plan = p;
  return RAR_OK;
}

int rar_bucketed_launch(const rar_bucketed_plan* plan, void* stream) {
  if (!plan || plan->nranks < 1 || plan->nranks > RAR_MAX_RANKS || !dt_ok(plan->dtype)) return RAR_EINVAL;
  if (plan->grid && (!plan->workspace || ((uintptr_t)plan->workspace & 15u) || (plan->desc_offset & 15u) ||
                     plan->desc_offset == 0))
    return RAR_EINVAL;
  g_last.reset(plan->nranks);
  for (int r = 0; r < plan->nranks; ++r) {
    g_last.sent[r] = plan->sent[r];
    g_last.recv[r] = plan->recv[r];
  }
  if (plan->grid == 0) return RAR_OK;
  const char* desc = (const char*)plan->workspace + plan->desc_offset;
  return hip_rc(launch_bucket_fold(desc, plan->nranks, plan->grid, plan->dtype, (hipStream_t)stream));
}

int rar_bucketed_allreduce_ex(void* const* tensors, const size_t* counts, size_t ntensors, int nranks,
                              int dtype, size_t cap_bytes, int algo, void* workspace, size_t ws_bytes,
                              void* stream) {
  if (algo == RAR_ALGO_STEPWISE) {
    const int rc = bucketed_check(tensors, counts, ntensors, nranks, dtype, cap_bytes, algo, workspace, ws_bytes);
    if (rc) return rc;
    return bucketed_packed(tensors, counts, ntensors, nranks, dtype, cap_bytes, workspace, (hipStream_t)stream);
  }
  if (algo != RAR_ALGO_FUSED) return RAR_EINVAL;
  rar_bucketed_plan plan;
  const int rc = rar_bucketed_prepare(tensors, counts, ntensors, nranks, dtype, cap_bytes, workspace, ws_bytes,
                                      &plan, stream);
  if (rc) return rc;
  return rar_bucketed_launch(&plan, stream);
}

int rar_bucketed_allreduce(void* const* tensors, const size_t* counts, size_t ntensors, int nranks, int dtype,
                           size_t cap_bytes, void* workspace, size_t ws_bytes, void* stream) {
  return rar_bucketed_allreduce_ex(tensors, counts, ntensors, nranks, dtype, cap_bytes, RAR_ALGO_FUSED, workspace,
                                   ws_bytes, stream);
}

// ------------------------------------------------------------------ misc

const char* rar_status_string(int status) {
  switch (status) {
    case RAR_OK: return "ok";
    case RAR_EINVAL: return "invalid argument";
    case RAR_EDTYPE: return "unsupported element type";
    case RAR_EALIGN: return "device pointer not 16-byte aligned";
    case RAR_EWORKSPACE: return "workspace missing or too small";
    case RAR_EHIP: return "HIP runtime error";
    case RAR_ENOTSUP: return "not supported";
    case RAR_EOVERLAP: return "rank buffers overlap or are NULL";
    case RAR_EABORT: return "ring aborted: every member failed";
    default: return "unknown status";
  }
}

const char* rar_version(void) { return "rar 0.1.0 (gfx950)"; }

}  // extern "C"
