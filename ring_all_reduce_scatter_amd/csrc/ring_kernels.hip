// Uncompressed ring kernels for gfx950.
//
// Ring schedule (page "从零实现集合通信", two-pass ring allreduce section):
// at reduce-scatter step s rank r receives chunk (r-s-1) mod N from rank
// r-1 and adds it to its own copy; after N-1 steps rank r holds chunk r's
// full sum; N-1 allgather rotations then give every rank the whole result.
//
// On one GPU all N rank buffers sit in the same HBM, so a "receive" is a load
// from the neighbour's buffer.  Two schedules:
//  * rs_step / copy_jobs: one launch per ring step, each materialising the
//    step for all N ranks (what the ring's messages would leave behind);
//  * ring_fold: the whole allreduce in one launch.  A workgroup owns a tile
//    of one chunk c; it loads that tile from all N ranks (16-byte vector
//    loads, all issued before the adds), folds them in registers in the
//    order the reduce-scatter steps produce (ranks c+1, c+2, ..., c+N-1, c),
//    and stores the sum to every rank.  HBM traffic is the minimum: N*S read,
//    N*S written.
#include "launch.hpp"

namespace rar {

namespace {

constexpr int kFoldGroups = 2;  // 8-element groups per thread in ring_fold
constexpr int kStepGroups = 2;  // ... in rs_step
constexpr int kCopyVecs = 4;    // 16-byte vectors per thread in copy_jobs

template <int DT, int NR, int G, bool STORE_ALL>
__global__ __launch_bounds__(kThreads) void ring_fold_kernel(RankPtrs bufs, int nranks,
                                                              uint64_t count, uint64_t L,
                                                              uint32_t tiles_per_chunk) {
  const int N = NR > 0 ? NR : nranks;
  const uint32_t c = blockIdx.x / tiles_per_chunk;
  const uint32_t t = blockIdx.x - c * tiles_per_chunk;
  const uint64_t lo = (uint64_t)c * L;
  if (lo >= count) return;
  const uint64_t hi = lo + L < count ? lo + L : count;
  constexpr uint64_t kTile = (uint64_t)kThreads * kGroupElems * G;
  const uint64_t tile0 = lo + (uint64_t)t * kTile;
  if (tile0 >= hi) return;
  const uint64_t e0 = tile0 + (uint64_t)threadIdx.x * kGroupElems;
  const int first = (int)c + 1 < N ? (int)c + 1 : 0;

  if (tile0 + kTile <= hi) {
    // Full tile: vector loads, fold in ring order in registers.
    G8 acc[G];
#pragma unroll
    for (int g = 0; g < G; ++g)
      acc[g] = unpack8<DT>(load_raw8<DT, true>(bufs.p[first], e0 + (uint64_t)g * kThreads * kGroupElems));
    int r = first;
    auto hop = [&]() {
      r = r + 1 == N ? 0 : r + 1;
#pragma unroll
      for (int g = 0; g < G; ++g) {
        G8 x = unpack8<DT>(load_raw8<DT, true>(bufs.p[r], e0 + (uint64_t)g * kThreads * kGroupElems));
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[g].v[i] = round_to<DT>(x.v[i] + acc[g].v[i]);
      }
    };
    if constexpr (NR > 0) {
#pragma unroll
      for (int k = 2; k <= NR; ++k) hop();
    } else {
      for (int k = 2; k <= N; ++k) hop();
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      Raw8<DT> out = pack8<DT>(acc[g]);
      const uint64_t e = e0 + (uint64_t)g * kThreads * kGroupElems;
      if constexpr (STORE_ALL) {
        for (int d = 0; d < N; ++d) store_raw8<DT, true>(bufs.p[d], e, out);
      } else {
        store_raw8<DT, true>(bufs.p[c], e, out);
      }
    }
    return;
  }

  // Ragged tile (only the last tile of the last non-empty chunk).
  for (int g = 0; g < G; ++g) {
    const uint64_t e = e0 + (uint64_t)g * kThreads * kGroupElems;
    if (e >= hi) break;
    const int nv = hi - e >= 8 ? 8 : (int)(hi - e);
    G8 acc = load_part8<DT>(bufs.p[first], e, nv);
    int r = first;
    for (int k = 2; k <= N; ++k) {
      r = r + 1 == N ? 0 : r + 1;
      G8 x = load_part8<DT>(bufs.p[r], e, nv);
      for (int i = 0; i < 8; ++i) acc.v[i] = round_to<DT>(x.v[i] + acc.v[i]);
    }
    if constexpr (STORE_ALL) {
      for (int d = 0; d < N; ++d) store_part8<DT>(bufs.p[d], e, nv, acc);
    } else {
      store_part8<DT>(bufs.p[c], e, nv, acc);
    }
  }
}

template <int DT, int G>
__global__ __launch_bounds__(kThreads) void rs_step_kernel(RankPtrs bufs, int N, uint64_t count,
                                                            uint64_t L, int s,
                                                            uint32_t tiles_per_chunk) {
  const int r = (int)(blockIdx.x / tiles_per_chunk);
  const uint32_t t = blockIdx.x - (uint32_t)r * tiles_per_chunk;
  const int c = ((r - s - 1) % N + N) % N;
  const int src = r == 0 ? N - 1 : r - 1;
  const uint64_t lo = (uint64_t)c * L;
  if (lo >= count) return;
  const uint64_t hi = lo + L < count ? lo + L : count;
  constexpr uint64_t kTile = (uint64_t)kThreads * kGroupElems * G;
  const uint64_t tile0 = lo + (uint64_t)t * kTile;
  if (tile0 >= hi) return;
  const uint64_t e0 = tile0 + (uint64_t)threadIdx.x * kGroupElems;
  if (tile0 + kTile <= hi) {
    Raw8<DT> mine[G], theirs[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const uint64_t e = e0 + (uint64_t)g * kThreads * kGroupElems;
      mine[g] = load_raw8<DT, false>(bufs.p[r], e);
      theirs[g] = load_raw8<DT, true>(bufs.p[src], e);
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      G8 a = unpack8<DT>(mine[g]), b = unpack8<DT>(theirs[g]);
#pragma unroll
      for (int i = 0; i < 8; ++i) a.v[i] = round_to<DT>(a.v[i] + b.v[i]);
      store_raw8<DT, false>(bufs.p[r], e0 + (uint64_t)g * kThreads * kGroupElems, pack8<DT>(a));
    }
    return;
  }
  for (int g = 0; g < G; ++g) {
    const uint64_t e = e0 + (uint64_t)g * kThreads * kGroupElems;
    if (e >= hi) break;
    const int nv = hi - e >= 8 ? 8 : (int)(hi - e);
    G8 a = load_part8<DT>(bufs.p[r], e, nv), b = load_part8<DT>(bufs.p[src], e, nv);
    for (int i = 0; i < 8; ++i) a.v[i] = round_to<DT>(a.v[i] + b.v[i]);
    store_part8<DT>(bufs.p[r], e, nv, a);
  }
}

// Copy jobs: job j copies bytes [lo, lo+len) of rank src[j] to the same range
// of every rank in dstmask[j].  The 16-byte aligned middle is tiled over the
// job's workgroups; the unaligned head and tail (2-byte units) are done by
// the job's first workgroup.
__global__ __launch_bounds__(kThreads) void copy_jobs_kernel(CopyJobs jobs, uint32_t tiles_per_job) {
  const int j = (int)(blockIdx.x / tiles_per_job);
  const uint32_t t = blockIdx.x - (uint32_t)j * tiles_per_job;
  const uint64_t lo = jobs.lo[j], end = lo + jobs.len[j];
  const uint64_t alo = (lo + 15) / 16 * 16 < end ? (lo + 15) / 16 * 16 : end;
  const uint64_t ahi = end / 16 * 16 > alo ? end / 16 * 16 : alo;
  const char* src = jobs.ptrs.p[jobs.src[j]];
  const uint64_t mask = jobs.dstmask[j];
  if (t == 0 && threadIdx.x < 16) {
    // head [lo, alo) and tail [ahi, end): at most 7 two-byte units each
    const uint64_t off = threadIdx.x < 8 ? lo + 2 * threadIdx.x : ahi + 2 * (threadIdx.x - 8);
    const uint64_t lim = threadIdx.x < 8 ? alo : end;
    if (off < lim) {
      uint16_t v = *(const uint16_t*)(src + off);
      for (uint64_t m = mask; m; m &= m - 1) *(uint16_t*)(jobs.ptrs.p[__builtin_ctzll(m)] + off) = v;
    }
  }
  constexpr uint64_t kTileBytes = (uint64_t)kThreads * 16 * kCopyVecs;
  const uint64_t b0 = alo + (uint64_t)t * kTileBytes + (uint64_t)threadIdx.x * 16;
  u32x4 v[kCopyVecs];
  bool ok[kCopyVecs];
#pragma unroll
  for (int i = 0; i < kCopyVecs; ++i) {
    const uint64_t b = b0 + (uint64_t)i * kThreads * 16;
    ok[i] = b + 16 <= ahi;
    if (ok[i]) v[i] = ld16<true>(src + b);
  }
  for (uint64_t m = mask; m; m &= m - 1) {
    char* dst = jobs.ptrs.p[__builtin_ctzll(m)];
#pragma unroll
    for (int i = 0; i < kCopyVecs; ++i)
      if (ok[i]) st16<true>(dst + b0 + (uint64_t)i * kThreads * 16, v[i]);
  }
}

template <int DT, int NR>
hipError_t fold_dispatch_store(const RankPtrs& bufs, int n, uint64_t count, uint64_t L,
                               bool store_all, uint32_t tiles, hipStream_t stream) {
  dim3 grid((unsigned)((uint64_t)n * tiles)), block(kThreads);
  if (store_all)
    hipLaunchKernelGGL((ring_fold_kernel<DT, NR, kFoldGroups, true>), grid, block, 0, stream, bufs, n,
                       count, L, tiles);
  else
    hipLaunchKernelGGL((ring_fold_kernel<DT, NR, kFoldGroups, false>), grid, block, 0, stream, bufs, n,
                       count, L, tiles);
  return hipGetLastError();
}

template <int DT>
hipError_t fold_dispatch_n(const RankPtrs& bufs, int n, uint64_t count, uint64_t L, bool store_all,
                           uint32_t tiles, hipStream_t stream) {
  switch (n) {
    case 2: return fold_dispatch_store<DT, 2>(bufs, n, count, L, store_all, tiles, stream);
    case 4: return fold_dispatch_store<DT, 4>(bufs, n, count, L, store_all, tiles, stream);
    case 8: return fold_dispatch_store<DT, 8>(bufs, n, count, L, store_all, tiles, stream);
    case 16: return fold_dispatch_store<DT, 16>(bufs, n, count, L, store_all, tiles, stream);
    default: return fold_dispatch_store<DT, 0>(bufs, n, count, L, store_all, tiles, stream);
  }
}

}  // namespace

hipError_t launch_ring_fold(const RankPtrs& bufs, int n, uint64_t count, uint64_t L, int dt,
                            bool store_all, hipStream_t stream) {
  const uint64_t tile = (uint64_t)kThreads * kGroupElems * kFoldGroups;
  const uint32_t tiles = (uint32_t)((L + tile - 1) / tile);
  if (tiles == 0) return hipSuccess;
  switch (dt) {
    case DT_F32: return fold_dispatch_n<DT_F32>(bufs, n, count, L, store_all, tiles, stream);
    case DT_F16: return fold_dispatch_n<DT_F16>(bufs, n, count, L, store_all, tiles, stream);
    default: return fold_dispatch_n<DT_BF16>(bufs, n, count, L, store_all, tiles, stream);
  }
}

hipError_t launch_rs_step(const RankPtrs& bufs, int n, uint64_t count, uint64_t L, int dt, int s,
                          hipStream_t stream) {
  const uint64_t tile = (uint64_t)kThreads * kGroupElems * kStepGroups;
  const uint32_t tiles = (uint32_t)((L + tile - 1) / tile);
  if (tiles == 0) return hipSuccess;
  dim3 grid((unsigned)((uint64_t)n * tiles)), block(kThreads);
  switch (dt) {
    case DT_F32:
      hipLaunchKernelGGL((rs_step_kernel<DT_F32, kStepGroups>), grid, block, 0, stream, bufs, n, count, L, s, tiles);
      break;
    case DT_F16:
      hipLaunchKernelGGL((rs_step_kernel<DT_F16, kStepGroups>), grid, block, 0, stream, bufs, n, count, L, s, tiles);
      break;
    default:
      hipLaunchKernelGGL((rs_step_kernel<DT_BF16, kStepGroups>), grid, block, 0, stream, bufs, n, count, L, s, tiles);
      break;
  }
  return hipGetLastError();
}

hipError_t launch_copy_jobs(const CopyJobs& jobs, hipStream_t stream) {
  uint64_t maxlen = 0;
  for (int j = 0; j < jobs.njobs; ++j) maxlen = jobs.len[j] > maxlen ? jobs.len[j] : maxlen;
  if (jobs.njobs == 0 || maxlen == 0) return hipSuccess;
  const uint64_t tile = (uint64_t)kThreads * 16 * kCopyVecs;
  const uint32_t tiles = (uint32_t)((maxlen + tile - 1) / tile);
  dim3 grid((unsigned)((uint64_t)jobs.njobs * tiles)), block(kThreads);
  hipLaunchKernelGGL(copy_jobs_kernel, grid, block, 0, stream, jobs, tiles);
  return hipGetLastError();
}

}  // namespace rar
