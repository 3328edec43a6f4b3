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
#include <atomic>

#include <cstdlib>
#include <cstring>

#include "launch.hpp"

namespace rar {

namespace {

// 16-byte vectors per thread and workgroups per CU of the fused fold, tuned
// for N = 8 on MI355X (about 64 KiB of loads in flight per CU).  bf16 spends
// more ALU per byte on its software rounding, so it keeps one vector per rank
// and more workgroups per CU to hide that latency (fold_wgs_per_cu).
template <int DT>
struct FoldVecs {
  static constexpr int value = DT == DT_BF16 ? 1 : 2;
};
constexpr int kStepVecs = 4;  // ... in rs_step
constexpr int kCopyVecs = 4;  // ... in copy_jobs

// Workgroup -> (chunk, tile) with the chunk fastest: workgroups resident at
// the same time cover every chunk (and the ring rotation of every chunk).
// Workgroup w goes to XCD w mod 8, so at N = 8 each XCD streams one chunk;
// rank counts prime to 8 spread each chunk over all XCDs alike.
__device__ __forceinline__ void chunk_tile(int N, uint32_t* c, uint32_t* t) {
  *c = blockIdx.x % (uint32_t)N;
  *t = blockIdx.x / (uint32_t)N;
}

// Workgroup -> (chunk, tile) for the fused fold: K consecutive workgroups
// take K consecutive tiles of one chunk, then the next chunk (K = 1 is
// chunk_tile's order; K = the tiles per chunk makes tiles fastest).  The
// grid covers tiles rounded up to a multiple of K; the extra workgroups
// find their tile past the chunk's end and return.
__device__ __forceinline__ void chunk_tile_k(int N, uint32_t K, uint32_t* c, uint32_t* t) {
  const uint32_t b = blockIdx.x;
  *c = (b / K) % (uint32_t)N;
  *t = (b / (K * (uint32_t)N)) * K + b % K;
}

template <int DT, int NR, int V, bool STORE_ALL>
__global__ __launch_bounds__(kThreads) void ring_fold_kernel(RankPtrs bufs, int nranks,
                                                              uint64_t count, uint64_t L, uint32_t K) {
  constexpr int E = Vec<DT>::E;
  constexpr int ES = DtypeSize<DT>::value;
  const int N = NR > 0 ? NR : nranks;
  uint32_t c, t;
  chunk_tile_k(N, K, &c, &t);
  const uint64_t lo = (uint64_t)c * L;
  if (lo >= count) return;
  const uint64_t hi = lo + L < count ? lo + L : count;
  constexpr uint64_t kTile = (uint64_t)kThreads * E * V;
  const uint64_t tile0 = lo + (uint64_t)t * kTile;
  if (tile0 >= hi) return;
  const int first = (int)c + 1 < N ? (int)c + 1 : 0;
  auto elem = [&](int v) -> uint64_t { return tile0 + ((uint64_t)v * kThreads + threadIdx.x) * E; };

  if (tile0 + kTile <= hi) {
    // Full tile: every rank's vectors are loaded before the fold, which runs
    // in ring order (ranks c+1, ..., c+N-1, c) in registers.
    Vec<DT> acc[V];
    if constexpr (NR > 0) {
      u32x4 x[NR][V];
      int r = first;
#pragma unroll
      for (int k = 0; k < NR; ++k) {
#pragma unroll
        for (int v = 0; v < V; ++v) x[k][v] = ld16<true>(bufs.p[r] + elem(v) * ES);
        r = r + 1 == NR ? 0 : r + 1;
      }
#pragma unroll
      for (int v = 0; v < V; ++v) {
        acc[v] = unpack16<DT>(x[0][v]);
#pragma unroll
        for (int k = 1; k < NR; ++k) {
          const Vec<DT> y = unpack16<DT>(x[k][v]);
#pragma unroll
          for (int i = 0; i < E; ++i) acc[v].v[i] = round_to<DT>(y.v[i] + acc[v].v[i]);
        }
      }
    } else {
      int r = first;
#pragma unroll
      for (int v = 0; v < V; ++v) acc[v] = unpack16<DT>(ld16<true>(bufs.p[r] + elem(v) * ES));
      for (int k = 1; k < N; ++k) {
        r = r + 1 == N ? 0 : r + 1;
        u32x4 x[V];
#pragma unroll
        for (int v = 0; v < V; ++v) x[v] = ld16<true>(bufs.p[r] + elem(v) * ES);
#pragma unroll
        for (int v = 0; v < V; ++v) {
          const Vec<DT> y = unpack16<DT>(x[v]);
#pragma unroll
          for (int i = 0; i < E; ++i) acc[v].v[i] = round_to<DT>(y.v[i] + acc[v].v[i]);
        }
      }
    }
    // all-reduce: write-through stores over the tile's range in each rank;
    // the reduce-scatter (N reads, one write) keeps plain nontemporal stores
    // (write-through measured 3 % slower there: 0.409 against 0.398 ms)
    constexpr uint32_t kTileBytes = (uint32_t)(kTile * ES);
    auto lane_off = [&](int v) -> uint32_t { return ((uint32_t)v * kThreads + threadIdx.x) * E * ES; };
#pragma unroll
    for (int v = 0; v < V; ++v) {
      const u32x4 out = pack16<DT>(acc[v]);
      if constexpr (STORE_ALL) {
        for (int d = 0; d < N; ++d) st16_wt(wt_range(bufs.p[d] + tile0 * ES, kTileBytes), lane_off(v), out);
      } else {
        st16<true>(bufs.p[c] + elem(v) * ES, out);
      }
    }
    return;
  }

  // Ragged tile (the last tile of a chunk): element by element.
  for (int v = 0; v < V; ++v) {
    const uint64_t e = elem(v);
    for (int i = 0; i < E && e + i < hi; ++i) {
      int r = first;
      float acc = load_elem<DT>(bufs.p[r], e + i);
      for (int k = 1; k < N; ++k) {
        r = r + 1 == N ? 0 : r + 1;
        acc = round_to<DT>(load_elem<DT>(bufs.p[r], e + i) + acc);
      }
      if constexpr (STORE_ALL) {
        for (int d = 0; d < N; ++d) store_elem<DT>(bufs.p[d], e + i, acc);
      } else {
        store_elem<DT>(bufs.p[c], e + i, acc);
      }
    }
  }
}

template <int DT, int V>
__global__ __launch_bounds__(kThreads) void rs_step_kernel(RankPtrs bufs, int N, uint64_t count,
                                                            uint64_t L, int s) {
  constexpr int E = Vec<DT>::E;
  constexpr int ES = DtypeSize<DT>::value;
  uint32_t r_, t;
  chunk_tile(N, &r_, &t);
  const int r = (int)r_;
  const int c = ((r - s - 1) % N + N) % N;
  const int src = r == 0 ? N - 1 : r - 1;
  const uint64_t lo = (uint64_t)c * L;
  if (lo >= count) return;
  const uint64_t hi = lo + L < count ? lo + L : count;
  constexpr uint64_t kTile = (uint64_t)kThreads * E * V;
  const uint64_t tile0 = lo + (uint64_t)t * kTile;
  if (tile0 >= hi) return;
  auto elem = [&](int v) -> uint64_t { return tile0 + ((uint64_t)v * kThreads + threadIdx.x) * E; };
  if (tile0 + kTile <= hi) {
    u32x4 mine[V], theirs[V];
#pragma unroll
    for (int v = 0; v < V; ++v) {
      mine[v] = ld16<false>(bufs.p[r] + elem(v) * ES);
      theirs[v] = ld16<true>(bufs.p[src] + elem(v) * ES);
    }
#pragma unroll
    for (int v = 0; v < V; ++v) {
      Vec<DT> a = unpack16<DT>(mine[v]);
      const Vec<DT> b = unpack16<DT>(theirs[v]);
#pragma unroll
      for (int i = 0; i < E; ++i) a.v[i] = round_to<DT>(a.v[i] + b.v[i]);
      st16<false>(bufs.p[r] + elem(v) * ES, pack16<DT>(a));
    }
    return;
  }
  for (int v = 0; v < V; ++v) {
    const uint64_t e = elem(v);
    for (int i = 0; i < E && e + i < hi; ++i)
      store_elem<DT>(bufs.p[r], e + i, round_to<DT>(load_elem<DT>(bufs.p[r], e + i) + load_elem<DT>(bufs.p[src], e + i)));
  }
}

// ---------------------------------------------------------------- tree allreduce
// Binomial tree (page "从零实现集合通信", ring-vs-tree table: depth log2 N):
// in the reduce round with distance span, rank rel (rel % 2span == 0,
// rel + span < N) adds rank rel+span into its own copy; rank 0 ends with
// the sum, which the binomial broadcast then gives to every rank.  The fused
// kernel applies the same rounds to all N ranks' vectors in registers and
// stores rank 0's result to every rank.
//
// Workgroup -> tile: the launch has kRegions * per workgroups, and workgroup b
// takes tile (b % kRegions) * per + b / kRegions, so the workgroups dealt to
// one XCD (b % 8) stream one contiguous region of every rank, as the ring
// fold's chunk-fastest order does.  The reduction order does not depend on
// the mapping.
constexpr uint32_t kRegions = 8;

template <int DT, int NR, int V>
__global__ __launch_bounds__(kThreads) void tree_fold_kernel(RankPtrs bufs, uint64_t count, uint32_t per) {
  constexpr int E = Vec<DT>::E;
  constexpr int ES = DtypeSize<DT>::value;
  constexpr uint64_t kTile = (uint64_t)kThreads * E * V;
  const uint32_t region = blockIdx.x % kRegions;
  const uint64_t tile0 = ((uint64_t)region * per + blockIdx.x / kRegions) * kTile;
  if (tile0 >= count) return;
  auto elem = [&](int v) -> uint64_t { return tile0 + ((uint64_t)v * kThreads + threadIdx.x) * E; };
  if (tile0 + kTile <= count) {
    Vec<DT> x[NR][V];
#pragma unroll
    for (int r = 0; r < NR; ++r)
#pragma unroll
      for (int v = 0; v < V; ++v) x[r][v] = unpack16<DT>(ld16<true>(bufs.p[r] + elem(v) * ES));
#pragma unroll
    for (int span = 1; span < NR; span *= 2)
#pragma unroll
      for (int rel = 0; rel + span < NR; rel += 2 * span)
#pragma unroll
        for (int v = 0; v < V; ++v)
#pragma unroll
          for (int i = 0; i < E; ++i) x[rel][v].v[i] = round_to<DT>(x[rel][v].v[i] + x[rel + span][v].v[i]);
    // write-through stores over the tile's range in each rank
#pragma unroll
    for (int v = 0; v < V; ++v) {
      const u32x4 out = pack16<DT>(x[0][v]);
      const uint32_t off = ((uint32_t)v * kThreads + threadIdx.x) * E * ES;
      for (int d = 0; d < NR; ++d) st16_wt(wt_range(bufs.p[d] + tile0 * ES, (uint32_t)(kTile * ES)), off, out);
    }
    return;
  }
  for (int v = 0; v < V; ++v) {
    const uint64_t e = elem(v);
    for (int i = 0; i < E && e + i < count; ++i) {
      float x[NR];
#pragma unroll
      for (int r = 0; r < NR; ++r) x[r] = load_elem<DT>(bufs.p[r], e + i);
#pragma unroll
      for (int span = 1; span < NR; span *= 2)
#pragma unroll
        for (int rel = 0; rel + span < NR; rel += 2 * span) x[rel] = round_to<DT>(x[rel] + x[rel + span]);
      for (int d = 0; d < NR; ++d) store_elem<DT>(bufs.p[d], e + i, x[0]);
    }
  }
}

// One stepwise reduce round: pair j adds rank src[j]'s whole buffer into rank dst[j].
template <int DT, int V>
__global__ __launch_bounds__(kThreads) void pair_add_kernel(RankPtrs bufs, PairJobs pairs, uint64_t count,
                                                             uint32_t tiles) {
  constexpr int E = Vec<DT>::E;
  constexpr int ES = DtypeSize<DT>::value;
  const int j = (int)(blockIdx.x % (uint32_t)pairs.npairs);
  const uint64_t t = blockIdx.x / (uint32_t)pairs.npairs;
  const char* src = bufs.p[pairs.src[j]];
  char* dst = bufs.p[pairs.dst[j]];
  constexpr uint64_t kTile = (uint64_t)kThreads * E * V;
  const uint64_t tile0 = t * kTile;
  if (tile0 >= count) return;
  auto elem = [&](int v) -> uint64_t { return tile0 + ((uint64_t)v * kThreads + threadIdx.x) * E; };
  if (tile0 + kTile <= count) {
    u32x4 a[V], b[V];
#pragma unroll
    for (int v = 0; v < V; ++v) {
      a[v] = ld16<false>(dst + elem(v) * ES);
      b[v] = ld16<true>(src + elem(v) * ES);
    }
#pragma unroll
    for (int v = 0; v < V; ++v) {
      Vec<DT> x = unpack16<DT>(a[v]);
      const Vec<DT> y = unpack16<DT>(b[v]);
#pragma unroll
      for (int i = 0; i < E; ++i) x.v[i] = round_to<DT>(x.v[i] + y.v[i]);
      st16<false>(dst + elem(v) * ES, pack16<DT>(x));
    }
    return;
  }
  for (int v = 0; v < V; ++v) {
    const uint64_t e = elem(v);
    for (int i = 0; i < E && e + i < count; ++i)
      store_elem<DT>(dst, e + i, round_to<DT>(load_elem<DT>(dst, e + i) + load_elem<DT>(src, e + i)));
  }
  (void)tiles;
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
  // A one-to-one copy stores write-through over the tile's range (2 GiB:
  // 0.696 against 0.70-0.71 ms); a fan-out keeps plain nontemporal stores
  // (write-through measured slower there: broadcast 0.116 against 0.110 ms,
  // allgather 0.821 against 0.775 ms)
  if (__builtin_popcountll(mask) == 1) {  // uniform
    const uint64_t tb = alo + (uint64_t)t * kTileBytes;  // the tile's first byte
    const WtRange rg = wt_range(jobs.ptrs.p[__builtin_ctzll(mask)] + tb, (uint32_t)kTileBytes);
#pragma unroll
    for (int i = 0; i < kCopyVecs; ++i)
      if (ok[i]) st16_wt(rg, (uint32_t)(b0 - tb + (uint64_t)i * kThreads * 16), v[i]);
    return;
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
                               bool store_all, hipStream_t stream) {
  constexpr int V = FoldVecs<DT>::value;
  const uint64_t tile = (uint64_t)kThreads * Vec<DT>::E * V;
  const uint64_t tiles = (L + tile - 1) / tile;
  const uint64_t K = fold_tile_group(DT, n, tiles);
  const uint64_t ktiles = (tiles + K - 1) / K * K;
  dim3 grid((unsigned)((uint64_t)n * ktiles)), block(kThreads);
  const size_t lds = residency_lds(fold_wgs_per_cu(DT, n));
  if (store_all)
    hipLaunchKernelGGL((ring_fold_kernel<DT, NR, V, true>), grid, block, lds, stream, bufs, n, count, L,
                       (uint32_t)K);
  else
    hipLaunchKernelGGL((ring_fold_kernel<DT, NR, V, false>), grid, block, lds, stream, bufs, n, count, L,
                       (uint32_t)K);
  return launch_status(stream);
}

template <int DT>
hipError_t fold_dispatch_n(const RankPtrs& bufs, int n, uint64_t count, uint64_t L, bool store_all,
                           hipStream_t stream) {
  switch (n) {
    case 2: return fold_dispatch_store<DT, 2>(bufs, n, count, L, store_all, stream);
    case 4: return fold_dispatch_store<DT, 4>(bufs, n, count, L, store_all, stream);
    case 8: return fold_dispatch_store<DT, 8>(bufs, n, count, L, store_all, stream);
    case 16: return fold_dispatch_store<DT, 16>(bufs, n, count, L, store_all, stream);
    default: return fold_dispatch_store<DT, 0>(bufs, n, count, L, store_all, stream);
  }
}

template <int DT>
hipError_t step_dispatch(const RankPtrs& bufs, int n, uint64_t count, uint64_t L, int s, hipStream_t stream) {
  const uint64_t tile = (uint64_t)kThreads * Vec<DT>::E * kStepVecs;
  const uint64_t tiles = (L + tile - 1) / tile;
  dim3 grid((unsigned)((uint64_t)n * tiles)), block(kThreads);
  hipLaunchKernelGGL((rs_step_kernel<DT, kStepVecs>), grid, block, 0, stream, bufs, n, count, L, s);
  return launch_status(stream);
}

template <int DT, int NR>
hipError_t tree_dispatch_v(const RankPtrs& bufs, uint64_t count, hipStream_t stream) {
  constexpr int V = DT == DT_BF16 ? 1 : 2;
  const uint64_t tile = (uint64_t)kThreads * Vec<DT>::E * V;
  const uint64_t tiles = (count + tile - 1) / tile;
  const uint64_t per = (tiles + kRegions - 1) / kRegions;
  // the ring fold's residency table, except bf16 at 8 ranks: the tree's
  // shorter add chain runs best at two workgroups per CU (709-715 us for
  // 8 x 128M against 747 at three)
  const int wgs = DT == DT_BF16 && NR == 8 ? 2 : fold_wgs_per_cu(DT, NR);
  hipLaunchKernelGGL((tree_fold_kernel<DT, NR, V>), dim3((unsigned)(per * kRegions)), dim3(kThreads),
                     residency_lds(wgs), stream, bufs, count, (uint32_t)per);
  return launch_status(stream);
}

template <int DT>
hipError_t tree_dispatch_n(const RankPtrs& bufs, int n, uint64_t count, hipStream_t stream) {
  switch (n) {
    case 2: return tree_dispatch_v<DT, 2>(bufs, count, stream);
    case 3: return tree_dispatch_v<DT, 3>(bufs, count, stream);
    case 4: return tree_dispatch_v<DT, 4>(bufs, count, stream);
    case 5: return tree_dispatch_v<DT, 5>(bufs, count, stream);
    case 6: return tree_dispatch_v<DT, 6>(bufs, count, stream);
    case 7: return tree_dispatch_v<DT, 7>(bufs, count, stream);
    case 8: return tree_dispatch_v<DT, 8>(bufs, count, stream);
    case 16: return tree_dispatch_v<DT, 16>(bufs, count, stream);
    default: return hipErrorInvalidValue;
  }
}

template <int DT>
hipError_t pair_dispatch(const RankPtrs& bufs, const PairJobs& pairs, uint64_t count, hipStream_t stream) {
  constexpr int V = 4;
  const uint64_t tile = (uint64_t)kThreads * Vec<DT>::E * V;
  const uint64_t tiles = (count + tile - 1) / tile;
  hipLaunchKernelGGL((pair_add_kernel<DT, V>), dim3((unsigned)(tiles * (uint64_t)pairs.npairs)), dim3(kThreads), 0,
                     stream, bufs, pairs, count, (uint32_t)tiles);
  return launch_status(stream);
}

}  // namespace

// Workgroups per CU for the fold over n ranks, measured on MI355X (fused
// allreduce, 2 GiB per launch).  fp32/fp16: N = 2 -> 3 (6.28 TB/s against
// 5.84 uncapped), N = 4 -> 1 (5.77 against 4.94 at 2), N = 8 and 16 -> 1;
// bf16 needs more waves to hide its rounding ALU: N = 2 -> 4, N = 4 -> 2
// (6.35), N = 8 -> 3 (8 x 128M: 728 us against 766 at 2), N = 16 -> 2.
// Rank counts without a specialised kernel
// (runtime loop, loads not hoisted) -> 2 (N = 5: 5.11 against 4.57 at 1).
// Tile order of the fused fold (chunk_tile_k's K).  Which XCD streams which
// chunk changes the HBM rate more than any per-workgroup change, differently
// per rank count and dtype (MI355X, contiguous rank buffers a power of two
// apart, fraction of 8 TB/s): N = 8 keeps one chunk per XCD (K = 1: bf16
// 0.73, fp32 0.72-0.73; K = 2..32: 0.67-0.70 bf16); N = 16 bf16 (64M per
// rank) 0.68 at K = 1, 0.718 at K = 32, 0.64-0.66 tiles fastest; N = 16 fp32
// (32M per rank) 0.67 at K = 1, 0.60-0.67 at K = 2..32, 0.727 tiles fastest;
// at N = 16 each XCD x streaming chunk x to its end and then chunk x + 8
// measured 0.708 bf16 and 0.707 fp32.  Starting chunk c's tiles at tile
// c*tiles/N (N = 8 fp32, K = 1) measured 0.751-0.755 against 0.767-0.770.
uint64_t fold_tile_group(int dt, int n, uint64_t tiles) {
  if (n == 16) return dt == DT_F32 ? (tiles > 0 ? tiles : 1) : 32;
  return 1;
}

int fold_wgs_per_cu(int dt, int n) {
  const bool b16 = dt == DT_BF16;
  switch (n) {
    case 2: return b16 ? 4 : 3;
    case 4: return b16 ? 2 : 1;
    case 8: return b16 ? 3 : 1;  // bf16 8 x 128M: 728 us at 3, 766 at 2, 741 at 1, 734 at 4
    case 16: return b16 ? 2 : 1;
    default: return 2;
  }
}
hipError_t launch_status(hipStream_t stream) {
  static const bool sync = [] {
    const char* v = std::getenv("RAR_DEBUG_SYNC");
    return v && *v && std::strcmp(v, "0") != 0;
  }();
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess || !sync) return e;
  return hipStreamSynchronize(stream);
}

size_t residency_lds(int wgs_per_cu) {
  if (wgs_per_cu <= 0) return 0;
  static std::atomic<uint64_t> cache[kMaxRanks];  // per device: LDS per CU << 32 | LDS per workgroup
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxRanks) return 0;
  uint64_t c = cache[dev].load(std::memory_order_relaxed);
  if (c == 0) {
    int a = 0, b = 0;
    if (hipDeviceGetAttribute(&a, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev) != hipSuccess ||
        hipDeviceGetAttribute(&b, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess || a <= 0 || b <= 0)
      return 0;
    c = (uint64_t)a << 32 | (uint64_t)b;
    cache[dev].store(c, std::memory_order_relaxed);
  }
  const size_t per_cu = (size_t)(c >> 32), per_wg = (size_t)(c & 0xffffffffu);
  const size_t want = per_cu / (size_t)(wgs_per_cu + 1) + 1024;
  return want <= per_wg ? want : 0;
}

hipError_t launch_ring_fold(const RankPtrs& bufs, int n, uint64_t count, uint64_t L, int dt,
                            bool store_all, hipStream_t stream) {
  if (L == 0 || count == 0) return hipSuccess;
  switch (dt) {
    case DT_F32: return fold_dispatch_n<DT_F32>(bufs, n, count, L, store_all, stream);
    case DT_F16: return fold_dispatch_n<DT_F16>(bufs, n, count, L, store_all, stream);
    default: return fold_dispatch_n<DT_BF16>(bufs, n, count, L, store_all, stream);
  }
}

hipError_t launch_rs_step(const RankPtrs& bufs, int n, uint64_t count, uint64_t L, int dt, int s,
                          hipStream_t stream) {
  if (L == 0 || count == 0) return hipSuccess;
  switch (dt) {
    case DT_F32: return step_dispatch<DT_F32>(bufs, n, count, L, s, stream);
    case DT_F16: return step_dispatch<DT_F16>(bufs, n, count, L, s, stream);
    default: return step_dispatch<DT_BF16>(bufs, n, count, L, s, stream);
  }
}

hipError_t launch_copy_jobs(const CopyJobs& jobs, hipStream_t stream) {
  uint64_t maxlen = 0;
  int fanout = 0;
  for (int j = 0; j < jobs.njobs; ++j) {
    maxlen = jobs.len[j] > maxlen ? jobs.len[j] : maxlen;
    const int f = __builtin_popcountll(jobs.dstmask[j]);
    fanout = f > fanout ? f : fanout;
  }
  if (jobs.njobs == 0 || maxlen == 0) return hipSuccess;
  const uint64_t tile = (uint64_t)kThreads * 16 * kCopyVecs;
  const uint32_t tiles = (uint32_t)((maxlen + tile - 1) / tile);
  dim3 grid((unsigned)((uint64_t)jobs.njobs * tiles)), block(kThreads);
  // Residency (MI355X): a 1-to-7 fan-out copy runs best at 3 workgroups per
  // CU (+8% over uncapped), a 1-to-1 copy at 6 (+3%).
  const size_t lds = residency_lds(fanout >= 4 ? 3 : 6);
  hipLaunchKernelGGL(copy_jobs_kernel, grid, block, lds, stream, jobs, tiles);
  return launch_status(stream);
}

bool tree_fold_supported(int n) { return (n >= 2 && n <= 8) || n == 16; }

hipError_t launch_tree_fold(const RankPtrs& bufs, int n, uint64_t count, int dt, hipStream_t stream) {
  if (count == 0) return hipSuccess;
  switch (dt) {
    case DT_F32: return tree_dispatch_n<DT_F32>(bufs, n, count, stream);
    case DT_F16: return tree_dispatch_n<DT_F16>(bufs, n, count, stream);
    default: return tree_dispatch_n<DT_BF16>(bufs, n, count, stream);
  }
}

hipError_t launch_pair_add(const RankPtrs& bufs, const PairJobs& pairs, uint64_t count, int dt, hipStream_t stream) {
  if (count == 0 || pairs.npairs == 0) return hipSuccess;
  switch (dt) {
    case DT_F32: return pair_dispatch<DT_F32>(bufs, pairs, count, stream);
    case DT_F16: return pair_dispatch<DT_F16>(bufs, pairs, count, stream);
    default: return pair_dispatch<DT_BF16>(bufs, pairs, count, stream);
  }
}

}  // namespace rar
