// Gradient-bucket pack / unpack for gfx950 (page "从零实现集合通信",
// production patterns: small gradient tensors are fused into ~25 MB buckets
// and reduced with one allreduce per bucket).
//
// A launch carries up to kMaxRanks segment jobs in its arguments: copy
// `bytes` from src to dst and then zero dst up to `zero_to`.  Inside a bucket
// every tensor starts on a 16-byte boundary, so both ends of every job are
// 16-byte aligned and the body is 16-byte vector copies; only a tensor's
// last partial vector is copied in 2-byte units.
#include "launch.hpp"

namespace rar {

namespace {

constexpr int kSegVecs = 4;  // 16-byte vectors per thread

__global__ __launch_bounds__(kThreads) void seg_copy_kernel(SegJobs jobs, uint32_t tiles_per_job) {
  const int j = (int)(blockIdx.x / tiles_per_job);
  const uint32_t t = blockIdx.x - (uint32_t)j * tiles_per_job;
  const char* src = jobs.src[j];
  char* dst = jobs.dst[j];
  const uint64_t bytes = jobs.bytes[j], zero_to = jobs.zero_to[j];
  const uint64_t body = bytes / 16 * 16;
  constexpr uint64_t kTileBytes = (uint64_t)kThreads * 16 * kSegVecs;
  const uint64_t b0 = (uint64_t)t * kTileBytes + (uint64_t)threadIdx.x * 16;
  u32x4 v[kSegVecs];
#pragma unroll
  for (int i = 0; i < kSegVecs; ++i) {
    const uint64_t b = b0 + (uint64_t)i * kThreads * 16;
    if (b + 16 <= body) v[i] = ld16<true>(src + b);
  }
#pragma unroll
  for (int i = 0; i < kSegVecs; ++i) {
    const uint64_t b = b0 + (uint64_t)i * kThreads * 16;
    if (b + 16 <= body) st16<false>(dst + b, v[i]);
  }
  if (t == 0 && threadIdx.x < 8) {
    // tail of the data (< 16 bytes, 2-byte units) and the zero gap after it
    const uint64_t off = body + 2 * threadIdx.x;
    if (off < zero_to) {
      const uint16_t x = off < bytes ? *(const uint16_t*)(src + off) : (uint16_t)0;
      *(uint16_t*)(dst + off) = x;
    }
  }
}

}  // namespace

hipError_t launch_seg_copy(const SegJobs& jobs, hipStream_t stream) {
  uint64_t maxb = 0;
  for (int j = 0; j < jobs.njobs; ++j) maxb = jobs.bytes[j] > maxb ? jobs.bytes[j] : maxb;
  if (jobs.njobs == 0) return hipSuccess;
  const uint64_t tile = (uint64_t)kThreads * 16 * kSegVecs;
  uint32_t tiles = (uint32_t)((maxb + tile - 1) / tile);
  if (tiles == 0) tiles = 1;
  dim3 grid((unsigned)((uint64_t)jobs.njobs * tiles)), block(kThreads);
  hipLaunchKernelGGL(seg_copy_kernel, grid, block, 0, stream, jobs, tiles);
  return launch_status(stream);
}

}  // namespace rar

// ---------------------------------------------------------------- zero-copy bucket fold
// All buckets of a bucketed allreduce in one launch, reading and writing the
// gradient tensors in place.  A bucket is the virtual concatenation of its
// tensors, each starting on a 16-byte boundary; the chunk rule and the ring
// order apply to that flat index space exactly as if the bucket had been
// packed, so the results equal pack -> ring allreduce -> unpack.  Because
// every 16-byte vector of the flat space lies inside one tensor (or in its
// zero gap), a vector is loaded straight from the N ranks' copies of that
// tensor.
//
// Device table (uint64 words, written by the host before the launch):
//   [0]                       number of buckets nb
//   [1, nb+2)                 first workgroup of each bucket (prefix sums)
//   per bucket b at hdr+4b:   padded length, chunk length L, first tensor, tensors
//   per tensor t at ten+2t:   flat offset inside its bucket, element count
//   pointers at ptr + r*nt+t: rank r's copy of tensor t
// followed (256-byte aligned) by one descriptor per fold workgroup
// (bucket_desc_stride(N) bytes each), written on the device by
// bucket_desc_kernel.
namespace rar {
namespace {

__device__ __forceinline__ uint64_t ld_u64(const uint64_t* p) { return *p; }

// Largest i in [lo, hi) with key(i) <= x, where key is ascending.
template <typename F>
__device__ __forceinline__ uint64_t upper_index(uint64_t lo, uint64_t hi, uint64_t x, F key) {
  while (hi - lo > 1) {
    const uint64_t mid = (lo + hi) / 2;
    if (key(mid) <= x) lo = mid;
    else hi = mid;
  }
  return lo;
}

// Where workgroup g of the launch works: bucket b, chunk c, and the flat
// element range [tile0, tile1) of its tile (empty when the chunk or the
// tile lies past the bucket's end).
struct TileLoc {
  uint64_t tile0, tile1, t0, nt;
  int c;
  bool empty;
};

__device__ __forceinline__ TileLoc locate_tile(const uint64_t* tab, int N, uint64_t g, uint64_t kTile) {
  TileLoc loc{};
  const uint64_t nb = ld_u64(tab);
  const uint64_t* start = tab + 1;
  const uint64_t* hdr = tab + 2 + nb;
  const uint64_t b = upper_index(0, nb, g, [&](uint64_t i) { return ld_u64(start + i); });
  const uint64_t local = g - ld_u64(start + b);
  const uint64_t total = ld_u64(hdr + 4 * b), L = ld_u64(hdr + 4 * b + 1);
  loc.t0 = ld_u64(hdr + 4 * b + 2);
  loc.nt = ld_u64(hdr + 4 * b + 3);
  loc.c = (int)(local % (uint64_t)N);
  const uint64_t tile = local / (uint64_t)N;
  const uint64_t lo = (uint64_t)loc.c * L;
  loc.empty = true;
  if (lo >= total) return loc;
  const uint64_t hi = lo + L < total ? lo + L : total;
  loc.tile0 = lo + tile * kTile;
  if (loc.tile0 >= hi) return loc;
  loc.tile1 = loc.tile0 + kTile < hi ? loc.tile0 + kTile : hi;
  loc.empty = false;
  return loc;
}

// Per-workgroup descriptor of the fold: 16 bytes of header (word 0 the
// tensor index of a whole tile inside one tensor, or kDescEmpty /
// kDescSlow; word 1 the chunk; words 2-3 the tile's first element inside
// that tensor), then for a whole tile the N ranks' addresses of that first
// element.  Computed by bucket_desc_kernel when the plan is prepared, so a
// fold workgroup issues its loads after one round of independent scalar
// loads (header and addresses together) instead of the searches through the
// bucket and tensor tables.
constexpr uint32_t kDescEmpty = 0xffffffffu;
constexpr uint32_t kDescSlow = 0xfffffffeu;

__global__ __launch_bounds__(kThreads) void bucket_desc_kernel(const uint64_t* __restrict__ tab, int N,
                                                                uint64_t ntensors, uint64_t grid, uint64_t kTile,
                                                                uint64_t es, char* __restrict__ descs,
                                                                uint64_t dstride) {
  const uint64_t g = (uint64_t)blockIdx.x * kThreads + threadIdx.x;
  if (g >= grid) return;
  const uint64_t nb = ld_u64(tab);
  const uint64_t* ten = tab + 2 + 5 * nb;
  const uint64_t* ptr = ten + 2 * ntensors;
  char* dp = descs + g * dstride;
  const TileLoc loc = locate_tile(tab, N, g, kTile);
  u32x4 d = {kDescEmpty, 0u, 0u, 0u};
  if (!loc.empty) {
    auto tensor_of = [&](uint64_t f) {
      return upper_index(0, loc.nt, f, [&](uint64_t i) { return ld_u64(ten + 2 * (loc.t0 + i)); });
    };
    const uint64_t ja = tensor_of(loc.tile0), jb = tensor_of(loc.tile1 - 1);
    const uint64_t t = loc.t0 + ja;
    const uint64_t off = ld_u64(ten + 2 * t), cnt = ld_u64(ten + 2 * t + 1);
    d[0] = kDescSlow;
    d[1] = (uint32_t)loc.c;
    if (ja == jb && loc.tile1 <= off + cnt && loc.tile0 + kTile == loc.tile1 && t < (uint64_t)kDescSlow) {
      const uint64_t e = loc.tile0 - off;
      d[0] = (uint32_t)t;
      d[2] = (uint32_t)e;
      d[3] = (uint32_t)(e >> 32);
      uint64_t* addr = (uint64_t*)(dp + 16);
      for (int r = 0; r < N; ++r) addr[r] = ld_u64(ptr + (uint64_t)r * ntensors + t) + e * es;
    }
  }
  *(u32x4*)dp = d;
}

template <int DT, int NR, int V>
__global__ __launch_bounds__(kThreads) void bucket_fold_kernel(const uint64_t* __restrict__ tab,
                                                                const char* __restrict__ descs, uint64_t dstride,
                                                                int nranks, uint64_t ntensors) {
  constexpr int E = Vec<DT>::E;
  constexpr int ES = DtypeSize<DT>::value;
  constexpr uint64_t kTile = (uint64_t)kThreads * E * V;
  const int N = NR > 0 ? NR : nranks;
  const char* dp = descs + (uint64_t)blockIdx.x * dstride;
  const u32x4 dsc = *(const u32x4*)dp;
  if (dsc[0] == kDescEmpty) return;
  const uint64_t nb = ld_u64(tab);
  const uint64_t* ten = tab + 2 + 5 * nb;
  const uint64_t* ptr = ten + 2 * ntensors;
  const int c = (int)dsc[1];
  const int first = c + 1 < N ? c + 1 : 0;

  if (dsc[0] != kDescSlow) {
    // The whole tile lies in one tensor: the N ranks' addresses of its first
    // element come with the descriptor; uniform pointers, vector loads.
    const uint64_t* addr = (const uint64_t*)(dp + 16);
    auto elem = [&](int v) -> uint64_t { return ((uint64_t)v * kThreads + threadIdx.x) * E; };
    Vec<DT> acc[V];
    if constexpr (NR > 0) {
      u32x4 x[NR][V];
      int r = first;
#pragma unroll
      for (int k = 0; k < NR; ++k) {
        const char* p = (const char*)addr[r];
#pragma unroll
        for (int v = 0; v < V; ++v) x[k][v] = ld16<true>(p + elem(v) * ES);
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
      const char* p = (const char*)addr[r];
#pragma unroll
      for (int v = 0; v < V; ++v) acc[v] = unpack16<DT>(ld16<true>(p + elem(v) * ES));
      for (int k = 1; k < N; ++k) {
        r = r + 1 == N ? 0 : r + 1;
        p = (const char*)addr[r];
#pragma unroll
        for (int v = 0; v < V; ++v) {
          const Vec<DT> y = unpack16<DT>(ld16<true>(p + elem(v) * ES));
#pragma unroll
          for (int i = 0; i < E; ++i) acc[v].v[i] = round_to<DT>(y.v[i] + acc[v].v[i]);
        }
      }
    }
#pragma unroll
    for (int v = 0; v < V; ++v) {
      const u32x4 out = pack16<DT>(acc[v]);
      for (int d = 0; d < N; ++d) st16<true>((char*)addr[d] + elem(v) * ES, out);
    }
    return;
  }
  // Tiles that cross a tensor boundary, reach into a zero gap, or are the
  // ragged end of a chunk.  Tensors start on 16-byte boundaries inside the
  // bucket, so each lane's 16-byte vector lies in one tensor (or in its zero
  // gap): the lane finds that tensor and moves whole vectors, and only a
  // tensor's last, partial vector goes element by element.  Chunk ends and
  // padded tensor ends are multiples of the vector, so no vector crosses the
  // tile's end.
  const TileLoc loc = locate_tile(tab, N, blockIdx.x, kTile);
  if (loc.empty) return;
  auto tensor_of = [&](uint64_t f) {
    return upper_index(0, loc.nt, f, [&](uint64_t i) { return ld_u64(ten + 2 * (loc.t0 + i)); });
  };
  for (int v = 0; v < V; ++v) {
    const uint64_t f = loc.tile0 + ((uint64_t)v * kThreads + threadIdx.x) * E;
    if (f >= loc.tile1) continue;
    const uint64_t t = loc.t0 + tensor_of(f);
    const uint64_t off = ld_u64(ten + 2 * t), cnt = ld_u64(ten + 2 * t + 1);
    const uint64_t rel = f - off;
    if (rel >= cnt) continue;  // zero gap after the tensor: nothing stored
    auto rank_ptr = [&](int r) { return (char*)ld_u64(ptr + (uint64_t)r * ntensors + t); };
    if (cnt - rel >= (uint64_t)E) {
      int r = first;
      Vec<DT> acc = unpack16<DT>(ld16<true>(rank_ptr(r) + rel * ES));
      for (int k = 1; k < N; ++k) {
        r = r + 1 == N ? 0 : r + 1;
        const Vec<DT> y = unpack16<DT>(ld16<true>(rank_ptr(r) + rel * ES));
#pragma unroll
        for (int i = 0; i < E; ++i) acc.v[i] = round_to<DT>(y.v[i] + acc.v[i]);
      }
      const u32x4 out = pack16<DT>(acc);
      for (int d = 0; d < N; ++d) st16<true>(rank_ptr(d) + rel * ES, out);
      continue;
    }
    const int nv = (int)(cnt - rel);
    for (int i = 0; i < nv; ++i) {
      int r = first;
      float acc = load_elem<DT>(rank_ptr(r), rel + i);
      for (int k = 1; k < N; ++k) {
        r = r + 1 == N ? 0 : r + 1;
        acc = round_to<DT>(load_elem<DT>(rank_ptr(r), rel + i) + acc);
      }
      for (int d = 0; d < N; ++d) store_elem<DT>(rank_ptr(d), rel + i, acc);
    }
  }
}

template <int DT, int NR>
hipError_t bucket_fold_dispatch(const uint64_t* tab, const char* desc, uint64_t dstride, int n, uint64_t ntensors,
                                uint64_t grid, hipStream_t stream) {
  constexpr int V = DT == DT_BF16 ? 1 : 2;
  hipLaunchKernelGGL((bucket_fold_kernel<DT, NR, V>), dim3((unsigned)grid), dim3(kThreads),
                     residency_lds(fold_wgs_per_cu(DT, n)), stream, tab, desc, dstride, n, ntensors);
  return launch_status(stream);
}

template <int DT>
hipError_t bucket_fold_n(const uint64_t* tab, const char* desc, uint64_t dstride, int n, uint64_t ntensors,
                         uint64_t grid, hipStream_t stream) {
  switch (n) {
    case 8: return bucket_fold_dispatch<DT, 8>(tab, desc, dstride, n, ntensors, grid, stream);
    case 16: return bucket_fold_dispatch<DT, 16>(tab, desc, dstride, n, ntensors, grid, stream);
    default: return bucket_fold_dispatch<DT, 0>(tab, desc, dstride, n, ntensors, grid, stream);
  }
}

}  // namespace

uint64_t bucket_fold_tile_elems(int dt) {
  return (uint64_t)kThreads * (dt == DT_F32 ? 4 : 8) * (dt == DT_BF16 ? 1 : 2);
}

uint64_t bucket_desc_stride(int n) { return (16 + 8 * (uint64_t)n + 15) / 16 * 16; }

hipError_t launch_bucket_desc(const uint64_t* dev_table, void* dev_desc, int n, uint64_t ntensors, uint64_t grid,
                              int dt, hipStream_t stream) {
  if (grid == 0) return hipSuccess;
  const uint64_t dgrid = (grid + kThreads - 1) / kThreads;
  hipLaunchKernelGGL(bucket_desc_kernel, dim3((unsigned)dgrid), dim3(kThreads), 0, stream, dev_table, n, ntensors,
                     grid, bucket_fold_tile_elems(dt), (uint64_t)(dt == DT_F32 ? 4 : 2), (char*)dev_desc,
                     bucket_desc_stride(n));
  return launch_status(stream);
}

hipError_t launch_bucket_fold(const uint64_t* dev_table, const void* dev_desc, int n, uint64_t ntensors,
                              uint64_t grid, int dt, hipStream_t stream) {
  if (grid == 0) return hipSuccess;
  const char* desc = (const char*)dev_desc;
  const uint64_t dstride = bucket_desc_stride(n);
  switch (dt) {
    case DT_F32: return bucket_fold_n<DT_F32>(dev_table, desc, dstride, n, ntensors, grid, stream);
    case DT_F16: return bucket_fold_n<DT_F16>(dev_table, desc, dstride, n, ntensors, grid, stream);
    default: return bucket_fold_n<DT_BF16>(dev_table, desc, dstride, n, ntensors, grid, stream);
  }
}

}  // namespace rar
