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
// packed, so the results equal pack -> ring allreduce -> unpack.  An
// element's result depends only on its chunk (which fixes the order of the
// sum), so the fold may group elements into workgroups freely: it works on
// runs, each the elements that one tensor shares with one chunk, and tiles a
// run from its tensor's start (rounded down to kRunAlign elements), so every
// wavefront's accesses start on a cache-line boundary of the tensor whatever
// the tensor's offset inside the bucket.  (Tiles of the flat index space
// would start anywhere on a 16-byte grid of the tensor, and each wavefront's
// kilobyte would then touch one cache line more: measured on 16 bf16 ranks
// of the 200-tensor workload, 0.663 of 8 TB/s against 0.693 with tensor
// sizes rounded to 64 elements.)
//
// A bucket has N*M workgroup slots, M its largest chunk's tile count (the
// slots past a smaller chunk's tiles stay empty); a chunk's tiles go in the
// order of its elements.  The chip hands workgroups to its 8 XCDs in turn
// (workgroup w to XCD w mod 8), and the HBM rate depends on how many
// separate ranges each XCD streams at once.  With N a multiple of 8 (every
// bucket then starts on a multiple of 8 slots) slot 8j + x goes to chunk
// x + 8*(j / M), tile j mod M: XCD x streams chunk x to its end, then chunk
// x + 8, and so on.  Otherwise slot N*i + c takes the i-th tile of chunk c
// (chunk fastest; the same order as above for N = 8).  On 16 bf16 ranks of
// the 200-tensor workload, fraction of 8 TB/s: 0.735 with the XCD-major
// order; 0.709 chunk fastest (each XCD alternating between chunks x and
// x + 8); 0.63 with the chunk rotated by one per tile row (every XCD over
// every chunk); 0.57 in the order of the elements (every resident
// workgroup inside one chunk).
//
// Device table (uint64 words, written by the host before the launch):
//   [0]                       number of buckets nb
//   [1, nb+2)                 first workgroup of each bucket (prefix sums)
//   crun = tab + nb + 2:      first run of chunk c of bucket b at b*N + c,
//                             nb*N + 1 words (the runs of a chunk are
//                             consecutive; the last word is the run count)
//   per run j at run+4j:      tensor t, first and end element of the run
//                             inside tensor t, tiles of the chunk's runs
//                             before it
//   pointers at ptr + r*nt+t: rank r's copy of tensor t
// followed (256-byte aligned) by one descriptor per fold workgroup
// (bucket_desc_stride(N) bytes each), written on the device by
// bucket_desc_kernel.
namespace rar {
namespace {

__device__ __forceinline__ uint64_t ld_u64(const uint64_t* p) { return *p; }

// The tensors' addresses reach the fold as integers (from the descriptors).
// As pointers into the global address space they give global memory
// instructions: a uniform address becomes the scalar base of the load, and
// the scalar loads of further addresses do not wait for the data (a flat
// load counts against the scalar counter too, so each wait for an address
// would also wait for the load before it).  Whole vectors are stored
// write-through (st16_wt) over the tile's range in each rank.
typedef __attribute__((address_space(1))) char gchar;
typedef __attribute__((address_space(1))) u32x4 gu32x4;
__device__ __forceinline__ gchar* gptr(uint64_t a) { return (gchar*)a; }
__device__ __forceinline__ u32x4 gld16(const gchar* p) { return __builtin_nontemporal_load((const gu32x4*)p); }
template <int DT>
__device__ __forceinline__ float gload_elem(const gchar* base, uint64_t i) {
  typedef __attribute__((address_space(1))) const float gf32;
  typedef __attribute__((address_space(1))) const uint16_t gu16;
  if constexpr (DT == DT_F32) return ((gf32*)base)[i];
  else return widen16<DT>(((gu16*)base)[i]);
}
template <int DT>
__device__ __forceinline__ void gstore_elem(gchar* base, uint64_t i, float x) {
  typedef __attribute__((address_space(1))) float gf32;
  typedef __attribute__((address_space(1))) uint16_t gu16;
  if constexpr (DT == DT_F32) ((gf32*)base)[i] = x;
  else ((gu16*)base)[i] = (uint16_t)narrow16<DT>(x);
}

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

// Per-workgroup descriptor of the fold (bucket_desc_stride(N) bytes): a
// 16-byte header {kind, lo, hi, 0}, then the N ranks' addresses of the
// tile's base element in the fold's order (rank c+1 first, rank c last, c
// the run's chunk).  The tile covers the kTile elements from its base; the
// workgroup owns those in [lo, hi) of them (kDescWhole: all; kDescEmpty:
// none, and no addresses).  Computed by
// bucket_desc_kernel when the plan is prepared, so a fold workgroup issues
// its loads after one round of independent scalar loads.
constexpr uint32_t kDescWhole = 0u;
constexpr uint32_t kDescPart = 1u;
constexpr uint32_t kDescEmpty = 2u;

__global__ __launch_bounds__(kThreads) void bucket_desc_kernel(const uint64_t* __restrict__ tab, int N,
                                                                uint64_t ntensors, uint64_t grid, uint64_t kTile,
                                                                uint64_t es, char* __restrict__ descs,
                                                                uint64_t dstride) {
  const uint64_t g = (uint64_t)blockIdx.x * kThreads + threadIdx.x;
  if (g >= grid) return;
  const uint64_t nb = ld_u64(tab);
  const uint64_t* start = tab + 1;
  const uint64_t* crun = tab + nb + 2;
  const uint64_t nr = ld_u64(crun + nb * (uint64_t)N);
  const uint64_t* run = crun + nb * (uint64_t)N + 1;
  const uint64_t* ptr = run + 4 * nr;
  char* dp = descs + g * dstride;
  const uint64_t bk = upper_index(0, nb, g, [&](uint64_t i) { return ld_u64(start + i); });
  const uint64_t local = g - ld_u64(start + bk);
  uint64_t c = local % (uint64_t)N, i = local / (uint64_t)N;
  if (N % 8 == 0) {  // XCD-major
    const uint64_t m = (ld_u64(start + bk + 1) - ld_u64(start + bk)) / (uint64_t)N;  // M
    const uint64_t x = local % 8, j = local / 8;
    c = x + 8 * (j / m);
    i = j % m;
  }
  const uint64_t r0 = ld_u64(crun + bk * N + c), r1 = ld_u64(crun + bk * N + c + 1);
  u32x4 d = {kDescEmpty, 0u, 0u, 0u};
  if (r0 < r1) {
    const uint64_t j = upper_index(r0, r1, i, [&](uint64_t q) { return ld_u64(run + 4 * q + 3); });
    const uint64_t k = i - ld_u64(run + 4 * j + 3);
    const uint64_t t = ld_u64(run + 4 * j);
    const uint64_t a = ld_u64(run + 4 * j + 1), b = ld_u64(run + 4 * j + 2);
    const uint64_t e0 = a / kRunAlign * kRunAlign + k * kTile;  // the tile's base, inside tensor t
    if (e0 < b) {  // else a slot past the chunk's last tile
      const uint64_t lo = a > e0 ? a : e0, hi = b < e0 + kTile ? b : e0 + kTile;
      d[0] = lo == e0 && hi == e0 + kTile ? kDescWhole : kDescPart;
      d[1] = (uint32_t)(lo - e0);
      d[2] = (uint32_t)(hi - e0);
      uint64_t* addr = (uint64_t*)(dp + 16);
      for (int q = 0; q < N; ++q)
        addr[q] = ld_u64(ptr + (uint64_t)((c + 1 + (uint64_t)q) % (uint64_t)N) * ntensors + t) + e0 * es;
    }
  }
  *(u32x4*)dp = d;
}

// Whole 16-byte vectors: the fold over the N ranks (addresses in fold order)
// of the vectors at element offsets off[v] from each rank's base; all loads
// are issued before the sums.
template <int DT, int NR, int V>
__device__ __forceinline__ void fold_vectors(const uint64_t* addr, int N, const uint32_t* off, Vec<DT>* acc) {
  constexpr int E = Vec<DT>::E;
  constexpr int ES = DtypeSize<DT>::value;
  if constexpr (NR > 0) {
    uint64_t a[NR];
#pragma unroll
    for (int k = 0; k < NR; ++k) a[k] = addr[k];
    u32x4 x[NR][V];
#pragma unroll
    for (int k = 0; k < NR; ++k)
#pragma unroll
      for (int v = 0; v < V; ++v) x[k][v] = gld16(gptr(a[k]) + off[v] * ES);
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
#pragma unroll
    for (int v = 0; v < V; ++v) acc[v] = unpack16<DT>(gld16(gptr(addr[0]) + off[v] * ES));
    for (int k = 1; k < N; ++k) {
      const gchar* p = gptr(addr[k]);
#pragma unroll
      for (int v = 0; v < V; ++v) {
        const Vec<DT> y = unpack16<DT>(gld16(p + off[v] * ES));
#pragma unroll
        for (int i = 0; i < E; ++i) acc[v].v[i] = round_to<DT>(y.v[i] + acc[v].v[i]);
      }
    }
  }
}

template <int DT, int NR, int V>
__global__ __launch_bounds__(kThreads) void bucket_fold_kernel(const char* __restrict__ descs, uint64_t dstride,
                                                                int nranks) {
  constexpr int E = Vec<DT>::E;
  constexpr int ES = DtypeSize<DT>::value;
  constexpr uint32_t kTileBytes = (uint32_t)kThreads * E * V * ES;  // the tile's range in each rank
  const int N = NR > 0 ? NR : nranks;
  const char* dp = descs + (uint64_t)blockIdx.x * dstride;
  const u32x4 dsc = *(const u32x4*)dp;
  if (dsc[0] == kDescEmpty) return;
  const uint64_t* addr = (const uint64_t*)(dp + 16);
  uint32_t off[V];
#pragma unroll
  for (int v = 0; v < V; ++v) off[v] = ((uint32_t)v * kThreads + threadIdx.x) * E;
  Vec<DT> acc[V];
  if (dsc[0] == kDescWhole) {
    fold_vectors<DT, NR, V>(addr, N, off, acc);
    // write-through stores over the tile's range in each rank
#pragma unroll
    for (int v = 0; v < V; ++v) {
      const u32x4 out = pack16<DT>(acc[v]);
      for (int k = 0; k < N; ++k) st16_wt(wt_range((const char*)addr[k], kTileBytes), off[v] * ES, out);
    }
    return;
  }
  // Part of the tile: the run's first tile (it starts less than kRunAlign
  // elements past the base) or its last.  Runs start and end on 16-byte
  // boundaries of the tensor except at the tensor's end, whose last, partial
  // vector goes element by element.  When [lo, hi) holds a whole vector,
  // lanes whose vector lies outside it load the one at lo (never stored), so
  // every load is issued unconditionally.
  const uint32_t lo = dsc[1], hi = dsc[2];
  bool full[V], part[V];
  uint32_t lr[V];
#pragma unroll
  for (int v = 0; v < V; ++v) {
    full[v] = off[v] >= lo && off[v] + E <= hi;
    part[v] = off[v] >= lo && off[v] < hi && !full[v];
    lr[v] = full[v] ? off[v] : lo;
  }
  if (hi - lo >= (uint32_t)E) fold_vectors<DT, NR, V>(addr, N, lr, acc);  // uniform
#pragma unroll
  for (int v = 0; v < V; ++v) {
    if (!full[v]) continue;
    const u32x4 out = pack16<DT>(acc[v]);
    for (int k = 0; k < N; ++k) st16_wt(wt_range((const char*)addr[k], kTileBytes), off[v] * ES, out);
  }
#pragma unroll
  for (int v = 0; v < V; ++v) {
    if (!part[v]) continue;
    for (uint32_t e = off[v]; e < hi; ++e) {
      float x = gload_elem<DT>(gptr(addr[0]), e);
      for (int k = 1; k < N; ++k) x = round_to<DT>(gload_elem<DT>(gptr(addr[k]), e) + x);
      for (int k = 0; k < N; ++k) gstore_elem<DT>(gptr(addr[k]), e, x);
    }
  }
}

// Workgroups per CU of the bucket fold: the ring fold's, except 16 bf16
// ranks at one (the 200-tensor workload, fraction of 8 TB/s, XCD-major
// order: 0.742 at 1, 0.732 at 2, 0.716 at 3; chunk fastest: 0.709 at 1,
// 0.702 at 2, 0.699 at 3, 0.691 at 4, and 4096-element tiles 0.703 at 1).
int bucket_fold_wgs_per_cu(int dt, int n) { return n == 16 && dt == DT_BF16 ? 1 : fold_wgs_per_cu(dt, n); }

template <int DT, int NR>
hipError_t bucket_fold_dispatch(const char* desc, uint64_t dstride, int n, uint64_t grid, hipStream_t stream) {
  constexpr int V = DT == DT_BF16 ? 1 : 2;
  hipLaunchKernelGGL((bucket_fold_kernel<DT, NR, V>), dim3((unsigned)grid), dim3(kThreads),
                     residency_lds(bucket_fold_wgs_per_cu(DT, n)), stream, desc, dstride, n);
  return launch_status(stream);
}

template <int DT>
hipError_t bucket_fold_n(const char* desc, uint64_t dstride, int n, uint64_t grid, hipStream_t stream) {
  switch (n) {
    case 8: return bucket_fold_dispatch<DT, 8>(desc, dstride, n, grid, stream);
    case 16: return bucket_fold_dispatch<DT, 16>(desc, dstride, n, grid, stream);
    default: return bucket_fold_dispatch<DT, 0>(desc, dstride, n, grid, stream);
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

hipError_t launch_bucket_fold(const void* dev_desc, int n, uint64_t grid, int dt, hipStream_t stream) {
  if (grid == 0) return hipSuccess;
  const char* desc = (const char*)dev_desc;
  const uint64_t dstride = bucket_desc_stride(n);
  switch (dt) {
    case DT_F32: return bucket_fold_n<DT_F32>(desc, dstride, n, grid, stream);
    case DT_F16: return bucket_fold_n<DT_F16>(desc, dstride, n, grid, stream);
    default: return bucket_fold_n<DT_BF16>(desc, dstride, n, grid, stream);
  }
}

}  // namespace rar
