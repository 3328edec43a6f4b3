// Sparse-or-BFP messages of the compressed ring for gfx950 (page "CCCL通信压缩库
// ：突破LLM训练通信墙的工程实践", section 2.1: when a tensor's sparsity exceeds a
// threshold (e.g. 50%) only the non-zero values and their indices are sent
// and the receiver puts them back in place, losslessly; denser data goes as
// block floating point).
//
// A message describes one pipeline unit (`len` elements) and starts with a
// 16-byte header {nnz, kind, len, 0}:
//   kind 1 (sparse): values[nnz] in the element type, zero padding to 16
//                    bytes, then uint32 idx[nnz], ascending, unit-relative;
//   kind 0 (BFP):    nnz = 0, then the BFP layout of the whole unit.
// A unit is sparse iff zeros > threshold * len (zeros are +0 and -0).
//
// Encoding takes two launches over 2048-element tiles (256 lanes x 8):
//   count  - non-zeros per tile;
//   write  - a workgroup takes four consecutive tiles, sums the unit's tile
//            counts (the total and the ones before its first tile) and
//            takes the threshold decision itself, the same integers giving
//            the same decision everywhere; the first tile's workgroup writes
//            the header and the wire byte counters.  Sparse: each tile
//            compacts its non-zeros to its offset (ballot-free: a
//            block-wide exclusive scan of per-lane counts keeps the indices
//            ascending); BFP: the tiles' blocks.
// Decoding works per destination tile: a 64-way wavefront search finds the
// tile's slice of the ascending index array, so no two workgroups touch the
// same element and no atomics are needed.
#include "bfp_device.hpp"
#include "block_scan.hpp"

namespace rar {

namespace {

constexpr uint64_t kTileElems = (uint64_t)kThreads * kGroupElems;  // 2048

__device__ __forceinline__ uint64_t round16(uint64_t x) { return (x + 15) / 16 * 16; }

template <int DT>
__device__ __forceinline__ int nonzeros(const G8& x, int nv) {
  int c = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) c += (i < nv && x.v[i] != 0.0f) ? 1 : 0;
  return c;
}

template <int DT>
__global__ __launch_bounds__(kThreads) void comp_count_kernel(CompJobs jobs, uint32_t tiles_max) {
  const int j = (int)(blockIdx.x / tiles_max);
  const uint32_t t = blockIdx.x - (uint32_t)j * tiles_max;
  const uint64_t len = jobs.len[j];
  if ((uint64_t)t * kTileElems >= len) return;
  const uint64_t elem = (uint64_t)t * kTileElems + (uint64_t)threadIdx.x * 8;
  const int nv = elem >= len ? 0 : (len - elem >= 8 ? 8 : (int)(len - elem));
  const G8 x = load_group<DT>(jobs.src[j], elem, nv);
  uint32_t total, unused;
  block_sum2((uint32_t)nonzeros<DT>(x, nv), 0u, &total, &unused);
  if (threadIdx.x == 0) jobs.tiles[j][t] = total;
}

// Sum of the unit's tile counts before tile t, and of all of them, computed
// by the whole workgroup (T is at most a few thousand).
__device__ __forceinline__ void tile_prefix(const uint32_t* nnzs, uint32_t T, uint32_t t, uint32_t* before,
                                            uint32_t* total) {
  uint32_t a = 0, b = 0;
  for (uint32_t i = threadIdx.x; i < T; i += kThreads) {
    const uint32_t v = nnzs[i];
    b += v;
    if (i < t) a += v;
  }
  block_sum2(a, b, before, total);
}

// Tiles per workgroup of the write kernel: a workgroup loads its tiles'
// data first, sums the unit's tile counts once, then writes the tiles in
// order, carrying the running non-zero offset from one to the next.
constexpr uint32_t kWriteTiles = 4;

template <int DT, int LPB>
__global__ __launch_bounds__(kThreads) void comp_write_kernel(CompJobs jobs, uint32_t groups_per_job, int lpb_rt,
                                                               int mbits, float theta, uint64_t* traffic,
                                                               int block) {
  constexpr int ES = DtypeSize<DT>::value;
  const int j = (int)(blockIdx.x / groups_per_job);
  const uint32_t t0 = (blockIdx.x - (uint32_t)j * groups_per_job) * kWriteTiles;
  const uint64_t len = jobs.len[j];
  if ((uint64_t)t0 * kTileElems >= len) return;
  const uint32_t T = (uint32_t)((len + kTileElems - 1) / kTileElems);
  const char* src = jobs.src[j];
  uint8_t* msg = jobs.msg[j];
  // the tiles' data is loaded first, so its latency overlaps the prefix sums
  G8 x[kWriteTiles];
  int nv[kWriteTiles];
  uint64_t elem[kWriteTiles];
#pragma unroll
  for (uint32_t k = 0; k < kWriteTiles; ++k) {
    elem[k] = (uint64_t)(t0 + k) * kTileElems + (uint64_t)threadIdx.x * 8;
    nv[k] = elem[k] >= len ? 0 : (len - elem[k] >= 8 ? 8 : (int)(len - elem[k]));
    x[k] = load_group<DT>(src, elem[k], nv[k]);
  }
  uint32_t before, nnz32;
  tile_prefix(jobs.tiles[j], T, t0, &before, &nnz32);
  const uint64_t nnz = nnz32;
  const bool sparse = (double)(len - nnz) > (double)theta * (double)len;  // zeros > theta * len
  if (t0 == 0 && threadIdx.x == 0) {
    uint32_t* hdr = (uint32_t*)msg;
    hdr[0] = sparse ? (uint32_t)nnz : 0u;
    hdr[1] = sparse ? 1u : 0u;
    hdr[2] = (uint32_t)len;
    hdr[3] = 0u;
    const uint64_t bytes = sparse ? 16 + round16(nnz * (uint64_t)ES) + 4 * nnz
                                  : 16 + bfp_msg_bytes(len, block, mbits);
    const int n = jobs.nranks;
    for (int h = 0; h < jobs.hops[j]; ++h) {
      atomicAdd((unsigned long long*)&traffic[(jobs.from[j] + h) % n], (unsigned long long)bytes);
      atomicAdd((unsigned long long*)&traffic[kMaxRanks + (jobs.from[j] + h + 1) % n], (unsigned long long)bytes);
    }
  }
  if (sparse) {
    uint8_t* vals = msg + 16;
    uint32_t* idx = (uint32_t*)(msg + 16 + round16(nnz * ES));
    uint64_t base = before;
#pragma unroll
    for (uint32_t k = 0; k < kWriteTiles; ++k) {
      if (t0 + k >= T) break;  // uniform in the workgroup
      uint32_t total;
      uint64_t pos = base + block_exclusive_scan((uint32_t)nonzeros<DT>(x[k], nv[k]), &total);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if (i >= nv[k] || x[k].v[i] == 0.0f) continue;
        if constexpr (ES == 4) ((uint32_t*)vals)[pos] = ((const uint32_t*)src)[elem[k] + i];
        else ((uint16_t*)vals)[pos] = ((const uint16_t*)src)[elem[k] + i];
        idx[pos] = (uint32_t)(elem[k] + i);
        ++pos;
      }
      base += total;
    }
    if (t0 == 0 && threadIdx.x < 16) {
      // zero padding between the values and the indices
      const uint64_t pad0 = 16 + nnz * ES, pad1 = 16 + round16(nnz * ES);
      if (pad0 + threadIdx.x < pad1) msg[pad0 + threadIdx.x] = 0;
    }
  } else {
    const int lpb = LPB > 0 ? LPB : lpb_rt;
    const uint64_t block = (uint64_t)lpb * 8;
    uint8_t* payload = msg + 16;
    const uint64_t nb = (len + block - 1) / block;
    const uint64_t eb = (nb + 15) / 16 * 16;
    if (t0 == 0 && threadIdx.x < eb - nb) payload[nb + threadIdx.x] = 0;
    const float qmax = (float)((1 << (mbits - 1)) - 1);
#pragma unroll
    for (uint32_t k = 0; k < kWriteTiles; ++k) {
      if (t0 + k >= T) break;  // uniform: every lane takes part in the block maxima
      encode_group<DT, LPB>(x[k], nv[k], elem[k], payload, payload + eb, lpb, mbits, qmax);
    }
  }
}

// First position in idx[0, n) whose value is >= key (idx ascending),
// searched by a whole wavefront: each round the 64 lanes probe 64 evenly
// spaced positions and a ballot narrows the range 64-fold, so a message of
// nnz indices costs about log64(nnz) rounds of one load per lane instead of
// log2(nnz) dependent loads.  Every lane of the wavefront must call it and
// receives the result.
__device__ __forceinline__ uint64_t wave_lower_bound_u32(const uint32_t* idx, uint64_t n, uint64_t key) {
  const uint64_t lane = threadIdx.x & 63u;
  uint64_t lo = 0, hi = n;  // the answer lies in [lo, hi]
  while (hi - lo > 64) {
    const uint64_t step = (hi - lo + 63) / 64;
    const uint64_t pos = lo + lane * step;
    const bool below = pos < hi && (uint64_t)idx[pos] < key;
    const uint64_t c = (uint64_t)__popcll(__ballot(below));  // lanes 0..c-1 are below key
    const uint64_t nlo = c ? lo + (c - 1) * step + 1 : lo;
    const uint64_t nhi = lo + c * step < hi ? lo + c * step : hi;
    lo = nlo;
    hi = nhi;
  }
  const uint64_t pos = lo + lane;
  const bool below = pos < hi && (uint64_t)idx[pos] < key;
  return lo + (uint64_t)__popcll(__ballot(below));
}

// Decode one tile of one message into `nfan` destinations (rank buffers at
// elem_off, or the single job destination).  ACC: dst <- dst (+) value;
// otherwise dst <- value (sparse: the tile is zeroed first).
template <int DT, bool ACC>
__device__ __forceinline__ void comp_decode_tile(const uint8_t* msg, uint64_t len, uint32_t t, char* const* dsts,
                                                 int nfan, uint64_t elem_off, int block, int mbits) {
  constexpr int ES = DtypeSize<DT>::value;
  __shared__ uint64_t range[2];
  const uint32_t* hdr = (const uint32_t*)msg;
  const uint64_t tlo = (uint64_t)t * kTileElems;
  const uint64_t thi = tlo + kTileElems < len ? tlo + kTileElems : len;
  if (hdr[1] == 0u) {
    const uint8_t* payload = msg + 16;
    const uint64_t elem = tlo + (uint64_t)threadIdx.x * 8;
    if (elem >= thi) return;
    const int nv = thi - elem >= 8 ? 8 : (int)(thi - elem);
    G8 d = dequant_group(payload, bfp_exp_bytes(len, block), elem, nv, (uint64_t)block, mbits);
    for (int f = 0; f < nfan; ++f) {
      G8 out = d;
      if constexpr (ACC) {
        const G8 a = load_group<DT>(dsts[f], elem_off + elem, nv);
#pragma unroll
        for (int i = 0; i < 8; ++i) out.v[i] = round_to<DT>(a.v[i] + d.v[i]);
      }
      store_group<DT>(dsts[f], elem_off + elem, nv, out);
    }
    return;
  }
  const uint64_t nnz = hdr[0];
  const uint8_t* vals = msg + 16;
  const uint32_t* idx = (const uint32_t*)(msg + 16 + round16(nnz * ES));
  // wavefront 0 finds the slice's start, wavefront 1 its end
  if (threadIdx.x < 128) {
    const uint64_t r = wave_lower_bound_u32(idx, nnz, threadIdx.x < 64 ? tlo : thi);
    if ((threadIdx.x & 63u) == 0) range[threadIdx.x >> 6] = r;
  }
  if constexpr (!ACC) {
    const uint64_t elem = tlo + (uint64_t)threadIdx.x * 8;
    if (elem < thi) {
      const int nv = thi - elem >= 8 ? 8 : (int)(thi - elem);
      G8 z;
#pragma unroll
      for (int i = 0; i < 8; ++i) z.v[i] = 0.0f;
      for (int f = 0; f < nfan; ++f) store_group<DT>(dsts[f], elem_off + elem, nv, z);
    }
  }
  __syncthreads();
  const uint64_t j0 = range[0], j1 = range[1];
  for (uint64_t q = j0 + threadIdx.x; q < j1; q += kThreads) {
    const uint64_t i = elem_off + idx[q];
    if constexpr (ES == 4) {
      const uint32_t raw = ((const uint32_t*)vals)[q];
      for (int f = 0; f < nfan; ++f) {
        float* p = (float*)dsts[f] + i;
        *p = ACC ? *p + __uint_as_float(raw) : __uint_as_float(raw);
      }
    } else {
      const uint16_t raw = ((const uint16_t*)vals)[q];
      for (int f = 0; f < nfan; ++f) {
        uint16_t* p = (uint16_t*)dsts[f] + i;
        *p = ACC ? (uint16_t)narrow16<DT>(widen16<DT>(*p) + widen16<DT>(raw)) : raw;
      }
    }
  }
}

// Decode + accumulate one tile and count the non-zeros the tile holds
// afterwards (the receiver's partial is what it encodes next, so the count
// its encoder would take is produced here).  BFP messages: the sums are in
// registers.  Sparse messages: the tile's non-zeros before the scatter, plus
// the change at every scattered element (indices are unique).
template <int DT>
__device__ __forceinline__ void comp_decode_acc_count_tile(const uint8_t* msg, uint64_t len, uint32_t t, char* dst,
                                                           uint32_t* count_out, int block, int mbits) {
  constexpr int ES = DtypeSize<DT>::value;
  __shared__ uint64_t range[2];
  const uint32_t* hdr = (const uint32_t*)msg;
  const uint64_t tlo = (uint64_t)t * kTileElems;
  const uint64_t thi = tlo + kTileElems < len ? tlo + kTileElems : len;
  const uint64_t elem = tlo + (uint64_t)threadIdx.x * 8;
  const int nv = elem >= thi ? 0 : (thi - elem >= 8 ? 8 : (int)(thi - elem));
  uint32_t mine = 0;
  if (hdr[1] == 0u) {
    if (nv > 0) {
      const G8 d = dequant_group(msg + 16, bfp_exp_bytes(len, block), elem, nv, (uint64_t)block, mbits);
      G8 out = load_group<DT>(dst, elem, nv);
#pragma unroll
      for (int i = 0; i < 8; ++i) out.v[i] = round_to<DT>(out.v[i] + d.v[i]);
      store_group<DT>(dst, elem, nv, out);
      mine = (uint32_t)nonzeros<DT>(out, nv);
    }
  } else {
    const uint64_t nnz = hdr[0];
    const uint8_t* vals = msg + 16;
    const uint32_t* idx = (const uint32_t*)(msg + 16 + round16(nnz * ES));
    // wavefront 0 finds the slice's start, wavefront 1 its end
    if (threadIdx.x < 128) {
      const uint64_t r = wave_lower_bound_u32(idx, nnz, threadIdx.x < 64 ? tlo : thi);
      if ((threadIdx.x & 63u) == 0) range[threadIdx.x >> 6] = r;
    }
    if (nv > 0) mine = (uint32_t)nonzeros<DT>(load_group<DT>(dst, elem, nv), nv);
    __syncthreads();  // every lane has read its elements before any scatter writes one
    const uint64_t j0 = range[0], j1 = range[1];
    for (uint64_t q = j0 + threadIdx.x; q < j1; q += kThreads) {
      const uint64_t i = idx[q];
      float before, after;
      if constexpr (ES == 4) {
        float* p = (float*)dst + i;
        before = *p;
        after = before + __uint_as_float(((const uint32_t*)vals)[q]);
        *p = after;
      } else {
        uint16_t* p = (uint16_t*)dst + i;
        const uint16_t old = *p;
        const uint16_t nw = (uint16_t)narrow16<DT>(widen16<DT>(old) + widen16<DT>(((const uint16_t*)vals)[q]));
        *p = nw;
        before = widen16<DT>(old);
        after = widen16<DT>(nw);
      }
      mine += (after != 0.0f ? 1u : 0u);
      mine -= (before != 0.0f ? 1u : 0u);
    }
  }
  uint32_t total, unused;
  block_sum2(mine, 0u, &total, &unused);
  if (threadIdx.x == 0) *count_out = total;
}

template <int DT>
__global__ __launch_bounds__(kThreads) void comp_decode_acc_kernel(CompAccJobs jobs, uint32_t tiles_max, int block,
                                                                    int mbits) {
  const int j = (int)(blockIdx.x / tiles_max);
  const uint32_t t = blockIdx.x - (uint32_t)j * tiles_max;
  const uint64_t len = jobs.len[j];
  if ((uint64_t)t * kTileElems >= len) return;
  char* dst = jobs.dst[j];
  if (jobs.counts[j]) comp_decode_acc_count_tile<DT>(jobs.msg[j], len, t, dst, jobs.counts[j] + t, block, mbits);
  else comp_decode_tile<DT, true>(jobs.msg[j], len, t, &dst, 1, 0, block, mbits);
}

template <int DT>
__global__ __launch_bounds__(kThreads) void comp_decode_fanout_kernel(BfpJobs jobs, RankPtrs fan, int nfan,
                                                                       uint32_t tiles_max, int block, int mbits) {
  const int j = (int)(blockIdx.x / tiles_max);
  const uint32_t t = blockIdx.x - (uint32_t)j * tiles_max;
  const uint64_t len = jobs.len[j];
  if ((uint64_t)t * kTileElems >= len) return;
  comp_decode_tile<DT, false>(jobs.msg[j], len, t, fan.p, nfan, (uint64_t)(uintptr_t)jobs.dst[j], block, mbits);
}

uint32_t tiles_of(uint64_t len) { return (uint32_t)((len + kTileElems - 1) / kTileElems); }

template <int DT>
hipError_t encode_dt(const CompJobs& jobs, int block, int mbits, float theta, uint64_t* traffic, bool counted,
                     hipStream_t stream) {
  uint64_t ml = 0;
  for (int j = 0; j < jobs.njobs; ++j) ml = jobs.len[j] > ml ? jobs.len[j] : ml;
  const uint32_t tm = tiles_of(ml);
  if (jobs.njobs == 0 || tm == 0) return hipSuccess;
  dim3 grid((unsigned)(jobs.njobs * tm)), blk(kThreads);
  if (!counted) hipLaunchKernelGGL((comp_count_kernel<DT>), grid, blk, 0, stream, jobs, tm);
  const uint32_t gpj = (tm + kWriteTiles - 1) / kWriteTiles;
  dim3 wgrid((unsigned)(jobs.njobs * gpj));
  if (block == 128)
    hipLaunchKernelGGL((comp_write_kernel<DT, 16>), wgrid, blk, 0, stream, jobs, gpj, 16, mbits, theta, traffic,
                       block);
  else
    hipLaunchKernelGGL((comp_write_kernel<DT, 0>), wgrid, blk, 0, stream, jobs, gpj, block / 8, mbits, theta,
                       traffic, block);
  return launch_status(stream);
}

}  // namespace

uint64_t comp_tiles_per_unit(uint64_t unit_elems) { return tiles_of(unit_elems); }

hipError_t launch_comp_encode(const CompJobs& jobs, int dt, int block, int mbits, float theta, uint64_t* traffic,
                              bool counted, hipStream_t stream) {
  switch (dt) {
    case DT_F32: return encode_dt<DT_F32>(jobs, block, mbits, theta, traffic, counted, stream);
    case DT_F16: return encode_dt<DT_F16>(jobs, block, mbits, theta, traffic, counted, stream);
    default: return encode_dt<DT_BF16>(jobs, block, mbits, theta, traffic, counted, stream);
  }
}

hipError_t launch_comp_decode_acc(const CompAccJobs& jobs, int dt, int block, int mbits, hipStream_t stream) {
  uint64_t ml = 0;
  for (int j = 0; j < jobs.njobs; ++j) ml = jobs.len[j] > ml ? jobs.len[j] : ml;
  const uint32_t tm = tiles_of(ml);
  if (jobs.njobs == 0 || tm == 0) return hipSuccess;
  dim3 grid((unsigned)(jobs.njobs * tm)), blk(kThreads);
  switch (dt) {
    case DT_F32: hipLaunchKernelGGL((comp_decode_acc_kernel<DT_F32>), grid, blk, 0, stream, jobs, tm, block, mbits); break;
    case DT_F16: hipLaunchKernelGGL((comp_decode_acc_kernel<DT_F16>), grid, blk, 0, stream, jobs, tm, block, mbits); break;
    default: hipLaunchKernelGGL((comp_decode_acc_kernel<DT_BF16>), grid, blk, 0, stream, jobs, tm, block, mbits); break;
  }
  return launch_status(stream);
}

hipError_t launch_comp_decode_fanout(const BfpJobs& jobs_in, const RankPtrs& fan, int nfan,
                                     const uint64_t* elem_off, int dt, int block, int mbits, hipStream_t stream) {
  BfpJobs jobs = jobs_in;
  for (int j = 0; j < jobs.njobs; ++j) jobs.dst[j] = (char*)(uintptr_t)elem_off[j];
  uint64_t ml = 0;
  for (int j = 0; j < jobs.njobs; ++j) ml = jobs.len[j] > ml ? jobs.len[j] : ml;
  const uint32_t tm = tiles_of(ml);
  if (jobs.njobs == 0 || tm == 0) return hipSuccess;
  dim3 grid((unsigned)(jobs.njobs * tm)), blk(kThreads);
  switch (dt) {
    case DT_F32:
      hipLaunchKernelGGL((comp_decode_fanout_kernel<DT_F32>), grid, blk, 0, stream, jobs, fan, nfan, tm, block, mbits);
      break;
    case DT_F16:
      hipLaunchKernelGGL((comp_decode_fanout_kernel<DT_F16>), grid, blk, 0, stream, jobs, fan, nfan, tm, block, mbits);
      break;
    default:
      hipLaunchKernelGGL((comp_decode_fanout_kernel<DT_BF16>), grid, blk, 0, stream, jobs, fan, nfan, tm, block, mbits);
      break;
  }
  return launch_status(stream);
}

}  // namespace rar
