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
  return hipGetLastError();
}

}  // namespace rar
