// Workgroup-wide integer scans and sums for the 256-lane streaming kernels
// (four wavefronts of 64 lanes).  Each call uses its own small LDS array
// and one or two barriers; every lane of the workgroup must call it.
#pragma once

#include "common.hpp"

namespace rar {

// Exclusive prefix sum of v over the workgroup's lanes in lane order; *total
// receives the sum of all lanes.
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, uint32_t* total) {
  __shared__ uint32_t wsum[kThreads / 64];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  uint32_t x = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const uint32_t y = (uint32_t)__shfl_up((int)x, d, 64);
    if (lane >= d) x += y;
  }
  if (lane == 63) wsum[w] = x;
  __syncthreads();
  uint32_t base = 0, tot = 0;
#pragma unroll
  for (int k = 0; k < kThreads / 64; ++k) {
    if (k < w) base += wsum[k];
    tot += wsum[k];
  }
  __syncthreads();
  *total = tot;
  return base + x - v;
}

// Workgroup sums of two per-lane integers (every lane receives both), with
// one barrier: wavefront butterflies, then the four wavefront sums via LDS.
// A second call must be separated from the first by a barrier (the lanes of
// the first may still be reading the LDS partials).
__device__ __forceinline__ void block_sum2(uint32_t a, uint32_t b, uint32_t* sa, uint32_t* sb) {
  __shared__ uint32_t part[2][kThreads / 64];
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) {
    a += (uint32_t)__shfl_xor((int)a, d, 64);
    b += (uint32_t)__shfl_xor((int)b, d, 64);
  }
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    part[0][w] = a;
    part[1][w] = b;
  }
  __syncthreads();
  uint32_t x = 0, y = 0;
#pragma unroll
  for (int k = 0; k < kThreads / 64; ++k) {
    x += part[0][k];
    y += part[1][k];
  }
  *sa = x;
  *sb = y;
}

}  // namespace rar
