// Per-rank 64-bit hash of the rank buffers: the shared-state check of the
// PCCL model (page "Prime Intellect 发布 PCCL 分布式训练通信库", section
// "PCCL 模型": a peer whose state hash differs from the majority gets the
// state again).
//
// The hash of an nbytes-byte buffer reads it as little-endian 64-bit words
// w_0 .. w_{W-1} (the last one zero-padded) and forms
//   h = sum_i mix64(w_i + (i+1) * 0x9E3779B97F4A7C15)  (mod 2^64),
// finished on the host as mix64(h xor nbytes); mix64 is the output function
// of the splitmix64 generator (Steele, Lea and Flood, OOPSLA 2014).  The sum
// is order-free, so workgroups reduce their lanes and add into one 64-bit
// accumulator per rank; integer addition makes the result independent of
// the order the adds land in.
#include "launch.hpp"

namespace rar {
namespace {

constexpr uint64_t kGolden = 0x9E3779B97F4A7C15ull;

__device__ __forceinline__ uint64_t term(uint64_t w, uint64_t i) { return hash_mix64(w + (i + 1) * kGolden); }

// blockIdx.y = position in the rank table; 16-byte vectors grid-strided over
// blockIdx.x.  acc[y] receives the rank's sum.
__global__ __launch_bounds__(kThreads) void rank_hash_kernel(RankPtrs bufs, uint64_t nbytes, uint64_t* acc) {
  const int y = blockIdx.y;
  const char* base = bufs.p[y];
  const uint64_t nvec = nbytes / 16;
  uint64_t sum = 0;
  for (uint64_t v = (uint64_t)blockIdx.x * kThreads + threadIdx.x; v < nvec; v += (uint64_t)gridDim.x * kThreads) {
    const u32x4 x = ld16<true>(base + v * 16);
    const uint64_t w0 = (uint64_t)x[0] | ((uint64_t)x[1] << 32);
    const uint64_t w1 = (uint64_t)x[2] | ((uint64_t)x[3] << 32);
    sum += term(w0, 2 * v) + term(w1, 2 * v + 1);
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    // the last nbytes % 16 bytes: at most two words, zero-padded
    const uint8_t* b = (const uint8_t*)base;
    for (uint64_t i = 2 * nvec; i * 8 < nbytes; ++i) {
      uint64_t w = 0;
      for (int k = 0; k < 8; ++k)
        if (i * 8 + k < nbytes) w |= (uint64_t)b[i * 8 + k] << (8 * k);
      sum += term(w, i);
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) sum += __shfl_xor(sum, off);
  __shared__ uint64_t part[kThreads / 64];
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = sum;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint64_t s = 0;
#pragma unroll
    for (int w = 0; w < kThreads / 64; ++w) s += part[w];
    atomicAdd((unsigned long long*)&acc[y], (unsigned long long)s);
  }
}

}  // namespace

hipError_t launch_rank_hash(const RankPtrs& bufs, int n, uint64_t nbytes, uint64_t* acc, hipStream_t stream) {
  uint64_t zeros[kMaxRanks] = {};
  hipError_t e = launch_fill_u64(acc, zeros, n, stream);
  if (e != hipSuccess) return e;
  const uint64_t nvec = nbytes / 16;
  uint64_t per_rank = (nvec + kThreads * 4 - 1) / (kThreads * 4);
  const uint64_t cap = (uint64_t)(4096 / n > 0 ? 4096 / n : 1);
  if (per_rank > cap) per_rank = cap;
  if (per_rank < 1) per_rank = 1;
  hipLaunchKernelGGL(rank_hash_kernel, dim3((unsigned)per_rank, (unsigned)n), dim3(kThreads), 0, stream, bufs, nbytes,
                     acc);
  return launch_status(stream);
}

}  // namespace rar
