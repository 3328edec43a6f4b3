// Pipelined compressed ring with materialised messages, one launch
// (page "CCCL通信压缩库：突破LLM训练通信墙的工程实践", section 2.2: chunks are
// compressed, sent, decompressed and reduced by the receiver, the next
// chunk being compressed while the previous one is in flight; section 2.1:
// block floating point with a shared exponent per block).
//
// Every message of the ring is written to its own slot in the workspace:
// for chunk c, message h (h = 1 .. N) is sent by rank (c + h) mod N; hops
// 1 .. N-1 carry the reduce-scatter partial of ranks c+1 .. c+h, and hop N
// is the owner's allgather message.  A workgroup owns one tile of one
// chunk and carries it through the hops in ring order:
//   encode the partial of rank c+1 -> store message 1;
//   for h = 2 .. N: load message h-1 back from its slot (the receiver's
//     side), decode, add rank (c+h)'s own copy, encode, store message h;
//   load message N back, decode, store the result to every rank.
// The hops of one tile run in program order, so no flag or barrier between
// workgroups is needed; at any moment the tiles in flight sit at different
// hops, which is the pipeline's overlap of compression and transfer.  All
// lanes of a BFP block are in one wavefront (the block's exponent byte is
// written by its first lane and read back by all of them), so the stores of
// a hop are ordered before the loads of the next by a wavefront-scope wait.
//
// HBM bytes per element position (N ranks, es bytes per element, message
// bytes m per element): N*es read + N*es written + N*m of messages written;
// most messages are read back while still in the L2 (N = 8 x 128M fp16,
// 8-bit: 0.29 of the 1.08 GB of messages came back from HBM).  (The fused fold
// writes no messages; the hop-per-launch forwarding schedule also reads
// every message back from HBM.)
#include "bfp_device.hpp"
#include "h16_codec.hpp"
#include "launch.hpp"

namespace rar {

namespace {

// The stores of this wavefront are complete (visible to its own later
// loads through the CU's L1) before any later load is issued.
__device__ __forceinline__ void wave_stores_done() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): stores acknowledged
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

struct PipeArgs {
  RankPtrs bufs;
  uint8_t* slots;      // message slots [hop 1..N][chunk][unit], slot bytes each
  uint64_t count, L, U, upc, slot;
  int nranks, lpb, mbits;
};

// Per lane: where its 8 elements sit in its unit's message.
struct LanePos {
  uint64_t e;        // first element (buffer index)
  int nv;            // valid elements (0..8)
  uint64_t unit;     // unit of the chunk
  uint64_t off;      // element offset inside the unit
  uint64_t ulen;     // elements of the unit
};

__device__ __forceinline__ LanePos lane_pos(uint64_t e, uint64_t lo, uint64_t hi, uint64_t U) {
  LanePos p;
  p.e = e;
  p.nv = e >= hi ? 0 : (hi - e >= 8 ? 8 : (int)(hi - e));
  const uint64_t rel = (e < hi ? e : hi - 1) - lo;
  p.unit = rel / U;
  p.off = rel - p.unit * U;
  const uint64_t ustart = p.unit * U, clen = hi - lo;
  p.ulen = clen - ustart < U ? clen - ustart : U;
  return p;
}

// Message of hop h (1-based) of chunk c, the lane's unit.
__device__ __forceinline__ uint8_t* slot_of(const PipeArgs& a, int n, int h, uint32_t c, uint64_t unit) {
  return a.slots + ((((uint64_t)(h - 1) * (uint64_t)n + c) * a.upc + unit) * a.slot);
}

// The unit's exponent bytes end at a multiple of 16; the lane holding the
// unit's first element writes the zero padding.
__device__ __forceinline__ void pad_exponents(uint8_t* msg, const LanePos& lp, uint64_t block) {
  if (lp.nv == 0 || lp.off != 0) return;
  const uint64_t nb = (lp.ulen + block - 1) / block, eb = (nb + 15) / 16 * 16;
  for (uint64_t i = nb; i < eb; ++i) msg[i] = 0;
}

// ------------------------------------------------------------ binary16, block 128
// One tile of G groups per lane (group g of lane l: elements
// tile0 + (g * 256 + l) * 8 ..  + 8, so each group is a contiguous 4 KiB of
// the tile); FULL = every group holds 8 valid elements.  The G hop chains are
// independent, so they share each wait for the message stores.
template <int NR, int G, bool M8, bool FULL>
__device__ __forceinline__ void pipe_h16_tile(const PipeArgs& a, int N, uint32_t c, uint64_t lo, uint64_t hi,
                                              uint64_t tile0) {
  const int mbits = a.mbits;
  const bool block_lead = (threadIdx.x & 15u) == 0;
  const uint64_t hstride = (uint64_t)N * a.upc * a.slot;  // message h+1 sits hstride bytes after message h
  uint64_t eoff[G];        // byte offset of the lane's elements in a rank buffer
  int nv[G];
  uint8_t* mp[G];          // the lane's mantissas in message 1
  uint8_t* ep[G];          // its block's exponent byte in message 1
  uint8_t* padp[G];        // unit start (exponent padding), or NULL
  int npad[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const LanePos lp = lane_pos(tile0 + ((uint64_t)g * kThreads + threadIdx.x) * kGroupElems, lo, hi, a.U);
    const uint64_t nb = (lp.ulen + 127) / 128, eb = (nb + 15) / 16 * 16;
    uint8_t* msg = a.slots + ((uint64_t)c * a.upc + lp.unit) * a.slot;
    eoff[g] = lp.e * 2;
    nv[g] = FULL ? 8 : lp.nv;
    mp[g] = msg + eb + (M8 ? lp.off : lp.off / 2);
    ep[g] = msg + lp.off / 128;
    const bool pads = lp.nv > 0 && lp.off == 0 && eb > nb;
    padp[g] = pads ? msg + nb : nullptr;
    npad[g] = pads ? (int)(eb - nb) : 0;
  }

  auto load_rank = [&](int rank, int g) -> u32x4 {
    if constexpr (FULL) return ld16<true>(a.bufs.p[rank] + eoff[g]);
    else return pack8<DT_F16>(load_part8<DT_F16>(a.bufs.p[rank], eoff[g] / 2, nv[g])).w[0];
  };
  auto store_msg = [&](int h, int g, const H16Code& q) {
    if (!FULL && nv[g] == 0) return;
    const uint64_t hoff = (uint64_t)(h - 1) * hstride;
    if (block_lead) ep[g][hoff] = (uint8_t)q.E;
    if (padp[g])
      for (int i = 0; i < npad[g]; ++i) padp[g][hoff + i] = 0;
    uint8_t* m = mp[g] + hoff;
    if (FULL || nv[g] == 8) {
      if constexpr (M8) *(u32x2*)m = q.bytes;
      else *(uint32_t*)m = q.bytes[0];
    } else if constexpr (M8) {
      for (int i = 0; i < nv[g]; ++i) m[i] = (uint8_t)(q.bytes[i >> 2] >> (8 * (i & 3)));
    } else {
      for (int i = 0; i < (nv[g] + 1) / 2; ++i) m[i] = (uint8_t)(q.bytes[0] >> (8 * i));
    }
  };
  auto load_msg = [&](int h, int g) -> u32x4 {
    if (!FULL && nv[g] == 0) return (u32x4){0u, 0u, 0u, 0u};
    const uint64_t hoff = (uint64_t)(h - 1) * hstride;
    const uint32_t E = ep[g][hoff];
    const uint8_t* m = mp[g] + hoff;
    u32x2 w = {0u, 0u};
    if (FULL || nv[g] == 8) {
      if constexpr (M8) w = *(const u32x2*)m;
      else w[0] = *(const uint32_t*)m;
    } else if constexpr (M8) {
      for (int i = 0; i < nv[g]; ++i) w[i >> 2] |= (uint32_t)m[i] << (8 * (i & 3));
    } else {
      for (int i = 0; i < (nv[g] + 1) / 2; ++i) w[0] |= (uint32_t)m[i] << (8 * i);
    }
    return dec_h16x8(E, w, mbits);
  };

  // every rank's copy of the tile, in ring order from rank c+1
  const int first = (int)c + 1 < N ? (int)c + 1 : 0;
  // the ragged tile loads each rank's copy at its hop (fewer live registers)
  constexpr bool kPrefetch = NR > 0 && FULL;
  u32x4 x[kPrefetch ? NR : 1][G];
  u32x4 p[G];
  if constexpr (kPrefetch) {
#pragma unroll
    for (int k = 0; k < NR; ++k)
#pragma unroll
      for (int g = 0; g < G; ++g) x[k][g] = load_rank((first + k) % NR, g);
#pragma unroll
    for (int g = 0; g < G; ++g) p[g] = x[0][g];
  } else {
#pragma unroll
    for (int g = 0; g < G; ++g) p[g] = load_rank(first, g);
  }
#pragma unroll
  for (int g = 0; g < G; ++g) store_msg(1, g, enc_h16x8(p[g], mbits));
  // hop h: the receiver (rank c+h) takes message h-1 from its slot, adds its
  // own copy and sends message h
  auto hop = [&](int h, const u32x4* xr) {
    wave_stores_done();
    u32x4 d[G];
#pragma unroll
    for (int g = 0; g < G; ++g) d[g] = load_msg(h - 1, g);
#pragma unroll
    for (int g = 0; g < G; ++g) {
#pragma unroll
      for (int i = 0; i < 4; ++i) p[g][i] = h2_bits(as_h2(xr[g][i]) + as_h2(d[g][i]));
      if (!FULL && nv[g] < 8)
        for (int i = nv[g]; i < 8; ++i) p[g][i >> 1] &= (i & 1) ? 0x0000ffffu : 0xffff0000u;  // idle: +0
      store_msg(h, g, enc_h16x8(p[g], mbits));
    }
  };
  if constexpr (kPrefetch) {
#pragma unroll
    for (int h = 2; h <= NR; ++h) hop(h, x[h - 1]);
  } else {
    for (int h = 2; h <= N; ++h) {
      u32x4 xr[G];
#pragma unroll
      for (int g = 0; g < G; ++g) xr[g] = load_rank((first + h - 1) % N, g);
      hop(h, xr);
    }
  }
  wave_stores_done();
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const u32x4 y = load_msg(N, g);
    if constexpr (FULL) {
      // write-through stores over the tile's range in each rank
      constexpr uint32_t kBytes = (uint32_t)kThreads * kGroupElems * G * 2;
      for (int d = 0; d < N; ++d) st16_wt(wt_range(a.bufs.p[d] + tile0 * 2, kBytes), (uint32_t)(eoff[g] - tile0 * 2), y);
    } else if (nv[g] > 0) {
      Raw8<DT_F16> yr;
      yr.w[0] = y;
      const G8 yg = unpack8<DT_F16>(yr);
      for (int d = 0; d < N; ++d) store_part8<DT_F16>(a.bufs.p[d], eoff[g] / 2, nv[g], yg);
    }
  }
}

template <int NR, int G, bool M8>
__global__ __launch_bounds__(kThreads) void bfp_pipe_h16_kernel(PipeArgs a) {
  const int N = NR > 0 ? NR : a.nranks;
  const uint32_t c = blockIdx.x % (uint32_t)N;
  const uint32_t t = blockIdx.x / (uint32_t)N;
  const uint64_t lo = (uint64_t)c * a.L;
  if (lo >= a.count) return;
  const uint64_t hi = lo + a.L < a.count ? lo + a.L : a.count;
  constexpr uint64_t kTile = (uint64_t)kThreads * kGroupElems * G;
  const uint64_t tile0 = lo + (uint64_t)t * kTile;
  if (tile0 >= hi) return;
  if (tile0 + kTile <= hi) pipe_h16_tile<NR, G, M8, true>(a, N, c, lo, hi, tile0);
  else pipe_h16_tile<NR, G, M8, false>(a, N, c, lo, hi, tile0);
}

// ------------------------------------------------------------ any dtype and block
// The binary32 formulation of the hop (encode_group / dequant_group), one
// 8-element group per lane.
template <int DT, int LPB>
__global__ __launch_bounds__(kThreads) void bfp_pipe_kernel(PipeArgs a) {
  const int N = a.nranks;
  const int lpb = LPB > 0 ? LPB : a.lpb;
  const uint64_t block = (uint64_t)lpb * 8;
  const uint32_t c = blockIdx.x % (uint32_t)N;
  const uint32_t t = blockIdx.x / (uint32_t)N;
  const uint64_t lo = (uint64_t)c * a.L;
  if (lo >= a.count) return;
  const uint64_t hi = lo + a.L < a.count ? lo + a.L : a.count;
  constexpr uint64_t kTile = (uint64_t)kThreads * kGroupElems;
  const uint64_t tile0 = lo + (uint64_t)t * kTile;
  if (tile0 >= hi) return;
  const LanePos lp = lane_pos(tile0 + (uint64_t)threadIdx.x * kGroupElems, lo, hi, a.U);
  const int mbits = a.mbits;
  const float qmax = (float)((1 << (mbits - 1)) - 1);
  const uint64_t nb = (lp.ulen + block - 1) / block, eb = (nb + 15) / 16 * 16;
  const int first = (int)c + 1 < N ? (int)c + 1 : 0;

  auto encode_to = [&](uint8_t* msg, const G8& p) {
    // encode_group writes the block's exponent at msg[elem / block] and the
    // mantissas from msg + eb; elem is the lane's offset inside the unit
    pad_exponents(msg, lp, block);
    encode_group<DT, LPB>(p, lp.nv, lp.off, msg, msg + eb, lpb, mbits, qmax);
  };
  auto decode_from = [&](const uint8_t* msg) -> G8 {
    if (lp.nv == 0) return G8{};
    return dequant_group(msg, eb, lp.off, lp.nv, block, mbits);
  };

  G8 p = load_group<DT>(a.bufs.p[first], lp.e, lp.nv);
  encode_to(slot_of(a, N, 1, c, lp.unit), p);
  int r = first;
  for (int h = 2; h <= N; ++h) {
    r = r + 1 == N ? 0 : r + 1;
    const G8 x = load_group<DT>(a.bufs.p[r], lp.e, lp.nv);
    wave_stores_done();
    const G8 d = decode_from(slot_of(a, N, h - 1, c, lp.unit));
#pragma unroll
    for (int i = 0; i < 8; ++i) p.v[i] = i < lp.nv ? round_to<DT>(x.v[i] + d.v[i]) : 0.0f;
    encode_to(slot_of(a, N, h, c, lp.unit), p);
  }
  wave_stores_done();
  const G8 y = decode_from(slot_of(a, N, N, c, lp.unit));
  if (lp.nv > 0)
    for (int d = 0; d < N; ++d) store_group<DT>(a.bufs.p[d], lp.e, lp.nv, y);
}

}  // namespace

// Workgroups per CU of the pipelined kernels (0 = no cap).  Binary16,
// N = 8 x 128M, 4 MiB units, measured on MI355X: 8-bit messages 1.033 ms at
// six against 1.078 uncapped, 1.39 at two and 2.23 at one; 4-bit 0.857
// against 0.884 uncapped.  Two 8-element groups per lane (98 VGPRs, four
// waves per SIMD) measured slower: 1.12-1.16 ms.
int pipe_wgs_per_cu(int dt) { return dt == DT_F16 ? 6 : 0; }

template <int NR, int G>
void pipe_h16_dispatch(const PipeArgs& a, uint64_t L, int n, size_t lds, hipStream_t stream) {
  const uint64_t tile = (uint64_t)kThreads * kGroupElems * G;
  const dim3 grid((unsigned)((uint64_t)n * ((L + tile - 1) / tile)));
  if (a.mbits > 4) hipLaunchKernelGGL((bfp_pipe_h16_kernel<NR, G, true>), grid, dim3(kThreads), lds, stream, a);
  else hipLaunchKernelGGL((bfp_pipe_h16_kernel<NR, G, false>), grid, dim3(kThreads), lds, stream, a);
}

hipError_t launch_bfp_pipe(const RankPtrs& bufs, int n, uint64_t count, uint64_t L, uint64_t U, uint64_t upc,
                           uint64_t slot, uint8_t* slots, int dt, int block, int mbits, hipStream_t stream) {
  if (L == 0 || count == 0) return hipSuccess;
  PipeArgs a;
  a.bufs = bufs;
  a.slots = slots;
  a.count = count;
  a.L = L;
  a.U = U;
  a.upc = upc;
  a.slot = slot;
  a.nranks = n;
  a.lpb = block / 8;
  a.mbits = mbits;
  const size_t lds = residency_lds(pipe_wgs_per_cu(dt));
  if (dt == DT_F16 && block == 128) {
    if (n == 8) pipe_h16_dispatch<8, 1>(a, L, n, lds, stream);
    else pipe_h16_dispatch<0, 1>(a, L, n, lds, stream);
    return launch_status(stream);
  }
  const uint64_t tile = (uint64_t)kThreads * kGroupElems;
  const dim3 grid((unsigned)((uint64_t)n * ((L + tile - 1) / tile)));
  if (block == 128) {
    switch (dt) {
      case DT_F32: hipLaunchKernelGGL((bfp_pipe_kernel<DT_F32, 16>), grid, dim3(kThreads), lds, stream, a); break;
      case DT_F16: hipLaunchKernelGGL((bfp_pipe_kernel<DT_F16, 16>), grid, dim3(kThreads), lds, stream, a); break;
      default: hipLaunchKernelGGL((bfp_pipe_kernel<DT_BF16, 16>), grid, dim3(kThreads), lds, stream, a); break;
    }
  } else {
    switch (dt) {
      case DT_F32: hipLaunchKernelGGL((bfp_pipe_kernel<DT_F32, 0>), grid, dim3(kThreads), lds, stream, a); break;
      case DT_F16: hipLaunchKernelGGL((bfp_pipe_kernel<DT_F16, 0>), grid, dim3(kThreads), lds, stream, a); break;
      default: hipLaunchKernelGGL((bfp_pipe_kernel<DT_BF16, 0>), grid, dim3(kThreads), lds, stream, a); break;
    }
  }
  return launch_status(stream);
}

}  // namespace rar
