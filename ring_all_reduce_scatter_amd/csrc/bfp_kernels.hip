// Block-floating-point kernels for gfx950 (page "CCCL通信压缩库：突破LLM训练通信墙
// 的工程实践", section 2.1: a block of elements shares one exponent and each
// element keeps a scaled 8- or 4-bit mantissa; section 2.2: compress ->
// communicate -> decompress -> reduce).
//
// Lane layout: a lane owns 8 consecutive elements, so a block of B elements
// is B/8 consecutive lanes (16 lanes = one DPP row for B = 128).  (The fused
// ring over binary32 buffers uses a quad layout instead; see
// bfp_ring_fold_f32q_kernel.)  The block's
// exponent is the max of |x| bit patterns, reduced across those lanes with
// DPP (group_max_u32): E = bits >> 23 (255 when an Inf/NaN is present).
// With e = max(E,1) - 127 and k = m - 2 - e every element is
//   q = clamp(rne(x * 2^k), +-(2^(m-1)-1)),  decoded as q * 2^-k,
// both scalings exact (v_ldexp_f32), rne = v_rndne_f32.
//
// Message layout: uint8 E[nblocks] zero-padded to 16 bytes, then one int8
// per element (m > 4) or two's-complement nibbles (element 2j in bits 3:0,
// 2j+1 in bits 7:4).  A lane's 8 mantissas are one 8-byte (or 4-byte) store.
#include "bfp_device.hpp"

namespace rar {

namespace {

// Grid-stride cap per job.  A single large job (one rank's 256 MiB) wants
// enough workgroups to fill the chip several times: at 1024 the encoder moved
// 4.46 TB/s, at 16384 5.50 TB/s (decode-accumulate 4.84 -> 5.48) on MI355X.
constexpr int kEncBlocksPerJob = 16384;

// ---------------------------------------------------------------- encode (K4)
// grid: njobs x blocks_per_job; grid-stride over the job's 8-element groups.
// The loop bound is rounded up to whole workgroups so every lane of a wave
// takes part in the cross-lane max; lanes past the end hold zeros.
template <int DT, int LPB>
__global__ __launch_bounds__(kThreads) void bfp_encode_kernel(BfpJobs jobs, int lpb_rt, int mbits,
                                                               uint32_t blocks_per_job) {
  const int j = (int)(blockIdx.x / blocks_per_job);
  const uint32_t b = blockIdx.x - (uint32_t)j * blocks_per_job;
  const int lpb = LPB > 0 ? LPB : lpb_rt;
  const uint64_t block = (uint64_t)lpb * 8;
  const uint64_t count = jobs.len[j];
  const char* src = jobs.src[j];
  uint8_t* msg = jobs.msg[j];
  const uint64_t nb = (count + block - 1) / block;
  const uint64_t eb = (nb + 15) / 16 * 16;
  uint8_t* mant = msg + eb;
  const float qmax = (float)((1 << (mbits - 1)) - 1);
  if (b == 0 && threadIdx.x < eb - nb) msg[nb + threadIdx.x] = 0;  // exponent padding
  const uint64_t ngroups = (count + 7) / 8;
  const uint64_t stride = (uint64_t)blocks_per_job * kThreads;
  for (uint64_t g0 = (uint64_t)b * kThreads; g0 < ngroups; g0 += stride) {
    const uint64_t elem = (g0 + threadIdx.x) * 8;
    const int nv = elem >= count ? 0 : (count - elem >= 8 ? 8 : (int)(count - elem));
    encode_group<DT, LPB>(load_group<DT>(src, elem, nv), nv, elem, msg, mant, lpb, mbits, qmax);
  }
}

// Forwarding hop: decode the incoming message (if any), add it to the local
// partial (local + received, rounded to the dtype) and encode the sum as the
// outgoing message, in one pass; the sum itself is not written back.  Same
// grid and lane rules as the encoder.
template <int DT, int LPB>
__global__ __launch_bounds__(kThreads) void bfp_forward_kernel(FwdJobs jobs, int lpb_rt, int mbits,
                                                                uint32_t blocks_per_job) {
  const int j = (int)(blockIdx.x / blocks_per_job);
  const uint32_t b = blockIdx.x - (uint32_t)j * blocks_per_job;
  const int lpb = LPB > 0 ? LPB : lpb_rt;
  const uint64_t block = (uint64_t)lpb * 8;
  const uint64_t count = jobs.len[j];
  const char* local = jobs.local[j];
  const uint8_t* in = jobs.in[j];
  uint8_t* out = jobs.out[j];
  const uint64_t nb = (count + block - 1) / block;
  const uint64_t eb = (nb + 15) / 16 * 16;
  const float qmax = (float)((1 << (mbits - 1)) - 1);
  if (b == 0 && threadIdx.x < eb - nb) out[nb + threadIdx.x] = 0;  // exponent padding
  const uint64_t ngroups = (count + 7) / 8;
  const uint64_t stride = (uint64_t)blocks_per_job * kThreads;
  for (uint64_t g0 = (uint64_t)b * kThreads; g0 < ngroups; g0 += stride) {
    const uint64_t elem = (g0 + threadIdx.x) * 8;
    const int nv = elem >= count ? 0 : (count - elem >= 8 ? 8 : (int)(count - elem));
    G8 p = load_group<DT>(local, elem, nv);
    if (in && nv > 0) {
      const G8 d = dequant_group(in, eb, elem, nv, block, mbits);
#pragma unroll
      for (int i = 0; i < 8; ++i) p.v[i] = i < nv ? round_to<DT>(p.v[i] + d.v[i]) : 0.0f;
    }
    encode_group<DT, LPB>(p, nv, elem, out, out + eb, lpb, mbits, qmax);
  }
}

template <int DT, bool ACC>
__global__ __launch_bounds__(kThreads) void bfp_decode_kernel(BfpJobs jobs, int block, int mbits,
                                                               uint32_t blocks_per_job) {
  const int j = (int)(blockIdx.x / blocks_per_job);
  const uint32_t b = blockIdx.x - (uint32_t)j * blocks_per_job;
  const uint64_t count = jobs.len[j];
  const uint8_t* msg = jobs.msg[j];
  char* dst = jobs.dst[j];
  const uint64_t eb = bfp_exp_bytes(count, block);
  const uint64_t ngroups = (count + 7) / 8;
  const uint64_t stride = (uint64_t)blocks_per_job * kThreads;
  for (uint64_t g = (uint64_t)b * kThreads + threadIdx.x; g < ngroups; g += stride) {
    const uint64_t elem = g * 8;
    const int nv = count - elem >= 8 ? 8 : (int)(count - elem);
    G8 d = dequant_group(msg, eb, elem, nv, (uint64_t)block, mbits);
    if constexpr (ACC) {
      G8 a = load_group<DT>(dst, elem, nv);
#pragma unroll
      for (int i = 0; i < 8; ++i) d.v[i] = round_to<DT>(a.v[i] + d.v[i]);
    }
    store_group<DT>(dst, elem, nv, d);
  }
}

// Decode once, store to `nfan` rank buffers at elem_off[j] + element.
template <int DT>
__global__ __launch_bounds__(kThreads) void bfp_decode_fanout_kernel(BfpJobs jobs, RankPtrs fan,
                                                                      int nfan, int block, int mbits,
                                                                      uint32_t blocks_per_job) {
  const int j = (int)(blockIdx.x / blocks_per_job);
  const uint32_t b = blockIdx.x - (uint32_t)j * blocks_per_job;
  const uint64_t count = jobs.len[j];
  const uint8_t* msg = jobs.msg[j];
  const uint64_t off = (uint64_t)(uintptr_t)jobs.dst[j];  // element offset carried in dst
  const uint64_t eb = bfp_exp_bytes(count, block);
  const uint64_t ngroups = (count + 7) / 8;
  const uint64_t stride = (uint64_t)blocks_per_job * kThreads;
  for (uint64_t g = (uint64_t)b * kThreads + threadIdx.x; g < ngroups; g += stride) {
    const uint64_t elem = g * 8;
    const int nv = count - elem >= 8 ? 8 : (int)(count - elem);
    G8 d = dequant_group(msg, eb, elem, nv, (uint64_t)block, mbits);
    if (nv == 8) {
      Raw8<DT> r = pack8<DT>(d);
      for (int f = 0; f < nfan; ++f) store_raw8<DT, true>(fan.p[f], off + elem, r);
    } else {
      for (int f = 0; f < nfan; ++f) store_part8<DT>(fan.p[f], off + elem, nv, d);
    }
  }
}

// ---------------------------------------------------------------- packed binary16 hop
// For binary16 buffers a whole hop runs on packed halves with the same bits
// as the binary32 formulation:
//  * the block exponent E comes from the max of |h| bit patterns, widened
//    once (widening is exact and monotonic, so E is the same);
//  * s = h * 2^k (v_ldexp_f16) is exact: |s| < 2^(m-1) <= 128 never
//    overflows, and a result below binary16's normal range is below 1/2, so
//    it rounds to q = 0 either way;
//  * round-half-even to an integer: t = s + 1536 lands in [1024, 2048) where
//    the binary16 spacing is 1, so t = 1536 + rne(s); 1536 is even;
//  * clamp to 1536 +- qmax on the bit patterns (t > 0, so unsigned order is
//    numeric order); q = t - 1536 is exact and +0 for a zero mantissa;
//  * q * 2^-k is exact in binary16: its lowest bit is at least 2^-24 when
//    e >= m-26, and below that the step is finer than binary16's grid, so
//    quantisation was lossless and the value is the input half itself;
//  * x + value in binary16 (v_pk_add_f16) equals the binary32 add rounded
//    once to binary16 (24 >= 2*11+2: double rounding is innocuous).
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ h2 as_h2(uint32_t w) { return __builtin_bit_cast(h2, w); }
__device__ __forceinline__ uint32_t h2_bits(h2 v) { return __builtin_bit_cast(uint32_t, v); }
__device__ __forceinline__ u16x2 as_u16x2(uint32_t w) { return __builtin_bit_cast(u16x2, w); }
__device__ __forceinline__ _Float16 ldexp_h(_Float16 x, int k) { return (_Float16)__builtin_amdgcn_ldexph(x, k); }

template <int LPB>
__device__ __forceinline__ u32x4 qdq_h16x8(u32x4 p, int lpb, int mbits, u16x2 lo, u16x2 hi) {
  u16x2 m = __builtin_elementwise_max(as_u16x2(p[0] & 0x7fff7fffu), as_u16x2(p[1] & 0x7fff7fffu));
  m = __builtin_elementwise_max(m, as_u16x2(p[2] & 0x7fff7fffu));
  m = __builtin_elementwise_max(m, as_u16x2(p[3] & 0x7fff7fffu));
  uint32_t mm = max((uint32_t)m[0], (uint32_t)m[1]);
  mm = group_max_sel<LPB>(mm, lpb);
  const int E = (int)(__float_as_uint(h16_to_f32(mm)) >> 23);
  const int k = mbits - 2 - ((E < 1 ? 1 : E) - 127);
  const h2 magic = {(_Float16)1536.0f, (_Float16)1536.0f};
  u32x4 d;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const h2 x = as_h2(p[i]);
    const h2 sc = {ldexp_h(x[0], k), ldexp_h(x[1], k)};
    const u16x2 t = __builtin_elementwise_min(__builtin_elementwise_max(as_u16x2(h2_bits(sc + magic)), lo), hi);
    const h2 q = as_h2(__builtin_bit_cast(uint32_t, t)) - magic;
    const h2 v = {ldexp_h(q[0], -k), ldexp_h(q[1], -k)};
    d[i] = mm >= 0x7c00u ? 0x7e007e00u : h2_bits(v);  // Inf/NaN in the block: NaN
  }
  return d;
}

// ---------------------------------------------------------------- fused compressed ring (K6)
// Workgroup = tile of one chunk c (chunk length L is a multiple of the block,
// so lanes [j*LPB, (j+1)*LPB) always hold one whole block).  Per block:
//   p = x_{c+1};  p = round(x_{c+k} + qdq(p)) for k = 2..N;  y = round(qdq(p))
// and y goes to every rank.  All lanes stay active through the cross-lane
// maxima; lanes past the end of the data hold zeros and store nothing.
template <int DT, int NR, int LPB, int G>
__global__ __launch_bounds__(kThreads) void bfp_ring_fold_kernel(RankPtrs bufs, int nranks,
                                                                  uint64_t count, uint64_t L, int lpb_rt,
                                                                  int mbits) {
  const int N = NR > 0 ? NR : nranks;
  const int lpb = LPB > 0 ? LPB : lpb_rt;
  // chunk fastest: resident workgroups cover every chunk's ring rotation
  const uint32_t c = blockIdx.x % (uint32_t)N;
  const uint32_t t = blockIdx.x / (uint32_t)N;
  const uint64_t lo = (uint64_t)c * L;
  if (lo >= count) return;
  const uint64_t hi = lo + L < count ? lo + L : count;
  constexpr uint64_t kTile = (uint64_t)kThreads * kGroupElems * G;
  const uint64_t tile0 = lo + (uint64_t)t * kTile;
  if (tile0 >= hi) return;
  const uint64_t e0 = tile0 + (uint64_t)threadIdx.x * kGroupElems;
  const int first = (int)c + 1 < N ? (int)c + 1 : 0;
  const float qmax = (float)((1 << (mbits - 1)) - 1);

  int nv[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const uint64_t e = e0 + (uint64_t)g * kThreads * kGroupElems;
    nv[g] = e >= hi ? 0 : (hi - e >= 8 ? 8 : (int)(hi - e));
  }
  const bool full = tile0 + kTile <= hi;

  auto load = [&](int rank, int g) -> G8 {
    const uint64_t e = e0 + (uint64_t)g * kThreads * kGroupElems;
    if (full) return unpack8<DT>(load_raw8<DT, true>(bufs.p[rank], e));
    return load_part8<DT>(bufs.p[rank], e, nv[g]);
  };
  auto qdq = [&](const G8& p) -> G8 {
    const uint32_t m = group_max_sel<LPB>(lane_absmax(p), lpb);
    return qdq8(p, bfp_scale(m, mbits), qmax);
  };

  if constexpr (DT == DT_F16) {
    // packed binary16 hops (bit-identical to the binary32 formulation below)
    const uint32_t qm = (uint32_t)((1 << (mbits - 1)) - 1);
    const u16x2 lo = {(uint16_t)(0x6600u - qm), (uint16_t)(0x6600u - qm)};  // bits of 1536 - qmax
    const u16x2 hi = {(uint16_t)(0x6600u + qm), (uint16_t)(0x6600u + qm)};  // bits of 1536 + qmax
    auto loadh = [&](int rank, int g) -> u32x4 {
      const uint64_t e = e0 + (uint64_t)g * kThreads * kGroupElems;
      if (full) return ld16<true>(bufs.p[rank] + e * 2);
      return pack8<DT>(load_part8<DT>(bufs.p[rank], e, nv[g])).w[0];
    };
    u32x4 ph[G];
#pragma unroll
    for (int g = 0; g < G; ++g) ph[g] = loadh(first, g);
    int rh = first;
    auto hoph = [&]() {
      rh = rh + 1 == N ? 0 : rh + 1;
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const u32x4 x = loadh(rh, g);
        const u32x4 d = qdq_h16x8<LPB>(ph[g], lpb, mbits, lo, hi);
#pragma unroll
        for (int i = 0; i < 4; ++i) ph[g][i] = h2_bits(as_h2(x[i]) + as_h2(d[i]));
      }
    };
    if constexpr (NR > 0) {
#pragma unroll
      for (int k = 2; k <= NR; ++k) hoph();
    } else {
      for (int k = 2; k <= N; ++k) hoph();
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const u32x4 y = qdq_h16x8<LPB>(ph[g], lpb, mbits, lo, hi);
      const uint64_t e = e0 + (uint64_t)g * kThreads * kGroupElems;
      if (full) {
        // write-through stores over the tile's range in each rank
        for (int d = 0; d < N; ++d)
          st16_wt(wt_range(bufs.p[d] + tile0 * 2, (uint32_t)(kTile * 2)), (uint32_t)((e - tile0) * 2), y);
      } else if (nv[g] > 0) {
        Raw8<DT> yr;
        yr.w[0] = y;
        const G8 yg = unpack8<DT>(yr);
        for (int d = 0; d < N; ++d) store_part8<DT>(bufs.p[d], e, nv[g], yg);
      }
    }
    return;
  }

  G8 p[G];
#pragma unroll
  for (int g = 0; g < G; ++g) p[g] = load(first, g);
  int r = first;
  auto hop = [&]() {
    r = r + 1 == N ? 0 : r + 1;
#pragma unroll
    for (int g = 0; g < G; ++g) {
      G8 x = load(r, g);
      G8 d = qdq(p[g]);
#pragma unroll
      for (int i = 0; i < 8; ++i) p[g].v[i] = round_to<DT>(x.v[i] + d.v[i]);
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
    G8 y = qdq(p[g]);
    const uint64_t e = e0 + (uint64_t)g * kThreads * kGroupElems;
    if (full) {
      Raw8<DT> out = pack8<DT>(y);
      constexpr int ES = DtypeSize<DT>::value;
      for (int d = 0; d < N; ++d)
        store_raw8_wt<DT>(wt_range(bufs.p[d] + tile0 * ES, (uint32_t)(kTile * ES)), (uint32_t)((e - tile0) * ES), out);
    } else if (nv[g] > 0) {
      for (int d = 0; d < N; ++d) store_part8<DT>(bufs.p[d], e, nv[g], y);
    }
  }
}

constexpr int kFillWords = 448;  // 3.5 KiB of kernel arguments per launch

struct U64Vals {
  uint64_t v[kFillWords];
};

// ---------------------------------------------------------------- fp32 fused ring, quad layout
// The fused compressed ring for binary32 buffers.  Eight consecutive floats
// per lane would make every load and store instruction touch 16-byte pieces
// 32 bytes apart; here a wavefront owns 512 consecutive elements and lane l
// holds the quads [4l, 4l+4) ("A") and [256+4l, 256+4l+4) ("B"), so every
// instruction covers 1 KiB of contiguous memory.  A block of b <= 256
// elements is b/4 consecutive lanes of one quad set; a 512-element block is
// the whole wavefront, both sets.  The arithmetic is the binary32 hop chain
// of bfp_ring_fold_kernel, element for element.
struct Q8 {
  float v[8];
};

template <int NR, int LPBQ>
__global__ __launch_bounds__(kThreads) void bfp_ring_fold_f32q_kernel(RankPtrs bufs, int nranks, uint64_t count,
                                                                       uint64_t L, int block, int mbits) {
  const int N = NR > 0 ? NR : nranks;
  const uint32_t c = blockIdx.x % (uint32_t)N;
  const uint32_t t = blockIdx.x / (uint32_t)N;
  const uint64_t lo = (uint64_t)c * L;
  if (lo >= count) return;
  const uint64_t hi = lo + L < count ? lo + L : count;
  const uint64_t tile0 = lo + (uint64_t)t * kThreads * kGroupElems;
  if (tile0 >= hi) return;
  const uint32_t lane = threadIdx.x & 63u;
  const uint64_t eA = tile0 + (uint64_t)(threadIdx.x >> 6) * 512 + 4 * lane, eB = eA + 256;
  auto nq = [&](uint64_t e) { return e >= hi ? 0 : (hi - e >= 4 ? 4 : (int)(hi - e)); };
  const int nA = nq(eA), nB = nq(eB);
  const int lpbq = LPBQ > 0 ? LPBQ : (block >= 256 ? 64 : block / 4);
  const bool whole = block == 512;
  const float qmax = (float)((1 << (mbits - 1)) - 1);
  auto ldq = [&](const char* base, uint64_t e, int nv, float* out) {
    if (nv == 4) {
      const u32x4 w = ld16<true>(base + e * 4);
#pragma unroll
      for (int i = 0; i < 4; ++i) out[i] = __uint_as_float(w[i]);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) out[i] = i < nv ? ((const float*)base)[e + i] : 0.0f;
    }
  };
  auto stq = [&](char* base, uint64_t e, int nv, const float* v) {
    if (nv == 4) {
      u32x4 w;
#pragma unroll
      for (int i = 0; i < 4; ++i) w[i] = __float_as_uint(v[i]);
      st16<true>(base + e * 4, w);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (i < nv) ((float*)base)[e + i] = v[i];
    }
  };
  auto load = [&](int rank, Q8& q) {
    ldq(bufs.p[rank], eA, nA, q.v);
    ldq(bufs.p[rank], eB, nB, q.v + 4);
  };
  auto qdq = [&](const Q8& p) -> Q8 {
    uint32_t ma = 0, mb = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ma = max(ma, absbits(p.v[i]));
      mb = max(mb, absbits(p.v[4 + i]));
    }
    if (whole) {
      ma = mb = group_max_u32<64>(max(ma, mb));
    } else {
      ma = group_max_sel<LPBQ>(ma, lpbq);
      mb = group_max_sel<LPBQ>(mb, lpbq);
    }
    const BfpScale sa = bfp_scale(ma, mbits), sb = bfp_scale(mb, mbits);
    const float nanv = __builtin_nanf("");
    Q8 d;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const BfpScale& sc = i < 4 ? sa : sb;
      d.v[i] = sc.nan ? nanv : bfp_dq(bfp_q(p.v[i], sc.k, qmax), sc.k);
    }
    return d;
  };
  const int first = (int)c + 1 < N ? (int)c + 1 : 0;
  Q8 p;
  if constexpr (NR > 0) {
    Q8 x[NR];
#pragma unroll
    for (int j = 0; j < NR; ++j) load(first + j < NR ? first + j : first + j - NR, x[j]);
    p = x[0];
#pragma unroll
    for (int j = 1; j < NR; ++j) {
      const Q8 d = qdq(p);
#pragma unroll
      for (int i = 0; i < 8; ++i) p.v[i] = x[j].v[i] + d.v[i];
    }
  } else {
    load(first, p);
    int r = first;
    for (int k = 2; k <= N; ++k) {
      r = r + 1 == N ? 0 : r + 1;
      Q8 x;
      load(r, x);
      const Q8 d = qdq(p);
#pragma unroll
      for (int i = 0; i < 8; ++i) p.v[i] = x.v[i] + d.v[i];
    }
  }
  const Q8 y = qdq(p);
  if (tile0 + (uint64_t)kThreads * kGroupElems <= hi) {
    // a whole tile: write-through stores over its range in each rank
    u32x4 wa, wb;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      wa[i] = __float_as_uint(y.v[i]);
      wb[i] = __float_as_uint(y.v[4 + i]);
    }
    constexpr uint32_t kBytes = (uint32_t)kThreads * kGroupElems * 4;
    for (int d = 0; d < N; ++d) {
      const WtRange rg = wt_range(bufs.p[d] + tile0 * 4, kBytes);
      st16_wt(rg, (uint32_t)((eA - tile0) * 4), wa);
      st16_wt(rg, (uint32_t)((eB - tile0) * 4), wb);
    }
    return;
  }
  for (int d = 0; d < N; ++d) {
    stq(bufs.p[d], eA, nA, y.v);
    stq(bufs.p[d], eB, nB, y.v + 4);
  }
}

// ---------------------------------------------------------------- stateful fused ring
// Error feedback (FB = 1) or delta coding (FB = 2) on the fused compressed
// ring ("CCCL..." page, section 2.1 differential layer, section 5 error
// feedback).  Each rank encodes each of its elements once per allreduce, so
// rank r keeps one binary32 state value per element (st.p[r]):
//   error feedback: v = p + e, send E(v), e <- v - D(E(v)), receiver gets D
//   delta:          v = p - ref, send E(v), ref <- ref + D(E(v)) = value the
//                   receiver gets
// The hop chain of a block is the one of bfp_ring_fold_kernel with v in place
// of p at every encode, in binary32.  This kernel takes any N, one hop's
// loads at a time; N = 4 and 8 run bfp_ring_fold_state_q_kernel below.
template <int DT, int LPB, int FB>
__global__ __launch_bounds__(kThreads) void bfp_ring_fold_state_kernel(RankPtrs bufs, RankPtrs st, int nranks,
                                                                        uint64_t count, uint64_t L, int lpb_rt,
                                                                        int mbits) {
  const int N = nranks;
  const int lpb = LPB > 0 ? LPB : lpb_rt;
  const uint32_t c = blockIdx.x % (uint32_t)N;
  const uint32_t t = blockIdx.x / (uint32_t)N;
  const uint64_t lo = (uint64_t)c * L;
  if (lo >= count) return;
  const uint64_t hi = lo + L < count ? lo + L : count;
  const uint64_t tile0 = lo + (uint64_t)t * kThreads * kGroupElems;
  if (tile0 >= hi) return;
  const uint64_t e = tile0 + (uint64_t)threadIdx.x * kGroupElems;
  const int nv = e >= hi ? 0 : (hi - e >= 8 ? 8 : (int)(hi - e));
  const float qmax = (float)((1 << (mbits - 1)) - 1);
  auto ld = [&](int rank) -> G8 {
    return nv == 8 ? unpack8<DT>(load_raw8<DT, true>(bufs.p[rank], e)) : load_part8<DT>(bufs.p[rank], e, nv);
  };
  auto ld_state = [&](int rank) -> G8 {
    return nv == 8 ? unpack8<DT_F32>(load_raw8<DT_F32, true>(st.p[rank], e)) : load_part8<DT_F32>(st.p[rank], e, nv);
  };
  auto st_state = [&](int rank, const G8& s) {
    if (nv == 8) store_raw8<DT_F32, true>(st.p[rank], e, pack8<DT_F32>(s));
    else store_part8<DT_F32>(st.p[rank], e, nv, s);
  };
  // Encode v = p +- s, update the sender's state s in place, return what the
  // receiver takes.
  auto message = [&](const G8& p, G8& s) -> G8 {
    G8 v, out;
#pragma unroll
    for (int i = 0; i < 8; ++i) v.v[i] = FB == 1 ? p.v[i] + s.v[i] : p.v[i] - s.v[i];
    const uint32_t m = group_max_sel<LPB>(lane_absmax(v), lpb);
    const G8 d = qdq8(v, bfp_scale(m, mbits), qmax);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (FB == 1) {
        s.v[i] = v.v[i] - d.v[i];
        out.v[i] = d.v[i];
      } else {
        s.v[i] = s.v[i] + d.v[i];
        out.v[i] = s.v[i];
      }
    }
    return out;
  };
  // ring order of chunk c: ranks c+1, ..., c+N-1 send their partials in the
  // reduce-scatter, c is the receiver of the last hop and the allgather owner
  const int first = (int)c + 1 < N ? (int)c + 1 : 0;
  {
    G8 p = ld(first);
    int r = first;
    for (int k = 2; k <= N; ++k) {
      const int sender = r;
      r = r + 1 == N ? 0 : r + 1;
      const G8 x = ld(r);
      G8 s = ld_state(sender);
      const G8 d = message(p, s);
      st_state(sender, s);
#pragma unroll
      for (int i = 0; i < 8; ++i) p.v[i] = round_to<DT>(x.v[i] + d.v[i]);
    }
    G8 s = ld_state((int)c);
    const G8 y = message(p, s);
    st_state((int)c, s);
    for (int d = 0; d < N; ++d) store_group<DT>(bufs.p[d], e, nv, y);
  }
}

// Stateful fused ring, quad layout (N = 4 or 8 ranks known at compile
// time, every rank's inputs and state loaded before the chain): the
// arithmetic of bfp_ring_fold_state_kernel element for element, with the
// lanes laid out as in bfp_ring_fold_f32q_kernel.  A wavefront owns
// 512 consecutive elements; lane l holds [4l, 4l+4) ("A") and [256+4l,
// 256+4l+4) ("B"), so each load or store instruction covers contiguous
// memory for the 16-bit inputs (8 bytes a lane) and for the binary32 state
// (16 bytes a lane) alike, with no LDS staging.  A block of b <= 256
// elements is b/4 consecutive lanes of one set; a 512-element block is the
// whole wavefront.
template <int DT, int NR, int LPBQ, int FB>
__global__ __launch_bounds__(kThreads) void bfp_ring_fold_state_q_kernel(RankPtrs bufs, RankPtrs st, uint64_t count,
                                                                          uint64_t L, int block, int mbits) {
  constexpr int N = NR;
  constexpr int ES = DtypeSize<DT>::value;
  const uint32_t c = blockIdx.x % (uint32_t)N;
  const uint32_t t = blockIdx.x / (uint32_t)N;
  const uint64_t lo = (uint64_t)c * L;
  if (lo >= count) return;
  const uint64_t hi = lo + L < count ? lo + L : count;
  const uint64_t tile0 = lo + (uint64_t)t * kThreads * kGroupElems;
  if (tile0 >= hi) return;
  const uint32_t lane = threadIdx.x & 63u;
  const uint64_t eA = tile0 + (uint64_t)(threadIdx.x >> 6) * 512 + 4 * lane, eB = eA + 256;
  auto nq = [&](uint64_t e) { return e >= hi ? 0 : (hi - e >= 4 ? 4 : (int)(hi - e)); };
  const int nA = nq(eA), nB = nq(eB);
  const int lpbq = LPBQ > 0 ? LPBQ : (block >= 256 ? 64 : block / 4);
  const bool whole = block == 512;
  const float qmax = (float)((1 << (mbits - 1)) - 1);

  // raw quads: 16-bit inputs as 2 words, binary32 (inputs or state) as 4
  typedef typename std::conditional<ES == 2, u32x2, u32x4>::type XQ;
  auto ld_x = [&](int rank, uint64_t e, int nv) -> XQ {
    const char* base = bufs.p[rank];
    XQ w = {};
    if (nv == 4) {
      if constexpr (ES == 2) w = __builtin_nontemporal_load((const u32x2*)(base + e * 2));
      else w = ld16<true>(base + e * 4);
    } else if constexpr (ES == 2) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (i < nv) w[i >> 1] |= (uint32_t)((const uint16_t*)base)[e + i] << (16 * (i & 1));
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (i < nv) w[i] = ((const uint32_t*)base)[e + i];
    }
    return w;
  };
  auto x_val = [&](const XQ& w, int i) -> float {
    if constexpr (ES == 2) return widen16<DT>((w[i >> 1] >> (16 * (i & 1))) & 0xffffu);
    else return __uint_as_float(w[i]);
  };
  auto ld_s = [&](int rank, uint64_t e, int nv) -> u32x4 {
    const char* base = st.p[rank];
    if (nv == 4) return ld16<true>(base + e * 4);
    u32x4 w = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (i < nv) w[i] = ((const uint32_t*)base)[e + i];
    return w;
  };
  auto st_f32 = [&](char* base, uint64_t e, int nv, const float* v) {
    if (nv == 4) {
      u32x4 w;
#pragma unroll
      for (int i = 0; i < 4; ++i) w[i] = __float_as_uint(v[i]);
      st16<true>(base + e * 4, w);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (i < nv) ((float*)base)[e + i] = v[i];
    }
  };
  // a whole tile stores write-through over its range in each rank
  const bool wt = tile0 + (uint64_t)kThreads * kGroupElems <= hi;  // uniform
  constexpr uint32_t kTileElems = (uint32_t)kThreads * kGroupElems;
  auto st_s = [&](int rank, uint64_t e, int nv, const float* v) {
    if (wt) {
      u32x4 w;
#pragma unroll
      for (int i = 0; i < 4; ++i) w[i] = __float_as_uint(v[i]);
      st16_wt(wt_range(st.p[rank] + tile0 * 4, kTileElems * 4), (uint32_t)((e - tile0) * 4), w);
    } else {
      st_f32(st.p[rank], e, nv, v);
    }
  };
  auto st_y = [&](int rank, uint64_t e, int nv, const float* v) {
    char* base = bufs.p[rank];
    if constexpr (ES == 2) {
      if (wt) {
        u32x2 w;
        w[0] = narrow16<DT>(v[0]) | narrow16<DT>(v[1]) << 16;
        w[1] = narrow16<DT>(v[2]) | narrow16<DT>(v[3]) << 16;
        st8_wt(wt_range(base + tile0 * 2, kTileElems * 2), (uint32_t)((e - tile0) * 2), w);
      } else if (nv == 4) {
        u32x2 w;
        w[0] = narrow16<DT>(v[0]) | narrow16<DT>(v[1]) << 16;
        w[1] = narrow16<DT>(v[2]) | narrow16<DT>(v[3]) << 16;
        __builtin_nontemporal_store(w, (u32x2*)(base + e * 2));
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (i < nv) ((uint16_t*)base)[e + i] = (uint16_t)narrow16<DT>(v[i]);
      }
    } else {
      st_f32(base, e, nv, v);
    }
  };
  // Encode v = p +- s, update the sender's state s in place, return what the
  // receiver takes (the hop of bfp_ring_fold_state_kernel).
  auto message = [&](const Q8& p, Q8& s) -> Q8 {
    Q8 v, out;
#pragma unroll
    for (int i = 0; i < 8; ++i) v.v[i] = FB == 1 ? p.v[i] + s.v[i] : p.v[i] - s.v[i];
    uint32_t ma = 0, mb = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ma = max(ma, absbits(v.v[i]));
      mb = max(mb, absbits(v.v[4 + i]));
    }
    if (whole) {
      ma = mb = group_max_u32<64>(max(ma, mb));
    } else {
      ma = group_max_sel<LPBQ>(ma, lpbq);
      mb = group_max_sel<LPBQ>(mb, lpbq);
    }
    const BfpScale sa = bfp_scale(ma, mbits), sb = bfp_scale(mb, mbits);
    const float nanv = __builtin_nanf("");
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const BfpScale& sc = i < 4 ? sa : sb;
      const float d = sc.nan ? nanv : bfp_dq(bfp_q(v.v[i], sc.k, qmax), sc.k);
      if (FB == 1) {
        s.v[i] = v.v[i] - d;
        out.v[i] = d;
      } else {
        s.v[i] = s.v[i] + d;
        out.v[i] = s.v[i];
      }
    }
    return out;
  };
  // ring order of chunk c: ranks c+1, ..., c+N-1 send their partials in the
  // reduce-scatter, c is the receiver of the last hop and the allgather owner
  const int first = (int)c + 1 < N ? (int)c + 1 : 0;
  auto rank_of = [&](int j) { return first + j < N ? first + j : first + j - N; };
  XQ xa[NR], xb[NR];
  u32x4 sa[NR], sb[NR];
#pragma unroll
  for (int j = 0; j < NR; ++j) {
    const int q = rank_of(j);
    xa[j] = ld_x(q, eA, nA);
    xb[j] = ld_x(q, eB, nB);
    sa[j] = ld_s(q, eA, nA);
    sb[j] = ld_s(q, eB, nB);
  }
  auto state_of = [&](int j) -> Q8 {
    Q8 s;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      s.v[i] = __uint_as_float(sa[j][i]);
      s.v[4 + i] = __uint_as_float(sb[j][i]);
    }
    return s;
  };
  Q8 p;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    p.v[i] = x_val(xa[0], i);
    p.v[4 + i] = x_val(xb[0], i);
  }
#pragma unroll
  for (int j = 1; j < NR; ++j) {
    Q8 s = state_of(j - 1);
    const Q8 d = message(p, s);
    st_s(rank_of(j - 1), eA, nA, s.v);
    st_s(rank_of(j - 1), eB, nB, s.v + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      p.v[i] = round_to<DT>(x_val(xa[j], i) + d.v[i]);
      p.v[4 + i] = round_to<DT>(x_val(xb[j], i) + d.v[4 + i]);
    }
  }
  Q8 s = state_of(NR - 1);
  const Q8 y = message(p, s);
  st_s(rank_of(NR - 1), eA, nA, s.v);
  st_s(rank_of(NR - 1), eB, nB, s.v + 4);
#pragma unroll
  for (int d = 0; d < N; ++d) {
    st_y(d, eA, nA, y.v);
    st_y(d, eB, nB, y.v + 4);
  }
}

__global__ void fill_u64_kernel(uint64_t* dst, int n, U64Vals vals) {
  for (int i = threadIdx.x; i < n; i += blockDim.x) dst[i] = vals.v[i];
}

uint32_t blocks_for(uint64_t maxlen) {
  const uint64_t groups = (maxlen + 7) / 8;
  uint64_t blocks = (groups + kThreads - 1) / kThreads;
  if (blocks > kEncBlocksPerJob) blocks = kEncBlocksPerJob;
  return (uint32_t)(blocks ? blocks : 1);
}

uint64_t max_len(const BfpJobs& jobs) {
  uint64_t m = 0;
  for (int j = 0; j < jobs.njobs; ++j) m = jobs.len[j] > m ? jobs.len[j] : m;
  return m;
}

template <int DT>
void encode_dispatch(const BfpJobs& jobs, int block, int mbits, dim3 grid, uint32_t bpj,
                     hipStream_t stream) {
  if (block == 128)
    hipLaunchKernelGGL((bfp_encode_kernel<DT, 16>), grid, dim3(kThreads), 0, stream, jobs, 16, mbits, bpj);
  else
    hipLaunchKernelGGL((bfp_encode_kernel<DT, 0>), grid, dim3(kThreads), 0, stream, jobs, block / 8, mbits,
                       bpj);
}

// 8-element groups per thread in the fused compressed fold.
template <int DT>
struct BfpFoldGroups {
  static constexpr int value = 1;
};

// Workgroups per CU of the fused compressed fold, measured on MI355X at
// N = 8, 2 GiB per launch.  The packed binary16 hop needs about half the VALU
// of the binary32 formulation, so four workgroups per CU (16 waves) hide its
// latency while keeping HBM requests moderate (5.55 TB/s uncapped, 6.06 at
// four).  fp32 buffers move twice the bytes per element and do best at two
// (5.38 TB/s against 4.82 uncapped); bf16 runs the binary32 hop on 2-byte
// elements, ALU-heavy, and needs six (5.82 against 5.67 uncapped, 3.83 at two).
int bfp_fold_wgs_per_cu(int dt) { return dt == DT_F16 ? 4 : (dt == DT_F32 ? 2 : 6); }

template <int DT, int NR>
void fold_dispatch_lpb(const RankPtrs& bufs, int n, uint64_t count, uint64_t L, int block, int mbits,
                       hipStream_t stream) {
  constexpr int G = BfpFoldGroups<DT>::value;
  const uint64_t tile = (uint64_t)kThreads * kGroupElems * G;
  const uint64_t tiles = (L + tile - 1) / tile;
  dim3 grid((unsigned)((uint64_t)n * tiles));
  const size_t lds = residency_lds(bfp_fold_wgs_per_cu(DT));
  if (block == 128)
    hipLaunchKernelGGL((bfp_ring_fold_kernel<DT, NR, 16, G>), grid, dim3(kThreads), lds, stream, bufs, n, count,
                       L, 16, mbits);
  else
    hipLaunchKernelGGL((bfp_ring_fold_kernel<DT, NR, 0, G>), grid, dim3(kThreads), lds, stream, bufs, n, count,
                       L, block / 8, mbits);
}

template <int NR>
void fold_f32q_dispatch(const RankPtrs& bufs, int n, uint64_t count, uint64_t L, int block, int mbits,
                        hipStream_t stream) {
  const uint64_t tile = (uint64_t)kThreads * kGroupElems;
  dim3 grid((unsigned)((uint64_t)n * ((L + tile - 1) / tile)));
  const size_t lds = residency_lds(bfp_fold_wgs_per_cu(DT_F32));
  if (block == 128)
    hipLaunchKernelGGL((bfp_ring_fold_f32q_kernel<NR, 32>), grid, dim3(kThreads), lds, stream, bufs, n, count, L,
                       block, mbits);
  else
    hipLaunchKernelGGL((bfp_ring_fold_f32q_kernel<NR, 0>), grid, dim3(kThreads), lds, stream, bufs, n, count, L,
                       block, mbits);
}

template <int DT>
void fold_dispatch_nr(const RankPtrs& bufs, int n, uint64_t count, uint64_t L, int block, int mbits,
                      hipStream_t stream) {
  if constexpr (DT == DT_F32) {
    if (n == 8) fold_f32q_dispatch<8>(bufs, n, count, L, block, mbits, stream);
    else fold_f32q_dispatch<0>(bufs, n, count, L, block, mbits, stream);
  } else {
    if (n == 8) fold_dispatch_lpb<DT, 8>(bufs, n, count, L, block, mbits, stream);
    else fold_dispatch_lpb<DT, 0>(bufs, n, count, L, block, mbits, stream);
  }
}

// Workgroups per CU of the stateful fold.  Each lane of the quad-layout
// kernel holds N inputs and N state quads in flight (N = 8, fp16: 384
// bytes, 96 KiB a workgroup).  Two workgroups per CU measured best on
// MI355X (N = 8, 128M fp16 with 128M-float state per rank: 2.24-2.25 ms,
// 0.715-0.720 of 8 TB/s; 3.0-3.1 ms at one, 2.28 ms at three, 2.32 ms
// uncapped at four), and so for the generic-N kernel (2.47 ms vs 2.60
// uncapped and 2.52 at three, measured with an earlier LDS-staged layout).
// Workgroups take the chunk fastest, as in the ring fold at 8 ranks;
// groups of K consecutive tiles per chunk measured 0.716 at K = 2, 0.680 at
// 4, 0.700 at 16 and 0.634 at 64 against 0.716-0.719.  Loading the 16-bit
// inputs as 16-byte lanes and moving them to the quad layout with cross-lane
// permutes (and the results back for 16-byte stores) measured 0.698-0.702
// against 0.713-0.715: the permutes cost more than the halved load and
// store counts save; regrouping only the output (eight permutes a tile, then
// 16-byte stores) measured 0.708-0.711 against 0.710-0.712.  Other tile
// orders: all tiles of one chunk before the next 0.675, the chunk rotated by
// one per tile row 0.677, each chunk starting at tile c*tiles/N 0.710-0.714.
// Stores: write-through state and output 0.714-0.717, plain nontemporal
// output 0.705-0.712, plain nontemporal state 0.693-0.696, both plain
// 0.711-0.716.  One quad set per lane (1024-element tiles, half the
// registers) at three, four and six workgroups per CU: 0.704-0.707,
// 0.704-0.706 and 0.694-0.698 against 0.707-0.709 on the same box.
int state_fold_wgs_per_cu() { return 2; }

template <int DT, int NR, int FB>
void fold_state_dispatch_nr(const RankPtrs& bufs, const RankPtrs& st, int n, uint64_t count, uint64_t L, int block,
                            int mbits, hipStream_t stream) {
  const uint64_t tile = (uint64_t)kThreads * kGroupElems;
  const uint64_t tiles = (L + tile - 1) / tile;
  dim3 grid((unsigned)((uint64_t)n * tiles));
  const size_t lds = residency_lds(state_fold_wgs_per_cu());
  if constexpr (NR > 0) {
    if (block == 128)
      hipLaunchKernelGGL((bfp_ring_fold_state_q_kernel<DT, NR, 32, FB>), grid, dim3(kThreads), lds, stream, bufs, st,
                         count, L, block, mbits);
    else
      hipLaunchKernelGGL((bfp_ring_fold_state_q_kernel<DT, NR, 0, FB>), grid, dim3(kThreads), lds, stream, bufs, st,
                         count, L, block, mbits);
  } else {
    if (block == 128)
      hipLaunchKernelGGL((bfp_ring_fold_state_kernel<DT, 16, FB>), grid, dim3(kThreads), lds, stream, bufs, st, n,
                         count, L, 16, mbits);
    else
      hipLaunchKernelGGL((bfp_ring_fold_state_kernel<DT, 0, FB>), grid, dim3(kThreads), lds, stream, bufs, st, n,
                         count, L, block / 8, mbits);
  }
}

template <int DT, int FB>
void fold_state_dispatch(const RankPtrs& bufs, const RankPtrs& st, int n, uint64_t count, uint64_t L, int block,
                         int mbits, hipStream_t stream) {
  if (n == 8) fold_state_dispatch_nr<DT, 8, FB>(bufs, st, n, count, L, block, mbits, stream);
  else if (n == 4) fold_state_dispatch_nr<DT, 4, FB>(bufs, st, n, count, L, block, mbits, stream);
  else fold_state_dispatch_nr<DT, 0, FB>(bufs, st, n, count, L, block, mbits, stream);
}

}  // namespace

hipError_t launch_bfp_forward(const FwdJobs& jobs, int dt, int block, int mbits, hipStream_t stream) {
  uint64_t ml = 0;
  for (int j = 0; j < jobs.njobs; ++j) ml = jobs.len[j] > ml ? jobs.len[j] : ml;
  if (jobs.njobs == 0 || ml == 0) return hipSuccess;
  const uint32_t bpj = blocks_for(ml);
  dim3 grid((unsigned)(jobs.njobs * bpj));
#define RAR_FWD(DTV)                                                                                          \
  if (block == 128)                                                                                           \
    hipLaunchKernelGGL((bfp_forward_kernel<DTV, 16>), grid, dim3(kThreads), 0, stream, jobs, 16, mbits, bpj); \
  else                                                                                                        \
    hipLaunchKernelGGL((bfp_forward_kernel<DTV, 0>), grid, dim3(kThreads), 0, stream, jobs, block / 8, mbits, bpj);
  switch (dt) {
    case DT_F32: RAR_FWD(DT_F32) break;
    case DT_F16: RAR_FWD(DT_F16) break;
    default: RAR_FWD(DT_BF16) break;
  }
#undef RAR_FWD
  return launch_status(stream);
}

hipError_t launch_bfp_encode(const BfpJobs& jobs, int dt, int block, int mbits, hipStream_t stream) {
  const uint64_t ml = max_len(jobs);
  if (jobs.njobs == 0 || ml == 0) return hipSuccess;
  const uint32_t bpj = blocks_for(ml);
  dim3 grid((unsigned)(jobs.njobs * bpj));
  switch (dt) {
    case DT_F32: encode_dispatch<DT_F32>(jobs, block, mbits, grid, bpj, stream); break;
    case DT_F16: encode_dispatch<DT_F16>(jobs, block, mbits, grid, bpj, stream); break;
    default: encode_dispatch<DT_BF16>(jobs, block, mbits, grid, bpj, stream); break;
  }
  return launch_status(stream);
}

hipError_t launch_bfp_decode(const BfpJobs& jobs, int dt, int block, int mbits, bool accumulate,
                             hipStream_t stream) {
  const uint64_t ml = max_len(jobs);
  if (jobs.njobs == 0 || ml == 0) return hipSuccess;
  const uint32_t bpj = blocks_for(ml);
  dim3 grid((unsigned)(jobs.njobs * bpj)), blk(kThreads);
#define RAR_DEC(DTV)                                                                                   \
  if (accumulate)                                                                                      \
    hipLaunchKernelGGL((bfp_decode_kernel<DTV, true>), grid, blk, 0, stream, jobs, block, mbits, bpj); \
  else                                                                                                 \
    hipLaunchKernelGGL((bfp_decode_kernel<DTV, false>), grid, blk, 0, stream, jobs, block, mbits, bpj);
  switch (dt) {
    case DT_F32: RAR_DEC(DT_F32) break;
    case DT_F16: RAR_DEC(DT_F16) break;
    default: RAR_DEC(DT_BF16) break;
  }
#undef RAR_DEC
  return launch_status(stream);
}

hipError_t launch_bfp_decode_fanout(const BfpJobs& jobs_in, const RankPtrs& fan, int nfan,
                                    uint64_t elem_off[kMaxRanks], int dt, int block, int mbits,
                                    hipStream_t stream) {
  BfpJobs jobs = jobs_in;
  for (int j = 0; j < jobs.njobs; ++j) jobs.dst[j] = (char*)(uintptr_t)elem_off[j];
  const uint64_t ml = max_len(jobs);
  if (jobs.njobs == 0 || ml == 0) return hipSuccess;
  const uint32_t bpj = blocks_for(ml);
  dim3 grid((unsigned)(jobs.njobs * bpj)), blk(kThreads);
  switch (dt) {
    case DT_F32:
      hipLaunchKernelGGL((bfp_decode_fanout_kernel<DT_F32>), grid, blk, 0, stream, jobs, fan, nfan, block, mbits, bpj);
      break;
    case DT_F16:
      hipLaunchKernelGGL((bfp_decode_fanout_kernel<DT_F16>), grid, blk, 0, stream, jobs, fan, nfan, block, mbits, bpj);
      break;
    default:
      hipLaunchKernelGGL((bfp_decode_fanout_kernel<DT_BF16>), grid, blk, 0, stream, jobs, fan, nfan, block, mbits, bpj);
      break;
  }
  return launch_status(stream);
}

hipError_t launch_bfp_ring_fold(const RankPtrs& bufs, int n, uint64_t count, uint64_t L, int dt,
                                int block, int mbits, hipStream_t stream) {
  if (L == 0 || count == 0) return hipSuccess;
  switch (dt) {
    case DT_F32: fold_dispatch_nr<DT_F32>(bufs, n, count, L, block, mbits, stream); break;
    case DT_F16: fold_dispatch_nr<DT_F16>(bufs, n, count, L, block, mbits, stream); break;
    default: fold_dispatch_nr<DT_BF16>(bufs, n, count, L, block, mbits, stream); break;
  }
  return launch_status(stream);
}

hipError_t launch_bfp_ring_fold_state(const RankPtrs& bufs, const RankPtrs& state, int n, uint64_t count, uint64_t L,
                                      int dt, int block, int mbits, int feedback, hipStream_t stream) {
  if (L == 0 || count == 0) return hipSuccess;
#define RAR_FS(DTV)                                                                         \
  if (feedback == 1) fold_state_dispatch<DTV, 1>(bufs, state, n, count, L, block, mbits, stream); \
  else fold_state_dispatch<DTV, 2>(bufs, state, n, count, L, block, mbits, stream);
  switch (dt) {
    case DT_F32: RAR_FS(DT_F32) break;
    case DT_F16: RAR_FS(DT_F16) break;
    default: RAR_FS(DT_BF16) break;
  }
#undef RAR_FS
  return launch_status(stream);
}

hipError_t launch_fill_u64(uint64_t* dst, const uint64_t* host_vals, int nvals, hipStream_t stream) {
  for (int base = 0; base < nvals; base += kFillWords) {
    U64Vals vals{};
    const int n = nvals - base < kFillWords ? nvals - base : kFillWords;
    for (int i = 0; i < n; ++i) vals.v[i] = host_vals[base + i];
    hipLaunchKernelGGL(fill_u64_kernel, dim3(1), dim3(256), 0, stream, dst + base, n, vals);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace rar
