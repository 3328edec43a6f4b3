// Device functions of the block-floating-point codec, shared by the BFP
// kernels and the sparse-or-BFP kernels of the compressed ring.
//
// Lane layout: a lane owns 8 consecutive elements, so a block of B elements
// is B/8 consecutive lanes of a wavefront (16 lanes = one DPP row for B = 128).
// The block exponent E is the max of |x| binary32 bit patterns reduced across
// those lanes, shifted down by 23 (255 when an Inf/NaN is present).
#pragma once

#include "launch.hpp"

namespace rar {

// Cross-lane max for a runtime lanes-per-block (power of two, 2..64).
__device__ __forceinline__ uint32_t group_max_dyn(uint32_t v, int lpb) {
  switch (lpb) {
    case 2: return group_max_u32<2>(v);
    case 4: return group_max_u32<4>(v);
    case 8: return group_max_u32<8>(v);
    case 16: return group_max_u32<16>(v);
    case 32: return group_max_u32<32>(v);
    default: return group_max_u32<64>(v);
  }
}

template <int LPB>
__device__ __forceinline__ uint32_t group_max_sel(uint32_t v, int lpb) {
  if constexpr (LPB > 0) return group_max_u32<LPB>(v);
  else return group_max_dyn(v, lpb);
}

__device__ __forceinline__ uint32_t lane_absmax(const G8& x) {
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) m = max(m, absbits(x.v[i]));
  return m;
}

// Quantise-dequantise a lane's 8 elements with the block's scale.
__device__ __forceinline__ G8 qdq8(const G8& x, const BfpScale& sc, float qmax) {
  G8 d;
  const float nanv = __builtin_nanf("");
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    float v = bfp_dq(bfp_q(x.v[i], sc.k, qmax), sc.k);
    d.v[i] = sc.nan ? nanv : v;
  }
  return d;
}

template <int DT>
__device__ __forceinline__ G8 load_group(const char* base, uint64_t elem, int nv) {
  return nv == 8 ? unpack8<DT>(load_raw8<DT, false>(base, elem)) : load_part8<DT>(base, elem, nv);
}

template <int DT>
__device__ __forceinline__ void store_group(char* base, uint64_t elem, int nv, const G8& g) {
  if (nv == 8) store_raw8<DT, false>(base, elem, pack8<DT>(g));
  else store_part8<DT>(base, elem, nv, g);
}

// Encode one lane's 8 elements (nv valid, starting at element `elem` of the
// message's data): the first lane of each block writes the exponent byte,
// every lane writes its mantissas (8 int8 or 8 nibbles).  All lanes of the
// wavefront must call this together (cross-lane max).
template <int DT, int LPB>
__device__ __forceinline__ void encode_group(const G8& x, int nv, uint64_t elem, uint8_t* msg, uint8_t* mant,
                                             int lpb, int mbits, float qmax) {
  const uint64_t block = (uint64_t)lpb * 8;
  const uint32_t m = group_max_sel<LPB>(lane_absmax(x), lpb);
  const BfpScale sc = bfp_scale(m, mbits);
  if (nv > 0 && (threadIdx.x & (lpb - 1)) == 0) msg[elem / block] = (uint8_t)(m >> 23);
  int q[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) q[i] = sc.nan ? 0 : (int)bfp_q(x.v[i], sc.k, qmax);
  if (mbits > 4) {
    u32x2 w;
    w[0] = (uint32_t)(q[0] & 0xff) | (uint32_t)(q[1] & 0xff) << 8 | (uint32_t)(q[2] & 0xff) << 16 |
           (uint32_t)(q[3] & 0xff) << 24;
    w[1] = (uint32_t)(q[4] & 0xff) | (uint32_t)(q[5] & 0xff) << 8 | (uint32_t)(q[6] & 0xff) << 16 |
           (uint32_t)(q[7] & 0xff) << 24;
    if (nv == 8) {
      *(u32x2*)(mant + elem) = w;
    } else {
      for (int i = 0; i < nv; ++i) mant[elem + i] = (uint8_t)q[i];
    }
  } else {
    uint32_t w = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) w |= (uint32_t)(q[i] & 0xf) << (4 * i);
    if (nv == 8) {
      *(uint32_t*)(mant + elem / 2) = w;
    } else {
      for (int i = 0; i < (nv + 1) / 2; ++i) mant[elem / 2 + i] = (uint8_t)(w >> (8 * i));
    }
  }
}

// ---------------------------------------------------------------- decode (K5)
__device__ __forceinline__ G8 dequant_group(const uint8_t* msg, uint64_t eb, uint64_t elem, int nv,
                                            uint64_t block, int mbits) {
  const int E = msg[elem / block];
  const int e = (E < 1 ? 1 : E) - 127;
  const int k = mbits - 2 - e;
  const uint8_t* mant = msg + eb;
  int q[8];
  if (mbits > 4) {
    if (nv == 8) {
      u32x2 w = *(const u32x2*)(mant + elem);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        q[i] = (int)(int8_t)(w[0] >> (8 * i));
        q[4 + i] = (int)(int8_t)(w[1] >> (8 * i));
      }
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) q[i] = i < nv ? (int)(int8_t)mant[elem + i] : 0;
    }
  } else {
    uint32_t w = 0;
    if (nv == 8) {
      w = *(const uint32_t*)(mant + elem / 2);
    } else {
      for (int i = 0; i < (nv + 1) / 2; ++i) w |= (uint32_t)mant[elem / 2 + i] << (8 * i);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) q[i] = ((int)(w << (28 - 4 * i))) >> 28;  // sign-extend nibble i
  }
  G8 d;
  const float nanv = __builtin_nanf("");
#pragma unroll
  for (int i = 0; i < 8; ++i) d.v[i] = E == 255 ? nanv : bfp_dq((float)q[i], k);
  return d;
}

}  // namespace rar
