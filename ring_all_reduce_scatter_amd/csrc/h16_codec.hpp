// Packed binary16 block-floating-point codec for blocks of 128 elements
// (16 lanes of 8 elements), shared by the pipelined compressed rings.  It
// gives the same exponent bytes and mantissas as the binary32 formulation
// of the codec (bfp_device.hpp) for binary16 data.
#pragma once

#include "common.hpp"

namespace rar {

// One lane's 8 binary16 elements (4 words) against a block of 128 = 16
// lanes.  Scaling s = h * 2^k by v_ldexp_f16 is exact, t = s + 1536 puts s on
// the binary16 grid of spacing 1 in [1024, 2048) (round half to even), and
// the clamp works on the bit patterns.  Then the low byte (m > 4) or low
// nibble (m <= 4) of t's pattern is q in two's complement, because
// 1536 = 0x6600 has a zero low byte.  Decoding reverses it: the pattern of
// 1536 + q is (b ^ 0x80) + 0x6580 for a byte b and (n ^ 8) + 0x65f8 for a
// nibble n; subtracting 1536 gives q exactly and v_ldexp_f16 scales it by
// 2^-k, exact in binary16 (see the packed hop of the fused fold).
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ h2 as_h2(uint32_t w) { return __builtin_bit_cast(h2, w); }
__device__ __forceinline__ uint32_t h2_bits(h2 v) { return __builtin_bit_cast(uint32_t, v); }
__device__ __forceinline__ u16x2 as_u16x2(uint32_t w) { return __builtin_bit_cast(u16x2, w); }
__device__ __forceinline__ _Float16 ldexp_h(_Float16 x, int k) { return (_Float16)__builtin_amdgcn_ldexph(x, k); }

struct H16Code {
  uint32_t E;      // biased binary32 exponent of the block max (255: Inf/NaN)
  u32x2 bytes;     // m > 4: 8 int8 mantissas; m <= 4: bytes.x holds 8 nibbles
};

// Block exponent and mantissas of 8 halves; all lanes of the wavefront call
// this together (cross-lane max over the block's 16 lanes).
__device__ __forceinline__ H16Code enc_h16x8(u32x4 p, int mbits) {
  u16x2 m = __builtin_elementwise_max(as_u16x2(p[0] & 0x7fff7fffu), as_u16x2(p[1] & 0x7fff7fffu));
  m = __builtin_elementwise_max(m, as_u16x2(p[2] & 0x7fff7fffu));
  m = __builtin_elementwise_max(m, as_u16x2(p[3] & 0x7fff7fffu));
  uint32_t mm = max((uint32_t)m[0], (uint32_t)m[1]);
  mm = group_max_u32<16>(mm);
  H16Code out;
  out.E = __float_as_uint(h16_to_f32(mm)) >> 23;
  const int E = (int)out.E;
  const int k = mbits - 2 - ((E < 1 ? 1 : E) - 127);
  const uint32_t qm = (uint32_t)((1 << (mbits - 1)) - 1);
  const u16x2 lo = {(uint16_t)(0x6600u - qm), (uint16_t)(0x6600u - qm)};
  const u16x2 hi = {(uint16_t)(0x6600u + qm), (uint16_t)(0x6600u + qm)};
  const h2 magic = {(_Float16)1536.0f, (_Float16)1536.0f};
  uint32_t t[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const h2 x = as_h2(p[i]);
    const h2 sc = {ldexp_h(x[0], k), ldexp_h(x[1], k)};
    const u16x2 c = __builtin_elementwise_min(__builtin_elementwise_max(as_u16x2(h2_bits(sc + magic)), lo), hi);
    t[i] = __builtin_bit_cast(uint32_t, c);
  }
  const bool special = mm >= 0x7c00u;  // Inf or NaN in the block: every mantissa 0
  if (mbits > 4) {
    // low byte of each half: bytes 0 and 2 of every word
    out.bytes[0] = special ? 0u : __builtin_amdgcn_perm(t[1], t[0], 0x06040200u);
    out.bytes[1] = special ? 0u : __builtin_amdgcn_perm(t[3], t[2], 0x06040200u);
  } else {
    uint32_t w = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) w |= ((t[i] & 0xfu) | ((t[i] >> 12) & 0xf0u)) << (8 * i);
    out.bytes[0] = special ? 0u : w;
    out.bytes[1] = 0u;
  }
  return out;
}

// Decoded values of a lane's 8 mantissas (packed binary16; NaN for E = 255).
__device__ __forceinline__ u32x4 dec_h16x8(uint32_t E, u32x2 w, int mbits) {
  const int k = mbits - 2 - (((int)E < 1 ? 1 : (int)E) - 127);
  const h2 magic = {(_Float16)1536.0f, (_Float16)1536.0f};
  uint32_t t[4];
  if (mbits > 4) {
    const uint32_t x0 = w[0] ^ 0x80808080u, x1 = w[1] ^ 0x80808080u;
    t[0] = __builtin_amdgcn_perm(0u, x0, 0x0c010c00u) + 0x65806580u;
    t[1] = __builtin_amdgcn_perm(0u, x0, 0x0c030c02u) + 0x65806580u;
    t[2] = __builtin_amdgcn_perm(0u, x1, 0x0c010c00u) + 0x65806580u;
    t[3] = __builtin_amdgcn_perm(0u, x1, 0x0c030c02u) + 0x65806580u;
  } else {
    const uint32_t x = w[0] ^ 0x88888888u;
#pragma unroll
    for (int i = 0; i < 4; ++i) t[i] = (((x >> (8 * i)) & 0xfu) | (((x >> (8 * i + 4)) & 0xfu) << 16)) + 0x65f865f8u;
  }
  u32x4 d;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const h2 q = as_h2(t[i]) - magic;
    const h2 v = {ldexp_h(q[0], -k), ldexp_h(q[1], -k)};
    d[i] = E == 255u ? 0x7e007e00u : h2_bits(v);
  }
  return d;
}

// Non-zero elements of a lane's 8 halves (+-0 counts as zero, NaN does not).
__device__ __forceinline__ uint32_t nonzeros_h16x8(u32x4 p) {
  uint32_t c = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) c += ((p[i] & 0x7fffu) != 0u ? 1u : 0u) + ((p[i] & 0x7fff0000u) != 0u ? 1u : 0u);
  return c;
}

// Halves nv .. 7 of a lane's group set to +0 (nv = 8 leaves it unchanged).
__device__ __forceinline__ u32x4 keep_h16x8(u32x4 p, int nv) {
#pragma unroll
  for (int i = 0; i < 8; ++i)
    if (i >= nv) p[i >> 1] &= (i & 1) ? 0x0000ffffu : 0xffff0000u;
  return p;
}

}  // namespace rar
