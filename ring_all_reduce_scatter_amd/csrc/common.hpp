// Device-side helpers shared by the kernels of librar.so (gfx950 / CDNA4).
//
// Data layout convention: a lane ("group") owns 8 consecutive elements of a
// buffer: one 16-byte vector for fp16/bf16, two for fp32.  A BFP block of B
// elements is then B/8 consecutive lanes of one wavefront, so the block's
// shared exponent is a cross-lane max inside a DPP row (B <= 128) or across
// rows (B = 256, 512).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rar {

enum Dtype : int { DT_F32 = 0, DT_F16 = 1, DT_BF16 = 2 };

constexpr int kMaxRanks = 64;
constexpr int kThreads = 256;   // workgroup size of every streaming kernel
constexpr int kGroupElems = 8;  // elements per lane-group

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

struct RankPtrs {
  char* p[kMaxRanks];
};

template <int DT>
struct DtypeSize {
  static constexpr int value = DT == DT_F32 ? 4 : 2;
};

// ------------------------------------------------------------ conversions
// binary16 and bfloat16: the gfx950 conversion instructions (v_cvt_f16_f32,
// v_cvt_pk_bf16_f32) round to nearest even under the default mode and keep
// subnormals; widening is exact (bfloat16 is the upper half of a binary32).

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 b16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float h16_to_f32(uint32_t h) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}
__device__ __forceinline__ uint32_t f32_to_h16(float f) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)f);
}
__device__ __forceinline__ float b16_to_f32(uint32_t h) { return __uint_as_float(h << 16); }
__device__ __forceinline__ uint32_t f32_to_b16(float f) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)f);
}
// Two binary32 values to packed bfloat16 (lo in bits 15:0) in one instruction.
__device__ __forceinline__ uint32_t f32x2_to_b16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){lo, hi}, b16x2));
}

template <int DT>
__device__ __forceinline__ float widen16(uint32_t h) {
  return DT == DT_F16 ? h16_to_f32(h) : b16_to_f32(h);
}
template <int DT>
__device__ __forceinline__ uint32_t narrow16(float f) {
  return DT == DT_F16 ? f32_to_h16(f) : f32_to_b16(f);
}

// Two binary32 values rounded to a 16-bit type, packed (first in bits 15:0).
template <int DT>
__device__ __forceinline__ uint32_t pack_pair(float lo, float hi) {
  if constexpr (DT == DT_BF16) return f32x2_to_b16x2(lo, hi);
  else return narrow16<DT>(lo) | (narrow16<DT>(hi) << 16);
}

// Round a binary32 value to the dtype and return it widened again.
template <int DT>
__device__ __forceinline__ float round_to(float f) {
  if constexpr (DT == DT_F32) return f;
  else return widen16<DT>(narrow16<DT>(f));
}

// ------------------------------------------------------------ 8-element groups

struct G8 {
  float v[8];
};

template <bool NT>
__device__ __forceinline__ u32x4 ld16(const char* p) {
  if constexpr (NT) return __builtin_nontemporal_load((const u32x4*)p);
  else return *(const u32x4*)p;
}
template <bool NT>
__device__ __forceinline__ void st16(char* p, u32x4 v) {
  if constexpr (NT) __builtin_nontemporal_store(v, (u32x4*)p);
  else *(u32x4*)p = v;
}

// Write-through stores for streaming outputs: 16-byte lane stores that are
// nontemporal and at device scope (the nt and sc1 cache-policy bits), so
// each output line goes on towards HBM as it is written instead of sitting
// dirty in the L2 until an eviction writes it back among the reads.  Global
// stores take no such bits, so these go through a buffer descriptor over a
// workgroup-uniform byte range [base, base + bytes) (scalar registers),
// each lane giving its byte offset in the range; a store past the range is
// dropped by the hardware.  Measured on the fused fold pattern (8 ranks x
// 256 MiB fp32, one launch): 680 us with these stores against 709 us with
// nontemporal stores alone (0.79 against 0.76 of 8 TB/s); device scope
// alone, without nt, gained nothing.
typedef __amdgpu_buffer_rsrc_t WtRange;
// base must be the same in every lane of the wavefront (it is taken from the
// first active lane, so the compiler keeps the descriptor in scalar
// registers where it cannot prove that itself).
__device__ __forceinline__ WtRange wt_range(const char* base, uint32_t bytes) {
  const uint64_t b = (uint64_t)base;
  // (readfirstlane returns int: zero-extend each half through uint32_t)
  const uint64_t u = (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b) |
                     (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32)) << 32;
  return __builtin_amdgcn_make_buffer_rsrc((void*)u, (short)0, (int)bytes, 0x00020000);
}
constexpr int kNtSc1 = 2 | 16;  // cache-policy operand: nt (bit 1), sc1 (bit 4)
__device__ __forceinline__ void st16_wt(WtRange r, uint32_t off, u32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, (int)off, 0, kNtSc1);
}
__device__ __forceinline__ void st8_wt(WtRange r, uint32_t off, u32x2 v) {
  __builtin_amdgcn_raw_buffer_store_b64(v, r, (int)off, 0, kNtSc1);
}

// Raw 8-element group as stored (fp32: 8 words; 16-bit: 4 words).
template <int DT>
struct Raw8 {
  u32x4 w[DT == DT_F32 ? 2 : 1];
};

// A whole group stored write-through at byte offset off of range r.
template <int DT>
__device__ __forceinline__ void store_raw8_wt(WtRange r, uint32_t off, const Raw8<DT>& v) {
  st16_wt(r, off, v.w[0]);
  if constexpr (DT == DT_F32) st16_wt(r, off + 16, v.w[1]);
}

template <int DT, bool NT>
__device__ __forceinline__ Raw8<DT> load_raw8(const char* base, uint64_t elem) {
  Raw8<DT> r;
  const char* p = base + elem * DtypeSize<DT>::value;
  r.w[0] = ld16<NT>(p);
  if constexpr (DT == DT_F32) r.w[1] = ld16<NT>(p + 16);
  return r;
}

template <int DT, bool NT>
__device__ __forceinline__ void store_raw8(char* base, uint64_t elem, const Raw8<DT>& r) {
  char* p = base + elem * DtypeSize<DT>::value;
  st16<NT>(p, r.w[0]);
  if constexpr (DT == DT_F32) st16<NT>(p + 16, r.w[1]);
}

template <int DT>
__device__ __forceinline__ G8 unpack8(const Raw8<DT>& r) {
  G8 g;
  if constexpr (DT == DT_F32) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      g.v[i] = __uint_as_float(r.w[0][i]);
      g.v[4 + i] = __uint_as_float(r.w[1][i]);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      g.v[2 * i] = widen16<DT>(r.w[0][i] & 0xffffu);
      g.v[2 * i + 1] = widen16<DT>(r.w[0][i] >> 16);
    }
  }
  return g;
}

template <int DT>
__device__ __forceinline__ Raw8<DT> pack8(const G8& g) {
  Raw8<DT> r;
  if constexpr (DT == DT_F32) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      r.w[0][i] = __float_as_uint(g.v[i]);
      r.w[1][i] = __float_as_uint(g.v[4 + i]);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) r.w[0][i] = pack_pair<DT>(g.v[2 * i], g.v[2 * i + 1]);
  }
  return r;
}

// 16-byte vectors: 4 fp32 or 8 fp16/bf16 elements.  In the streaming
// kernels lane t of a workgroup touches bytes [16 t, 16 t + 16) of each
// 16*kThreads-byte slab, so every load or store instruction of a wavefront
// covers 1 KiB of contiguous memory.
template <int DT>
struct Vec {
  static constexpr int E = 16 / DtypeSize<DT>::value;
  float v[E];
};

template <int DT>
__device__ __forceinline__ Vec<DT> unpack16(u32x4 w) {
  Vec<DT> x;
  if constexpr (DT == DT_F32) {
#pragma unroll
    for (int i = 0; i < 4; ++i) x.v[i] = __uint_as_float(w[i]);
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x.v[2 * i] = widen16<DT>(w[i] & 0xffffu);
      x.v[2 * i + 1] = widen16<DT>(w[i] >> 16);
    }
  }
  return x;
}

template <int DT>
__device__ __forceinline__ u32x4 pack16(const Vec<DT>& x) {
  u32x4 w;
  if constexpr (DT == DT_F32) {
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = __float_as_uint(x.v[i]);
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = pack_pair<DT>(x.v[2 * i], x.v[2 * i + 1]);
  }
  return w;
}

template <int DT>
__device__ __forceinline__ float load_elem(const char* base, uint64_t i) {
  if constexpr (DT == DT_F32) return ((const float*)base)[i];
  else return widen16<DT>(((const uint16_t*)base)[i]);
}

template <int DT>
__device__ __forceinline__ void store_elem(char* base, uint64_t i, float x) {
  if constexpr (DT == DT_F32) ((float*)base)[i] = x;
  else ((uint16_t*)base)[i] = (uint16_t)narrow16<DT>(x);
}

// Element-wise access for ragged tails (elements [elem, elem+n), n < 8);
// missing elements read as +0.
template <int DT>
__device__ __forceinline__ G8 load_part8(const char* base, uint64_t elem, int n) {
  G8 g;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    float x = 0.0f;
    if (i < n) {
      if constexpr (DT == DT_F32) x = ((const float*)base)[elem + i];
      else x = widen16<DT>(((const uint16_t*)base)[elem + i]);
    }
    g.v[i] = x;
  }
  return g;
}

template <int DT>
__device__ __forceinline__ void store_part8(char* base, uint64_t elem, int n, const G8& g) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    if (i < n) {
      if constexpr (DT == DT_F32) ((float*)base)[elem + i] = g.v[i];
      else ((uint16_t*)base)[elem + i] = (uint16_t)narrow16<DT>(g.v[i]);
    }
  }
}

// ------------------------------------------------------------ cross-lane max
// Max over aligned groups of LPB consecutive lanes (LPB a power of two <= 64),
// every lane of the group receives the result.  Inside a 16-lane DPP row the
// butterfly uses quad_perm [1,0,3,2], quad_perm [2,3,0,1], row_half_mirror and
// row_mirror; wider groups use ds_bpermute swaps.  All lanes must be active.

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, CTRL, 0xF, 0xF, false);
}

constexpr int kDppQuad1032 = 0xB1;       // quad_perm:[1,0,3,2]
constexpr int kDppQuad2301 = 0x4E;       // quad_perm:[2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141;
constexpr int kDppRowMirror = 0x140;

template <int LPB>
__device__ __forceinline__ uint32_t group_max_u32(uint32_t v) {
  if constexpr (LPB >= 2) v = max(v, dpp_u32<kDppQuad1032>(v));
  if constexpr (LPB >= 4) v = max(v, dpp_u32<kDppQuad2301>(v));
  if constexpr (LPB >= 8) v = max(v, dpp_u32<kDppRowHalfMirror>(v));
  if constexpr (LPB >= 16) v = max(v, dpp_u32<kDppRowMirror>(v));
  if constexpr (LPB >= 32) v = max(v, (uint32_t)__shfl_xor((int)v, 16, 64));
  if constexpr (LPB >= 64) v = max(v, (uint32_t)__shfl_xor((int)v, 32, 64));
  return v;
}

// ------------------------------------------------------------ BFP arithmetic
// Block exponent from the max of |x| bit patterns (binary32): E = bits >> 23.
// With e = max(E,1) - 127 and k = m - 2 - e:
//   q = clamp(rne(x * 2^k), +-qmax),  value = q * 2^-k  (exact in binary32).
// ldexp scales exactly (a result in the subnormal range is below 1/2 and
// rounds to q = 0 either way); q + 0 turns a -0 from rne into +0, so a zero
// mantissa always decodes to +0 as its integer form does.

struct BfpScale {
  int k;       // m - 2 - e
  bool nan;    // E == 255
};

__device__ __forceinline__ uint32_t absbits(float x) { return __float_as_uint(x) & 0x7fffffffu; }

__device__ __forceinline__ BfpScale bfp_scale(uint32_t blockmax_bits, int mbits) {
  int E = (int)(blockmax_bits >> 23);
  BfpScale s;
  s.nan = E == 255;
  int e = (E < 1 ? 1 : E) - 127;
  s.k = mbits - 2 - e;
  return s;
}

__device__ __forceinline__ float bfp_q(float x, int k, float qmax) {
  float q = __builtin_rintf(__builtin_amdgcn_ldexpf(x, k));
  q = __builtin_fminf(__builtin_fmaxf(q, -qmax), qmax);
  return q + 0.0f;
}

__device__ __forceinline__ float bfp_dq(float q, int k) { return __builtin_amdgcn_ldexpf(q, -k); }

}  // namespace rar
