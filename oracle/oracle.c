/*
 * oracle.c -- plain, slow, single-threaded CPU reference for the ring
 * all-reduce family and its compression-coupled variant.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file.  Only the test-suite, the smoke check and the CPU-baseline
 * leg of the benchmark use it, to decide whether the GPU library is right.
 * It shares no source with the GPU library: its own IEEE-754 conversions,
 * its own chunk rule, its own encoders.
 *
 * Sources (cited by page title and section):
 *  [P2] "从零实现集合通信" (collective ops from scratch), section on the
 *       two-pass ring allreduce and its per-rank byte table; the glossary
 *       (allreduce leaves every rank holding the same reduced tensor).
 *  [P4] "CCCL通信压缩库：突破LLM训练通信墙的工程实践", section 2.1 (layered
 *       compression: sparse value+index layer, block floating point layer,
 *       operator-aware layer) and section 2.2 (chunked compress ->
 *       communicate -> receiver decompress -> reduce pipeline).
 *
 * Readings of points the pages leave open (each is listed in the design
 * notes of the repository):
 *  - Steps are numbered s = 1..N-1; at RS step s rank r receives chunk
 *    (r-s-1) mod N from rank r-1 and adds it to its own copy (local + received).
 *  - At AG step s rank r receives chunk (r-s) mod N from rank r-1 and stores it.
 *  - Chunk length L = roundup(ceil(T/N), A), A = 128 elements (A = max(128,
 *    block) in the compressed ring); trailing chunks may be short or empty.
 *  - The reduce op is SUM.  fp32 adds are binary32 round-to-nearest-even;
 *    fp16/bf16 adds widen both operands to binary32, add, and round back.
 *  - BFP block: E = biased binary32 exponent of the block's largest |x|,
 *    e = max(E,1)-127, q = clamp(RNE(x * 2^(m-2-e)), +-(2^(m-1)-1)),
 *    decoded value q * 2^(e+2-m).  m counts the sign bit.  E = 255 (Inf/NaN
 *    in the block) decodes to NaN.
 *  - Sparse layer: zeros are +-0; a unit is sent as values+uint32 indices iff
 *    zeros > threshold * len.
 *
 * Floating point: binary32 adds are done in C `float` (SSE, no contraction:
 * build with -ffp-contract=off and without -ffast-math).  Quantisation
 * scaling is done in binary64, where every step used here is exact.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { ORC_F32 = 0, ORC_F16 = 1, ORC_BF16 = 2 };
enum { ORC_OK = 0, ORC_EINVAL = 1 };
enum { ORC_COMP_BFP = 1, ORC_COMP_SPARSE_AUTO = 2 };

#define ORC_MAXN 64

/* ------------------------------------------------------------------ */
/* IEEE-754 small formats, written from the format definition.          */
/* binary16: 5 exponent bits (bias 15), 10 fraction bits.               */
/* bfloat16: 8 exponent bits (bias 127), 7 fraction bits.               */
/* ------------------------------------------------------------------ */

static double small_decode(uint16_t h, int eb, int fb) {
  int bias = (1 << (eb - 1)) - 1;
  unsigned s = h >> 15;
  unsigned E = (h >> fb) & ((1u << eb) - 1u);
  unsigned F = h & ((1u << fb) - 1u);
  double mag;
  if (E == (1u << eb) - 1u)
    mag = F ? NAN : INFINITY;
  else if (E == 0)
    mag = ldexp((double)F, 1 - bias - fb);
  else
    mag = ldexp((double)((1u << fb) + F), (int)E - bias - fb);
  return s ? -mag : mag;
}

/* Round the real number x (given exactly as a double) to the nearest value
 * of the format, ties to the even significand, and return its encoding. */
static uint16_t small_encode(double x, int eb, int fb) {
  int bias = (1 << (eb - 1)) - 1;
  unsigned emax_field = (1u << eb) - 1u;
  int emin = 1 - bias; /* exponent of the smallest normal number */
  uint16_t sign = signbit(x) ? 0x8000u : 0u;
  if (isnan(x)) return (uint16_t)(0x7FFFu & ((emax_field << fb) | (1u << (fb - 1))));
  double a = fabs(x);
  if (a == 0.0) return sign;
  if (isinf(a)) return (uint16_t)(sign | (emax_field << fb));
  int e;
  frexp(a, &e);
  e -= 1; /* 2^e <= a < 2^(e+1) */
  if (e < emin) e = emin;                 /* subnormal range: fixed spacing */
  double quantum = ldexp(1.0, e - fb);    /* spacing of representable values */
  double n = a / quantum;                 /* exact: division by a power of 2 */
  double fl = floor(n);
  double rem = n - fl;
  if (rem > 0.5 || (rem == 0.5 && fmod(fl, 2.0) != 0.0)) fl += 1.0;
  double r = fl * quantum;
  if (r == 0.0) return sign;
  frexp(r, &e);
  e -= 1;
  if (e < emin) /* subnormal result */
    return (uint16_t)(sign | (unsigned)(r / ldexp(1.0, emin - fb)));
  if (e + bias >= (int)emax_field) return (uint16_t)(sign | (emax_field << fb)); /* overflow */
  unsigned F = (unsigned)(r / ldexp(1.0, e - fb)) - (1u << fb);
  return (uint16_t)(sign | ((unsigned)(e + bias) << fb) | F);
}

float orc_f16_to_f32(uint16_t h) { return (float)small_decode(h, 5, 10); }
uint16_t orc_f32_to_f16(float f) { return small_encode((double)f, 5, 10); }
float orc_bf16_to_f32(uint16_t h) { return (float)small_decode(h, 8, 7); }
uint16_t orc_f32_to_bf16(float f) { return small_encode((double)f, 8, 7); }

static size_t dtype_size(int dt) { return dt == ORC_F32 ? 4 : 2; }
static int dtype_ok(int dt) { return dt == ORC_F32 || dt == ORC_F16 || dt == ORC_BF16; }

/* Exact widening of element i to binary32. */
static float widen(const void* base, size_t i, int dt) {
  if (dt == ORC_F32) return ((const float*)base)[i];
  uint16_t h = ((const uint16_t*)base)[i];
  return dt == ORC_F16 ? orc_f16_to_f32(h) : orc_bf16_to_f32(h);
}

/* Round-to-nearest-even store of a binary32 value into element i. */
static void narrow_store(void* base, size_t i, int dt, float v) {
  if (dt == ORC_F32) {
    ((float*)base)[i] = v;
  } else {
    ((uint16_t*)base)[i] = dt == ORC_F16 ? orc_f32_to_f16(v) : orc_f32_to_bf16(v);
  }
}

/* local <- local (+) received: binary32 add, then round to the dtype. */
static void accumulate(void* base, size_t i, int dt, float received) {
  float local = widen(base, i, dt);
  float sum = local + received;
  narrow_store(base, i, dt, sum);
}

/* Convert n elements between dtypes (widen exactly, round to nearest even). */
int orc_convert(const void* src, int sdt, void* dst, int ddt, size_t n) {
  if (!dtype_ok(sdt) || !dtype_ok(ddt)) return ORC_EINVAL;
  for (size_t i = 0; i < n; ++i) narrow_store(dst, i, ddt, widen(src, i, sdt));
  return ORC_OK;
}

/* ------------------------------------------------------------------ */
/* Chunk rule and ring schedule                                         */
/* ------------------------------------------------------------------ */

size_t orc_chunk_len(size_t count, int nranks, size_t align) {
  if (nranks < 1 || align == 0) return 0;
  size_t per = (count + (size_t)nranks - 1) / (size_t)nranks;
  return (per + align - 1) / align * align;
}

static void chunk_range(size_t count, size_t L, int c, size_t* lo, size_t* hi) {
  size_t a = (size_t)c * L, b = a + L;
  *lo = a < count ? a : count;
  *hi = b < count ? b : count;
}

static int modn(int a, int n) { return ((a % n) + n) % n; }

static int check_bufs(void* const* bufs, int n, int dt) {
  if (n < 1 || n > ORC_MAXN || !dtype_ok(dt) || !bufs) return 0;
  for (int r = 0; r < n; ++r)
    if (!bufs[r]) return 0;
  return 1;
}

static void add_traffic(uint64_t* sent, uint64_t* recv, int from, int to, uint64_t bytes) {
  if (sent) sent[from] += bytes;
  if (recv) recv[to] += bytes;
}

/* One reduce-scatter step s (1..N-1) with chunk length L ([P2] two-pass ring):
 * every rank r receives chunk (r-s-1) mod N from rank (r-1) mod N and adds it
 * into its own copy.  In a step rank r writes only chunk (r-s-1) and rank r-1
 * writes only chunk (r-s-2), so visiting the ranks one after another gives
 * the same result as all of them acting at once. */
static void rs_step_L(void* const* bufs, int n, size_t count, int dt, int s, size_t L,
                      uint64_t* sent, uint64_t* recv) {
  size_t es = dtype_size(dt);
  for (int r = 0; r < n; ++r) {
    int src = modn(r - 1, n);
    int c = modn(r - s - 1, n);
    size_t lo, hi;
    chunk_range(count, L, c, &lo, &hi);
    for (size_t i = lo; i < hi; ++i) accumulate(bufs[r], i, dt, widen(bufs[src], i, dt));
    add_traffic(sent, recv, src, r, (uint64_t)(hi - lo) * es);
  }
}

/* One allgather step s (1..N-1): rank r receives finished chunk (r-s) mod N
 * from rank (r-1) mod N and stores it. */
static void ag_step_L(void* const* bufs, int n, size_t count, int dt, int s, size_t L,
                      uint64_t* sent, uint64_t* recv) {
  size_t es = dtype_size(dt);
  for (int r = 0; r < n; ++r) {
    int src = modn(r - 1, n);
    int c = modn(r - s, n);
    size_t lo, hi;
    chunk_range(count, L, c, &lo, &hi);
    memcpy((char*)bufs[r] + lo * es, (const char*)bufs[src] + lo * es, (hi - lo) * es);
    add_traffic(sent, recv, src, r, (uint64_t)(hi - lo) * es);
  }
}

int orc_rs_step(void* const* bufs, int n, size_t count, int dt, int s) {
  if (!check_bufs(bufs, n, dt) || s < 1 || s > n - 1) return ORC_EINVAL;
  rs_step_L(bufs, n, count, dt, s, orc_chunk_len(count, n, 128), NULL, NULL);
  return ORC_OK;
}

int orc_ag_step(void* const* bufs, int n, size_t count, int dt, int s) {
  if (!check_bufs(bufs, n, dt) || s < 1 || s > n - 1) return ORC_EINVAL;
  ag_step_L(bufs, n, count, dt, s, orc_chunk_len(count, n, 128), NULL, NULL);
  return ORC_OK;
}

/* Reduce-scatter: the first pass alone.  Afterwards rank r's chunk r holds
 * the full sum of chunk r; other chunks hold partial sums. */
int orc_reduce_scatter(void* const* bufs, int n, size_t count, int dt, uint64_t* sent,
                       uint64_t* recv) {
  if (!check_bufs(bufs, n, dt)) return ORC_EINVAL;
  size_t L = orc_chunk_len(count, n, 128);
  for (int s = 1; s <= n - 1; ++s) rs_step_L(bufs, n, count, dt, s, L, sent, recv);
  return ORC_OK;
}

/* Ring allreduce: reduce-scatter (N-1 steps) then allgather (N-1 steps). */
int orc_ring_allreduce(void* const* bufs, int n, size_t count, int dt, uint64_t* sent,
                       uint64_t* recv) {
  if (!check_bufs(bufs, n, dt)) return ORC_EINVAL;
  size_t L = orc_chunk_len(count, n, 128);
  for (int s = 1; s <= n - 1; ++s) rs_step_L(bufs, n, count, dt, s, L, sent, recv);
  for (int s = 1; s <= n - 1; ++s) ag_step_L(bufs, n, count, dt, s, L, sent, recv);
  return ORC_OK;
}

/* Allgather over shards: each buffer holds N shards of count/N elements and
 * rank r's own shard sits at shard position r.  N-1 ring rotations. */
int orc_allgather(void* const* bufs, int n, size_t count, int dt, uint64_t* sent,
                  uint64_t* recv) {
  if (!check_bufs(bufs, n, dt) || count % (size_t)n) return ORC_EINVAL;
  size_t L = count / (size_t)n;
  for (int s = 1; s <= n - 1; ++s) ag_step_L(bufs, n, count, dt, s, L, sent, recv);
  return ORC_OK;
}

/* Broadcast along a binomial tree rooted at `root`: in round k = 0,1,...
 * every rank whose distance from the root (rel) is below 2^k sends the whole
 * tensor to rel + 2^k, until every rank holds it (ceil(log2 N) rounds). */
int orc_broadcast(void* const* bufs, int n, size_t count, int dt, int root, uint64_t* sent,
                  uint64_t* recv) {
  if (!check_bufs(bufs, n, dt) || root < 0 || root >= n) return ORC_EINVAL;
  size_t bytes = count * dtype_size(dt);
  for (int span = 1; span < n; span *= 2) {
    for (int rel = 0; rel < span; ++rel) {
      int dst_rel = rel + span;
      if (dst_rel >= n) continue;
      int from = (root + rel) % n, to = (root + dst_rel) % n;
      memcpy(bufs[to], bufs[from], bytes);
      add_traffic(sent, recv, from, to, (uint64_t)bytes);
    }
  }
  return ORC_OK;
}

/* One reduce round of the tree allreduce ([P2] ring-vs-tree table: the
 * tree reduces along a binary tree of depth log2 N).  Round with distance
 * `span` (1, 2, 4, ...): every rank rel with rel % (2*span) == 0 and
 * rel + span < N adds rank rel+span's buffer into its own (local (+)
 * received).  Ranks are counted from rank 0. */
static void tree_reduce_round(void* const* bufs, int n, size_t count, int dt, int span, uint64_t* sent,
                              uint64_t* recv) {
  size_t es = dtype_size(dt);
  for (int rel = 0; rel + span < n; rel += 2 * span) {
    for (size_t i = 0; i < count; ++i) accumulate(bufs[rel], i, dt, widen(bufs[rel + span], i, dt));
    add_traffic(sent, recv, rel + span, rel, (uint64_t)count * es);
  }
}

int orc_tree_reduce_round(void* const* bufs, int n, size_t count, int dt, int span) {
  if (!check_bufs(bufs, n, dt) || span < 1 || span >= n || (span & (span - 1))) return ORC_EINVAL;
  tree_reduce_round(bufs, n, count, dt, span, NULL, NULL);
  return ORC_OK;
}

/* Tree allreduce: ceil(log2 N) reduce rounds into rank 0, then the
 * binomial broadcast from rank 0 (2 ceil(log2 N) steps in all). */
int orc_tree_allreduce(void* const* bufs, int n, size_t count, int dt, uint64_t* sent, uint64_t* recv) {
  if (!check_bufs(bufs, n, dt)) return ORC_EINVAL;
  for (int span = 1; span < n; span *= 2) tree_reduce_round(bufs, n, count, dt, span, sent, recv);
  return orc_broadcast(bufs, n, count, dt, 0, sent, recv);
}

/* The naive allreduce the ring replaces ([P2] problem background): every
 * rank's tensor is gathered at a root and summed there.  Summed in binary64
 * in rank order; for integer-valued inputs every partial sum is exact, which
 * makes it the brute-force answer any summation order must reproduce. */
int orc_naive_sum_f64(const void* const* bufs, int n, size_t count, int dt, double* out) {
  if (n < 1 || n > ORC_MAXN || !dtype_ok(dt) || !out) return ORC_EINVAL;
  for (size_t i = 0; i < count; ++i) {
    double acc = 0.0;
    for (int r = 0; r < n; ++r) acc += (double)widen(bufs[r], i, dt);
    out[i] = acc;
  }
  return ORC_OK;
}

/* ------------------------------------------------------------------ */
/* Block floating point ([P4] section 2.1, numeric-precision layer)     */
/* Message layout: uint8 E[nblocks] padded to a multiple of 16 bytes,   */
/* then the mantissas: one int8 per element when m > 4, else two's-     */
/* complement nibbles, element 2j in bits 3:0 and 2j+1 in bits 7:4.     */
/* ------------------------------------------------------------------ */

static int bfp_args_ok(int block, int mbits) {
  if (mbits < 2 || mbits > 8) return 0;
  if (block < 16 || block > 512 || (block & (block - 1))) return 0;
  return 1;
}

size_t orc_bfp_bytes(size_t count, int block, int mbits) {
  if (!bfp_args_ok(block, mbits)) return 0;
  size_t nb = (count + (size_t)block - 1) / (size_t)block;
  size_t eb = (nb + 15) / 16 * 16;
  size_t mb = mbits > 4 ? count : (count + 1) / 2;
  return eb + mb;
}

/* Biased binary32 exponent of the largest magnitude in x[0..k): 0 when all
 * are zero or below the normal range, 255 when an Inf or NaN is present. */
static int block_exponent(const float* x, size_t k, double* maxabs) {
  double m = 0.0;
  for (size_t i = 0; i < k; ++i) {
    if (isnan(x[i]) || isinf(x[i])) {
      *maxabs = INFINITY;
      return 255;
    }
    double a = fabs((double)x[i]);
    if (a > m) m = a;
  }
  *maxabs = m;
  if (m < ldexp(1.0, -126)) return 0;
  int e;
  frexp(m, &e); /* m = f * 2^e, 0.5 <= f < 1, so floor(log2 m) = e - 1 */
  return e - 1 + 127;
}

/* Nearest integer to d, ties to even (d exact in binary64). */
static double rne(double d) {
  double fl = floor(d), rem = d - fl;
  if (rem > 0.5 || (rem == 0.5 && fmod(fl, 2.0) != 0.0)) fl += 1.0;
  return fl;
}

static void put_q(uint8_t* mant, size_t i, int mbits, int q) {
  if (mbits > 4) {
    mant[i] = (uint8_t)(int8_t)q;
  } else {
    uint8_t nib = (uint8_t)(q & 0xF);
    if (i & 1)
      mant[i / 2] = (uint8_t)((mant[i / 2] & 0x0F) | (nib << 4));
    else
      mant[i / 2] = (uint8_t)((mant[i / 2] & 0xF0) | nib);
  }
}

static int get_q(const uint8_t* mant, size_t i, int mbits) {
  if (mbits > 4) return (int)(int8_t)mant[i];
  int nib = (i & 1) ? (mant[i / 2] >> 4) & 0xF : mant[i / 2] & 0xF;
  return nib >= 8 ? nib - 16 : nib;
}

/* Encode count elements of src (dtype dt) into msg.  If blockmax is given it
 * receives, per block, the largest |x| of that block (Inf for Inf/NaN). */
int orc_bfp_encode(const void* src, int dt, size_t count, int block, int mbits, uint8_t* msg,
                   double* blockmax) {
  if (!bfp_args_ok(block, mbits) || !dtype_ok(dt)) return ORC_EINVAL;
  size_t nb = (count + (size_t)block - 1) / (size_t)block;
  size_t eb = (nb + 15) / 16 * 16;
  memset(msg, 0, orc_bfp_bytes(count, block, mbits));
  uint8_t* mant = msg + eb;
  float* x = (float*)malloc(sizeof(float) * (size_t)block);
  int qmax = (1 << (mbits - 1)) - 1;
  for (size_t b = 0; b < nb; ++b) {
    size_t lo = b * (size_t)block;
    size_t k = count - lo < (size_t)block ? count - lo : (size_t)block;
    for (size_t i = 0; i < k; ++i) x[i] = widen(src, lo + i, dt);
    double mx;
    int E = block_exponent(x, k, &mx);
    if (blockmax) blockmax[b] = mx;
    msg[b] = (uint8_t)E;
    if (E == 255) continue; /* mantissas stay zero; the block decodes to NaN */
    int e = (E < 1 ? 1 : E) - 127;
    for (size_t i = 0; i < k; ++i) {
      double q = rne(ldexp((double)x[i], mbits - 2 - e));
      if (q > qmax) q = qmax;
      if (q < -qmax) q = -qmax;
      put_q(mant, lo + i, mbits, (int)q);
    }
  }
  free(x);
  return ORC_OK;
}

/* Value element i of a BFP message stands for (binary32, exact). */
static float bfp_value(const uint8_t* msg, size_t eb, size_t i, int block, int mbits) {
  int E = msg[i / (size_t)block];
  if (E == 255) return NAN;
  int e = (E < 1 ? 1 : E) - 127;
  int q = get_q(msg + eb, i, mbits);
  return (float)ldexp((double)q, e + 2 - mbits);
}

/* acc <- acc (+) decode(msg), elementwise. */
int orc_bfp_decode_acc(const uint8_t* msg, size_t count, int block, int mbits, void* acc,
                       int dt) {
  if (!bfp_args_ok(block, mbits) || !dtype_ok(dt)) return ORC_EINVAL;
  size_t nb = (count + (size_t)block - 1) / (size_t)block;
  size_t eb = (nb + 15) / 16 * 16;
  for (size_t i = 0; i < count; ++i) accumulate(acc, i, dt, bfp_value(msg, eb, i, block, mbits));
  return ORC_OK;
}

/* dst <- decode(msg), rounded to the dtype. */
int orc_bfp_decode(const uint8_t* msg, size_t count, int block, int mbits, void* dst, int dt) {
  if (!bfp_args_ok(block, mbits) || !dtype_ok(dt)) return ORC_EINVAL;
  size_t nb = (count + (size_t)block - 1) / (size_t)block;
  size_t eb = (nb + 15) / 16 * 16;
  for (size_t i = 0; i < count; ++i) narrow_store(dst, i, dt, bfp_value(msg, eb, i, block, mbits));
  return ORC_OK;
}

/* ------------------------------------------------------------------ */
/* Sparse value+index layer ([P4] section 2.1, sparsity-aware layer)    */
/* Message: uint32 header {nnz, 1, len, 0}; values[nnz] in the dtype;   */
/* padding to 16 bytes; uint32 idx[nnz], ascending, unit-relative.      */
/* ------------------------------------------------------------------ */

static size_t round16(size_t x) { return (x + 15) / 16 * 16; }

size_t orc_sparse_bytes(size_t nnz, int dt) { return 16 + round16(nnz * dtype_size(dt)) + 4 * nnz; }

size_t orc_count_zeros(const void* src, int dt, size_t len) {
  size_t z = 0;
  for (size_t i = 0; i < len; ++i)
    if (widen(src, i, dt) == 0.0f) ++z;
  return z;
}

/* Returns the message size in bytes. */
size_t orc_sparse_encode(const void* src, int dt, size_t len, uint8_t* msg) {
  size_t es = dtype_size(dt);
  size_t nnz = len - orc_count_zeros(src, dt, len);
  uint32_t hdr[4] = {(uint32_t)nnz, 1u, (uint32_t)len, 0u};
  memcpy(msg, hdr, sizeof hdr);
  uint8_t* vals = msg + 16;
  uint32_t* idx = (uint32_t*)(msg + 16 + round16(nnz * es));
  memset(vals, 0, round16(nnz * es));
  size_t j = 0;
  for (size_t i = 0; i < len; ++i) {
    if (widen(src, i, dt) == 0.0f) continue;
    memcpy(vals + j * es, (const char*)src + i * es, es);
    idx[j] = (uint32_t)i;
    ++j;
  }
  return orc_sparse_bytes(nnz, dt);
}

/* acc[idx_j] <- acc[idx_j] (+) v_j; other elements unchanged. */
int orc_sparse_decode_acc(const uint8_t* msg, void* acc, int dt) {
  uint32_t hdr[4];
  memcpy(hdr, msg, sizeof hdr);
  size_t nnz = hdr[0], es = dtype_size(dt);
  const uint8_t* vals = msg + 16;
  const uint32_t* idx = (const uint32_t*)(msg + 16 + round16(nnz * es));
  for (size_t j = 0; j < nnz; ++j) accumulate(acc, idx[j], dt, widen(vals, j, dt));
  return ORC_OK;
}

/* dst <- zeros, then dst[idx_j] <- v_j. */
int orc_sparse_decode(const uint8_t* msg, void* dst, int dt) {
  uint32_t hdr[4];
  memcpy(hdr, msg, sizeof hdr);
  size_t nnz = hdr[0], len = hdr[2], es = dtype_size(dt);
  const uint8_t* vals = msg + 16;
  const uint32_t* idx = (const uint32_t*)(msg + 16 + round16(nnz * es));
  memset(dst, 0, len * es);
  for (size_t j = 0; j < nnz; ++j) memcpy((char*)dst + (size_t)idx[j] * es, vals + j * es, es);
  return ORC_OK;
}

/* ------------------------------------------------------------------ */
/* Compression-coupled ring allreduce ([P4] sections 2.1 and 2.2 on the */
/* [P2] ring).  Every reduce-scatter hop quantises the sender's current */
/* partial of one pipeline unit, the receiver decodes it and adds it to */
/* its own copy.  In the allgather pass the owner encodes each finished */
/* unit once, relays forward those bytes unchanged, and every rank      */
/* (owner included) stores the decoded unit, so all ranks end equal.    */
/* Units split each chunk into pieces of `unit` elements; blocks are    */
/* counted from each unit's start.                                      */
/* ------------------------------------------------------------------ */

typedef struct {
  int method, block, mbits, dt;
  float theta; /* binary32, the type a configuration stores it in */
} comp_t;

/* Encode one unit; returns message size.  For SPARSE_AUTO every message
 * starts with a 16-byte header {nnz, kind, len, 0}: kind 1 is the sparse
 * layout (its own header), kind 0 a BFP payload following the header (nnz
 * unused, 0).  For plain BFP the message is the bare BFP layout. */
static size_t comp_encode(const comp_t* cf, const void* src, size_t len, uint8_t* msg,
                          double* blockmax) {
  if (cf->method == ORC_COMP_BFP) {
    orc_bfp_encode(src, cf->dt, len, cf->block, cf->mbits, msg, blockmax);
    return orc_bfp_bytes(len, cf->block, cf->mbits);
  }
  /* [P4] section 2.1: sparse when the zeros exceed the threshold share of
   * the unit.  The product of the binary32 threshold and the length is taken
   * in binary64, where it is exact for units below 2^29 elements. */
  size_t z = orc_count_zeros(src, cf->dt, len);
  if ((double)z > (double)cf->theta * (double)len) {
    size_t bytes = orc_sparse_encode(src, cf->dt, len, msg);
    if (blockmax) {
      size_t nb = (len + (size_t)cf->block - 1) / (size_t)cf->block;
      for (size_t b = 0; b < nb; ++b) {
        double m = 0.0;
        size_t lo = b * (size_t)cf->block;
        size_t hi = lo + (size_t)cf->block < len ? lo + (size_t)cf->block : len;
        for (size_t i = lo; i < hi; ++i) {
          double a = fabs((double)widen(src, i, cf->dt));
          if (a > m) m = a;
        }
        blockmax[b] = m;
      }
    }
    return bytes;
  }
  uint32_t hdr[4] = {0u, 0u, (uint32_t)len, 0u};
  memcpy(msg, hdr, sizeof hdr);
  orc_bfp_encode(src, cf->dt, len, cf->block, cf->mbits, msg + 16, blockmax);
  return 16 + orc_bfp_bytes(len, cf->block, cf->mbits);
}

static void comp_decode(const comp_t* cf, const uint8_t* msg, size_t len, void* dst, int acc) {
  if (cf->method == ORC_COMP_BFP) {
    if (acc)
      orc_bfp_decode_acc(msg, len, cf->block, cf->mbits, dst, cf->dt);
    else
      orc_bfp_decode(msg, len, cf->block, cf->mbits, dst, cf->dt);
    return;
  }
  uint32_t hdr[4];
  memcpy(hdr, msg, sizeof hdr);
  if (hdr[1] == 1u) { /* word 1 is the kind: 1 = sparse, 0 = BFP */
    if (acc)
      orc_sparse_decode_acc(msg, dst, cf->dt);
    else
      orc_sparse_decode(msg, dst, cf->dt);
  } else {
    if (acc)
      orc_bfp_decode_acc(msg + 16, len, cf->block, cf->mbits, dst, cf->dt);
    else
      orc_bfp_decode(msg + 16, len, cf->block, cf->mbits, dst, cf->dt);
  }
}

static void note_blockmax(double* out, const double* bm, size_t first_block, size_t nb) {
  if (!out) return;
  for (size_t b = 0; b < nb; ++b)
    if (bm[b] > out[first_block + b]) out[first_block + b] = bm[b];
}

size_t orc_comp_chunk_len(size_t count, int n, int block) {
  return orc_chunk_len(count, n, block > 128 ? (size_t)block : 128);
}

/* blockmax_out (optional): per block of the buffer (count/block rounded up),
 * the largest block maximum among all messages that carried that block.
 * unit must be a positive multiple of block. */
int orc_ring_allreduce_compressed(void* const* bufs, int n, size_t count, int dt, int method,
                                  int block, int mbits, float theta, size_t unit,
                                  double* blockmax_out, uint64_t* sent, uint64_t* recv) {
  if (!check_bufs(bufs, n, dt) || !bfp_args_ok(block, mbits)) return ORC_EINVAL;
  if (method != ORC_COMP_BFP && method != ORC_COMP_SPARSE_AUTO) return ORC_EINVAL;
  if (unit == 0 || unit % (size_t)block) return ORC_EINVAL;
  /* One rank sends nothing, so nothing is compressed: the buffer stays as it is. */
  if (n == 1) return ORC_OK;
  comp_t cf = {method, block, mbits, dt, theta};
  size_t es = dtype_size(dt);
  size_t L = orc_comp_chunk_len(count, n, block);
  size_t maxmsg = 16 + orc_bfp_bytes(unit, block, mbits);
  if (orc_sparse_bytes(unit, dt) > maxmsg) maxmsg = orc_sparse_bytes(unit, dt);
  uint8_t* msg = (uint8_t*)malloc(maxmsg);
  size_t nbu = unit / (size_t)block;
  double* bm = (double*)malloc(sizeof(double) * nbu);
  if (blockmax_out) {
    size_t nbt = (count + (size_t)block - 1) / (size_t)block;
    for (size_t b = 0; b < nbt; ++b) blockmax_out[b] = 0.0;
  }
  /* reduce-scatter pass */
  for (int s = 1; s <= n - 1; ++s) {
    for (int r = 0; r < n; ++r) {
      int src = modn(r - 1, n);
      int c = modn(r - s - 1, n);
      size_t lo, hi;
      chunk_range(count, L, c, &lo, &hi);
      for (size_t u = lo; u < hi; u += unit) {
        size_t len = hi - u < unit ? hi - u : unit;
        size_t bytes = comp_encode(&cf, (const char*)bufs[src] + u * es, len, msg, bm);
        note_blockmax(blockmax_out, bm, u / (size_t)block, (len + (size_t)block - 1) / (size_t)block);
        add_traffic(sent, recv, src, r, (uint64_t)bytes);
        comp_decode(&cf, msg, len, (char*)bufs[r] + u * es, 1);
      }
    }
  }
  /* allgather pass */
  for (int c = 0; c < n; ++c) {
    size_t lo, hi;
    chunk_range(count, L, c, &lo, &hi);
    for (size_t u = lo; u < hi; u += unit) {
      size_t len = hi - u < unit ? hi - u : unit;
      size_t bytes = comp_encode(&cf, (const char*)bufs[c] + u * es, len, msg, bm);
      note_blockmax(blockmax_out, bm, u / (size_t)block, (len + (size_t)block - 1) / (size_t)block);
      for (int s = 1; s <= n - 1; ++s) add_traffic(sent, recv, modn(c + s - 1, n), modn(c + s, n), (uint64_t)bytes);
      for (int r = 0; r < n; ++r) comp_decode(&cf, msg, len, (char*)bufs[r] + u * es, 0);
    }
  }
  free(bm);
  free(msg);
  return ORC_OK;
}

/* ------------------------------------------------------------------ */
/* Stateful BFP ring ([P4] section 2.1 differential encoding, section 3.3 */
/* 'diff' compression type, section 5 error feedback).  In the           */
/* compressed ring every rank encodes each of its elements exactly once  */
/* per allreduce (the N-1 chunks it sends in the reduce-scatter, its own */
/* chunk in the allgather), so one binary32 state value per rank and     */
/* element is well defined:                                              */
/*   error feedback:  v = p + e;  send E(v);  e <- v - D(E(v))           */
/*   delta:           v = p - ref; send E(v); p^ = ref + D(E(v));         */
/*                    ref <- p^ (both ends track the reconstruction)     */
/* where p is the sender's current value (its partial in the reduce-     */
/* scatter, the finished sum in the allgather) and the receiver uses     */
/* D(E(v)) (error feedback) or p^ (delta) in place of the message value. */
/* ------------------------------------------------------------------ */

enum { ORC_FB_ERROR = 1, ORC_FB_DELTA = 2 };

/* Encode len elements of `src` (dtype dt) with the sender's state st[] and
 * return in `val` the binary32 value the receiver takes for each element. */
static void stateful_message(const void* src, int dt, float* st, size_t len, int block, int mbits, int feedback,
                             float* v, uint8_t* msg, float* val) {
  for (size_t i = 0; i < len; ++i) {
    float p = widen(src, i, dt);
    v[i] = feedback == ORC_FB_ERROR ? p + st[i] : p - st[i];
  }
  orc_bfp_encode(v, ORC_F32, len, block, mbits, msg, NULL);
  size_t nb = (len + (size_t)block - 1) / (size_t)block;
  size_t eb = (nb + 15) / 16 * 16;
  for (size_t i = 0; i < len; ++i) {
    float d = bfp_value(msg, eb, i, block, mbits);
    if (feedback == ORC_FB_ERROR) {
      st[i] = v[i] - d;
      val[i] = d;
    } else {
      float rec = st[i] + d;
      st[i] = rec;
      val[i] = rec;
    }
  }
}

/* state[r]: rank r's binary32 state, count elements (zero before the first
 * call).  unit must be a positive multiple of block. */
int orc_ring_allreduce_compressed_state(void* const* bufs, float* const* state, int n, size_t count, int dt,
                                        int block, int mbits, size_t unit, int feedback, uint64_t* sent,
                                        uint64_t* recv) {
  if (!check_bufs(bufs, n, dt) || !bfp_args_ok(block, mbits) || !state) return ORC_EINVAL;
  if (feedback != ORC_FB_ERROR && feedback != ORC_FB_DELTA) return ORC_EINVAL;
  if (unit == 0 || unit % (size_t)block) return ORC_EINVAL;
  if (n == 1) return ORC_OK; /* nothing travels: buffer and state stay as they are */
  size_t es = dtype_size(dt);
  size_t L = orc_comp_chunk_len(count, n, block);
  float* v = (float*)malloc(sizeof(float) * unit);
  float* val = (float*)malloc(sizeof(float) * unit);
  uint8_t* msg = (uint8_t*)malloc(orc_bfp_bytes(unit, block, mbits));
  for (int s = 1; s <= n - 1; ++s) {
    for (int r = 0; r < n; ++r) {
      int src = modn(r - 1, n), c = modn(r - s - 1, n);
      size_t lo, hi;
      chunk_range(count, L, c, &lo, &hi);
      for (size_t u = lo; u < hi; u += unit) {
        size_t len = hi - u < unit ? hi - u : unit;
        stateful_message((const char*)bufs[src] + u * es, dt, state[src] + u, len, block, mbits, feedback, v, msg,
                         val);
        add_traffic(sent, recv, src, r, (uint64_t)orc_bfp_bytes(len, block, mbits));
        for (size_t i = 0; i < len; ++i) accumulate(bufs[r], u + i, dt, val[i]);
      }
    }
  }
  for (int c = 0; c < n; ++c) {
    size_t lo, hi;
    chunk_range(count, L, c, &lo, &hi);
    for (size_t u = lo; u < hi; u += unit) {
      size_t len = hi - u < unit ? hi - u : unit;
      stateful_message((const char*)bufs[c] + u * es, dt, state[c] + u, len, block, mbits, feedback, v, msg, val);
      for (int s = 1; s <= n - 1; ++s)
        add_traffic(sent, recv, modn(c + s - 1, n), modn(c + s, n), (uint64_t)orc_bfp_bytes(len, block, mbits));
      for (int r = 0; r < n; ++r)
        for (size_t i = 0; i < len; ++i) narrow_store(bufs[r], u + i, dt, val[i]);
    }
  }
  free(msg);
  free(val);
  free(v);
  return ORC_OK;
}

/* ------------------------------------------------------------------ */
/* Gradient bucketing ([P2] production patterns: fuse small gradients   */
/* into buckets of about 25 MB, one allreduce per bucket).  Greedy in   */
/* tensor order; a tensor larger than the cap travels alone.            */
/* ------------------------------------------------------------------ */

/* bucket_of[t] receives the bucket index of tensor t; returns the number
 * of buckets. */
size_t orc_bucket_plan(const size_t* counts, size_t nt, int dt, size_t cap_bytes, int* bucket_of) {
  size_t es = dtype_size(dt);
  size_t nb = 0, cur = 0;
  int open = 0;
  for (size_t t = 0; t < nt; ++t) {
    size_t b = counts[t] * es;
    if (b > cap_bytes) {
      if (open) ++nb;
      bucket_of[t] = (int)nb;
      ++nb;
      open = 0;
      cur = 0;
      continue;
    }
    if (open && cur + b > cap_bytes) {
      ++nb;
      open = 0;
      cur = 0;
    }
    bucket_of[t] = (int)nb;
    cur += b;
    open = 1;
  }
  if (open) ++nb;
  return nb;
}

/* Offset of each tensor inside its bucket: tensors are laid end to end, each
 * starting on a 16-byte boundary; the gap after a tensor is zero. */
static size_t padded_elems(size_t count, size_t es) { return (count * es + 15) / 16 * 16 / es; }

/* tensors[r * nt + t] is rank r's tensor t.  Each bucket is packed into a
 * flat buffer per rank (16-byte aligned tensor offsets, zero gaps),
 * ring-allreduced, and unpacked. */
int orc_bucketed_allreduce(void* const* tensors, const size_t* counts, size_t nt, int n, int dt,
                           size_t cap_bytes, uint64_t* sent, uint64_t* recv) {
  if (n < 1 || n > ORC_MAXN || !dtype_ok(dt)) return ORC_EINVAL;
  size_t es = dtype_size(dt);
  int* bof = (int*)malloc(sizeof(int) * (nt ? nt : 1));
  size_t nb = orc_bucket_plan(counts, nt, dt, cap_bytes, bof);
  size_t t0 = 0;
  void* flat[ORC_MAXN];
  for (size_t b = 0; b < nb; ++b) {
    size_t t1 = t0, total = 0;
    while (t1 < nt && bof[t1] == (int)b) total += padded_elems(counts[t1++], es);
    for (int r = 0; r < n; ++r) {
      flat[r] = calloc(total * es + 1, 1);
      size_t off = 0;
      for (size_t t = t0; t < t1; ++t) {
        memcpy((char*)flat[r] + off * es, tensors[(size_t)r * nt + t], counts[t] * es);
        off += padded_elems(counts[t], es);
      }
    }
    orc_ring_allreduce(flat, n, total, dt, sent, recv);
    for (int r = 0; r < n; ++r) {
      size_t off = 0;
      for (size_t t = t0; t < t1; ++t) {
        memcpy(tensors[(size_t)r * nt + t], (char*)flat[r] + off * es, counts[t] * es);
        off += padded_elems(counts[t], es);
      }
      free(flat[r]);
    }
    t0 = t1;
  }
  free(bof);
  return ORC_OK;
}

/* Reports whether the x86 flush-to-zero or denormals-are-zero modes are on
 * (they would break the binary32 reference arithmetic). */
int orc_fpenv_ok(void) {
#if defined(__x86_64__)
  unsigned csr = __builtin_ia32_stmxcsr();
  return (csr & 0x8040u) == 0;
#else
  return 1;
#endif
}

/* ------------------------------------------------------------------ */
/* Shared-state hash and fault injection on the simulated ring.         */
/* [P1] "Prime Intellect 发布 PCCL 分布式训练通信库", section "PCCL 模型"   */
/* (the PCCL model): peers keep a shared state that is checked by hash  */
/* and re-sent to a peer whose hash differs from the majority; a        */
/* collective interrupted by a failing peer is retried on the remaining */
/* peers.                                                               */
/* ------------------------------------------------------------------ */

/* Output function of the splitmix64 generator (Steele, Lea and Flood,
 * "Fast splittable pseudorandom number generators", OOPSLA 2014; the
 * constants of Vigna's public-domain splitmix64). */
static uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

#define ORC_GOLDEN 0x9E3779B97F4A7C15ull

uint64_t orc_mix64(uint64_t z) { return mix64(z); }

/* 64-bit hash of nbytes bytes (a reading: the pages name a hash of the
 * shared state, not which one).  The bytes are read as little-endian 64-bit
 * words w_0 .. w_{W-1}, the last one zero-padded;
 *   h = sum over i of mix64(w_i + (i+1) * GOLDEN)   (mod 2^64)
 *   H = mix64(h xor nbytes). */
uint64_t orc_hash64(const void* buf, size_t nbytes) {
  const uint8_t* b = (const uint8_t*)buf;
  uint64_t h = 0;
  size_t words = (nbytes + 7) / 8;
  for (size_t i = 0; i < words; ++i) {
    uint64_t w = 0;
    for (int k = 0; k < 8; ++k) {
      size_t j = i * 8 + (size_t)k;
      if (j < nbytes) w |= (uint64_t)b[j] << (8 * k);
    }
    h += mix64(w + (uint64_t)(i + 1) * ORC_GOLDEN);
  }
  return mix64(h ^ (uint64_t)nbytes);
}

/* Shared-state check: hash every rank's buffer; the majority hash is the one
 * held by the most ranks (a tie goes to the hash of the lowest rank among
 * the tied ones); the lowest rank holding it sends its buffer to every rank
 * whose hash differs.  Returns the number of ranks re-sent, -1 on bad args. */
int orc_shared_state_sync(void* const* bufs, int n, size_t nbytes, uint64_t* hashes, uint64_t* sent,
                          uint64_t* recv) {
  if (n < 1 || n > ORC_MAXN || !bufs) return -1;
  uint64_t h[ORC_MAXN];
  for (int r = 0; r < n; ++r) {
    h[r] = orc_hash64(bufs[r], nbytes);
    if (hashes) hashes[r] = h[r];
  }
  int src = 0, best = 0;
  for (int r = 0; r < n; ++r) {
    int votes = 0;
    for (int q = 0; q < n; ++q) votes += h[q] == h[r];
    if (votes > best) {
      best = votes;
      src = r;
    }
  }
  int resent = 0;
  for (int r = 0; r < n; ++r) {
    if (h[r] == h[src]) continue;
    memcpy(bufs[r], bufs[src], nbytes);
    add_traffic(sent, recv, src, r, (uint64_t)nbytes);
    ++resent;
  }
  return resent;
}

enum { ORC_EABORT = 2 };

/* Ring allreduce with injected faults.  Fault i says: rank fault_rank[i]
 * fails before step fault_step[i] (steps counted 1 .. 2(M-1) within one
 * pass over M members: reduce-scatter steps first, then allgather steps).
 * fault_stall[i] = 0: the rank is gone, and the check before the step finds
 * it at once.  fault_stall[i] = s > 0: the rank stops answering for s ms;
 * with a receive deadline D > 0 ([P2] exercise: a stuck rank raises a
 * deadline error instead of hanging) it is declared failed after D ms when
 * s > D, and the step goes ahead after s ms when s <= D; with D <= 0 every
 * stall is waited out.  The members are checked together before a step, so
 * the wait before a step is the largest wait any of its faults causes.
 * A fault fires the first time a pass reaches its step while its rank is
 * still a member.  A pass that meets a failed member is abandoned: every
 * rank's buffer is restored from the snapshot taken on entry, the failed
 * ranks leave the ring, and a new pass starts over the survivors (ascending
 * rank order, the ring closing over the gaps, chunk length from the survivor
 * count).  Bytes of abandoned steps count in the traffic.  Out: attempts =
 * passes started; dead_attempt[r] / dead_step[r] = pass and step at which
 * rank r was found failed (0 = never); dead_reason[r] = 0 alive, 1 gone,
 * 2 deadline; *waited_ms = total wait.  Returns ORC_OK when a pass
 * completed, ORC_EABORT when no rank is left (buffers restored). */
int orc_ring_allreduce_ft(void* const* bufs, int n, size_t count, int dt, const int* fault_rank,
                          const int* fault_step, const int* fault_stall, int nfaults, int deadline_ms, int* attempts,
                          int* dead_attempt, int* dead_step, int* dead_reason, long long* waited_ms, uint64_t* sent,
                          uint64_t* recv) {
  if (!check_bufs(bufs, n, dt) || nfaults < 0 || nfaults > 256 ||
      (nfaults && (!fault_rank || !fault_step || !fault_stall)))
    return ORC_EINVAL;
  for (int i = 0; i < nfaults; ++i)
    if (fault_rank[i] < 0 || fault_rank[i] >= n || fault_step[i] < 1 || fault_stall[i] < 0) return ORC_EINVAL;
  size_t bytes = count * dtype_size(dt);
  void* snap[ORC_MAXN];
  for (int r = 0; r < n; ++r) {
    snap[r] = malloc(bytes + 1);
    memcpy(snap[r], bufs[r], bytes);
  }
  int alive[ORC_MAXN], fired[256];
  for (int r = 0; r < n; ++r) {
    alive[r] = 1;
    dead_attempt[r] = dead_step[r] = dead_reason[r] = 0;
  }
  for (int i = 0; i < nfaults; ++i) fired[i] = 0;
  long long waited = 0;
  int attempt = 0, rc = ORC_OK;
  for (;;) {
    ++attempt;
    int members[ORC_MAXN], m = 0;
    void* sub[ORC_MAXN];
    for (int r = 0; r < n; ++r)
      if (alive[r]) {
        members[m] = r;
        sub[m++] = bufs[r];
      }
    if (m == 0) { /* no pass can start */
      --attempt;
      rc = ORC_EABORT;
      break;
    }
    size_t L = orc_chunk_len(count, m, 128);
    int aborted = 0;
    for (int g = 1; g <= 2 * (m - 1) && !aborted; ++g) {
      long long wait = 0;
      for (int i = 0; i < nfaults; ++i) {
        if (fired[i] || fault_step[i] != g) continue;
        fired[i] = 1;
        int k = fault_rank[i];
        if (!alive[k]) continue;
        int s = fault_stall[i];
        if (s > 0 && (deadline_ms <= 0 || s <= deadline_ms)) { /* answers again in time */
          if (s > wait) wait = s;
          continue;
        }
        if (s > 0 && deadline_ms > wait) wait = deadline_ms;
        alive[k] = 0;
        dead_attempt[k] = attempt;
        dead_step[k] = g;
        dead_reason[k] = s > 0 ? 2 : 1;
        aborted = 1;
      }
      waited += wait;
      if (aborted) break;
      uint64_t ps[ORC_MAXN] = {0}, pr[ORC_MAXN] = {0};
      if (g <= m - 1) rs_step_L(sub, m, count, dt, g, L, ps, pr);
      else ag_step_L(sub, m, count, dt, g - (m - 1), L, ps, pr);
      for (int j = 0; j < m; ++j) {
        if (sent) sent[members[j]] += ps[j];
        if (recv) recv[members[j]] += pr[j];
      }
    }
    if (!aborted) break;
    for (int r = 0; r < n; ++r) memcpy(bufs[r], snap[r], bytes);
  }
  if (rc == ORC_EABORT)
    for (int r = 0; r < n; ++r) memcpy(bufs[r], snap[r], bytes);
  *attempts = attempt;
  *waited_ms = waited;
  for (int r = 0; r < n; ++r) free(snap[r]);
  return rc;
}
