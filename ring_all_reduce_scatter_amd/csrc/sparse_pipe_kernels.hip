// Sparsity-aware compressed ring, pipelined in one cooperative launch
// (page "CCCL通信压缩库：突破LLM训练通信墙的工程实践", section 2.1: a message goes
// as non-zero values plus indices when its zeros exceed a threshold share,
// else as block floating point; section 2.2: compression, transfer and the
// receiver's decompress + reduce overlap chunk by chunk).
//
// The choice between the two formats is made per message unit, so every
// tile of a unit has to know the unit's non-zero total before it writes its
// part of the message, and a sparse unit's tiles need the non-zeros of the
// tiles before them to place their values and indices.  A gang of
// workgroups therefore carries one unit through all N hops, holding each
// tile's partial sum in LDS:
//   hop h: (h > 1) load the tile's part of message h-1 back from its slot,
//          decode it, add the receiver's own copy (rank c+h);
//          count the tile's non-zeros, publish the count, learn the unit's
//          decision; write the tile's part of message h.
//   then every rank stores the owner's message (h = N) decoded.
// Publishing: the tile stores count + 1 in a per-tile word and adds
// (1 << 32 | its count) to a per-(hop, unit) word; the value the add
// returns tells it the running sum.  Zeros only shrink as counts arrive,
// so once that sum rules "sparse" out the unit is BFP: the tile whose add
// crossed the threshold publishes that in a per-(hop, unit) decision word,
// and every later tile knows it from its own add.  If the last tile to
// arrive finds the threshold never crossed, the unit is sparse with that
// exact total, and it publishes so.  Only tiles that arrive before either
// event read the decision word, which is written once.  A sparse unit's
// tiles read the per-tile words before theirs for their offsets.
// Every wait is bounded: past kSpinLimit polls the tile raises the abort
// word and goes on, so no wave can wait forever.  The launch is cooperative:
// every workgroup of the grid is resident at once and a gang's members wait
// only for each other, so the waits end.
//
// Message layout (16-byte header {nnz, kind, len, 0} first): kind 0 = the
// unit's BFP layout; kind 1 = values in the element type, zero padding to 16
// bytes, uint32 indices ascending and unit-relative, this body starting
// after the slot's BFP area (16 + the BFP bytes rounded up to 16).  The sparse values are
// placed in tile order, lane order inside a tile and group order inside a
// lane's span, which is ascending index order.
#include "bfp_device.hpp"
#include "block_scan.hpp"
#include "h16_codec.hpp"
#include "launch.hpp"

namespace rar {

namespace {

// Polls of one wait before giving up (well under a second); every 256th
// poll also reads the abort word, so once one wait has given up the others
// end within a few microseconds.
constexpr uint32_t kSpinLimit = 1u << 19;

__device__ __forceinline__ uint64_t ld_agent64(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ld_agent32(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_agent32(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_agent64(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void wave_stores_done() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): this wavefront's stores acknowledged
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

__device__ __forceinline__ uint64_t round16(uint64_t x) { return (x + 15) / 16 * 16; }

template <int DT>
__device__ __forceinline__ uint32_t nonzeros(const G8& x, int nv) {
  uint32_t c = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) c += (i < nv && x.v[i] != 0.0f) ? 1u : 0u;
  return c;
}

// Bit i set: element i of the group is one of its nv valid elements and not +-0.
template <int DT>
__device__ __forceinline__ uint32_t nz_mask(const G8& x, int nv) {
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) m |= (i < nv && x.v[i] != 0.0f) ? 1u << i : 0u;
  return m;
}

template <int DT>
__device__ __forceinline__ uint32_t raw_bits(float v) {
  if constexpr (DT == DT_F32) return __float_as_uint(v);
  else return narrow16<DT>(v);
}
template <int DT>
__device__ __forceinline__ float from_raw(uint32_t r) {
  if constexpr (DT == DT_F32) return __uint_as_float(r);
  else return widen16<DT>(r);
}

// Element i of a group held in LDS, as stored (run-time i: LDS addressing,
// not register indexing).
template <int DT>
__device__ __forceinline__ uint32_t lds_elem(const Raw8<DT>* g, int i) {
  if constexpr (DT == DT_F32) return ((const uint32_t*)g)[i];
  else return ((const uint16_t*)g)[i];
}
template <int DT>
__device__ __forceinline__ void lds_set(Raw8<DT>* g, int i, uint32_t raw) {
  if constexpr (DT == DT_F32) ((uint32_t*)g)[i] = raw;
  else ((uint16_t*)g)[i] = (uint16_t)raw;
}

struct SpPipeArgs {
  RankPtrs bufs;
  uint8_t* slots;      // message slots [hop 1..N][chunk][unit]
  uint64_t* unitw;     // [hop][chunk][unit]: arrived tiles << 32 | non-zeros so far (zero at launch)
  uint64_t* decw;      // [hop][chunk][unit]: 0 undecided, 1 BFP, total << 8 | 2 sparse (zero at launch)
  uint32_t* tilecnt;   // [hop][chunk][unit][tile]: non-zeros + 1, 0 = not yet (zero at launch)
  uint64_t* traffic;   // u64 sent[64], recv[64] (zero at launch)
  uint32_t* abort;     // nonzero if a wait gave up
  uint64_t count, L, U, upc, slot;
  uint32_t kmax;       // tiles of a full unit
  uint32_t gangs;      // units in flight (grid = gangs * kmax)
  int nranks, lpb, mbits;
  float theta;
};

// Dynamic LDS of one workgroup: the tile's partial sums as stored (group g of
// lane l at [g * 256 + l], i.e. the tile's elements in order).
template <int DT, int GP>
constexpr size_t sp_lds_bytes() {
  return (size_t)GP * kThreads * sizeof(Raw8<DT>);
}

template <int DT, int LPB, int GP>
__global__ __launch_bounds__(kThreads) void sparse_pipe_kernel(SpPipeArgs a) {
  constexpr uint32_t ES = DtypeSize<DT>::value;
  constexpr uint64_t kTile = (uint64_t)kThreads * kGroupElems * GP;
  extern __shared__ __align__(16) unsigned char sp_lds[];
  Raw8<DT>* P = (Raw8<DT>*)sp_lds;
  const int N = a.nranks;
  const int lpb = LPB > 0 ? LPB : a.lpb;
  const int mbits = a.mbits;
  const uint64_t block = (uint64_t)lpb * 8;
  const float qmax = (float)((1 << (mbits - 1)) - 1);
  // binary16 with 128-element blocks: the packed codec (h16_codec.hpp)
  constexpr bool kH16 = DT == DT_F16 && LPB == 16;
  const uint32_t gang = blockIdx.x / a.kmax, k = blockIdx.x - gang * a.kmax;
  const uint32_t nunits = (uint32_t)N * (uint32_t)a.upc;  // units of one hop (< 2^32: at most 64 ranks)
  const uint64_t hstride = nunits * a.slot;  // message h+1 of a unit sits hstride bytes after message h
  __shared__ uint32_t s_dec[2];              // the unit's decision for this hop: kind, non-zero total

  // rank c + d for 0 <= d <= N (no division)
  auto ring = [N](uint32_t c, int d) -> int { const int r = (int)c + d; return r >= N ? r - N : r; };
  for (uint32_t uid = gang; uid < nunits; uid += a.gangs) {
    // uniform over the workgroup: the unit and whether this tile exists
    const uint32_t c = uid / (uint32_t)a.upc;
    const uint64_t u = uid - c * (uint32_t)a.upc;
    const uint64_t lo = (uint64_t)c * a.L;
    if (lo >= a.count) continue;
    const uint64_t hi = lo + a.L < a.count ? lo + a.L : a.count;
    const uint64_t ulo = lo + u * a.U;
    if (ulo >= hi) continue;
    const uint64_t ulen = hi - ulo < a.U ? hi - ulo : a.U;
    const uint32_t Ku = (uint32_t)((ulen + kTile - 1) / kTile);
    if (k >= Ku) continue;

    // group g of this lane: unit-relative elements off(g) .. off(g) + nv(g)
    const uint64_t off0 = (uint64_t)k * kTile + (uint64_t)threadIdx.x * kGroupElems;
    auto off = [&](int g) -> uint64_t { return off0 + (uint64_t)g * kThreads * kGroupElems; };
    auto nvof = [&](int g) -> int {
      const uint64_t o = off(g);
      return o >= ulen ? 0 : (ulen - o >= 8 ? 8 : (int)(ulen - o));
    };
    const bool full = (uint64_t)(k + 1) * kTile <= ulen;  // every group of every lane holds 8 elements
    const uint64_t nb = (ulen + block - 1) / block, eb = round16(nb);
    // a sparse message's body (values, padding, indices) follows the BFP
    // area of the slot: a tile may write its BFP part before it learns that
    // the unit goes sparse (see below), and the two must not overlap
    const uint64_t spoff = 16 + round16(bfp_msg_bytes(ulen, (int)block, mbits));
    uint8_t* msg1 = a.slots + (uint64_t)uid * a.slot;
    auto load = [&](int rank, int g) -> Raw8<DT> {
      if (full) return load_raw8<DT, true>(a.bufs.p[rank], ulo + off(g));
      return pack8<DT>(load_part8<DT>(a.bufs.p[rank], ulo + off(g), nvof(g)));
    };
    auto slot = [&](int g) -> int { return g * kThreads + (int)threadIdx.x; };

    // the last message's format and totals: unit, this tile, this tile's first entry
    bool sp_prev = false;
    uint32_t tot_prev = 0, tile_first = 0, tile_cnt = 0;

    // The lane's group g of BFP message m, decoded: acc = true adds it to xr
    // (local + received, as the receiver of a reduce-scatter hop), acc =
    // false gives the value itself (allgather).
    auto decode_own = [&](const uint8_t* m, int g, const Raw8<DT>& xr, bool acc) -> Raw8<DT> {
      const int nv = nvof(g);
      if constexpr (kH16) {
        // exponent byte and mantissas of the lane's group, decoded packed
        const uint8_t* pay = m + 16;
        u32x2 w = {0u, 0u};
        uint32_t E = 0;
        if (nv > 0) {
          const uint64_t o = off(g);
          E = pay[o / 128];
          const uint8_t* mp = pay + eb + (mbits > 4 ? o : o / 2);
          if (nv == 8) {
            if (mbits > 4) w = *(const u32x2*)mp;
            else w[0] = *(const uint32_t*)mp;
          } else if (mbits > 4) {
            for (int i = 0; i < nv; ++i) w[i >> 2] |= (uint32_t)mp[i] << (8 * (i & 3));
          } else {
            for (int i = 0; i < (nv + 1) / 2; ++i) w[0] |= (uint32_t)mp[i] << (8 * i);
          }
        }
        const u32x4 d = dec_h16x8(E, w, mbits);
        Raw8<DT> r;
#pragma unroll
        for (int i = 0; i < 4; ++i) r.w[0][i] = acc ? h2_bits(as_h2(xr.w[0][i]) + as_h2(d[i])) : d[i];
        r.w[0] = keep_h16x8(r.w[0], nv);
        return r;
      }
      const G8 d = nv > 0 ? dequant_group(m + 16, eb, off(g), nv, block, mbits) : G8{};
      const G8 x = unpack8<DT>(xr);
      G8 r;
#pragma unroll
      for (int t = 0; t < 8; ++t) r.v[t] = t < nv ? round_to<DT>(acc ? x.v[t] + d.v[t] : d.v[t]) : 0.0f;
      return pack8<DT>(r);
    };

    // This tile's entries of sparse message m, added to (acc) or stored into
    // the partials in LDS, which hold the tile's elements in order (group g
    // of lane l is elements (g * 256 + l) * 8 ..).  The entries are one
    // contiguous run of the message, so the workgroup loads them coalesced,
    // four per lane at a time; their indices are distinct, so no two lanes
    // touch one element.  Every lane calls this between two barriers.
    auto scatter_sparse = [&](const uint8_t* m, bool acc) {
      const uint8_t* vals = m + spoff;
      const uint32_t* idx = (const uint32_t*)(m + spoff + round16((uint64_t)tot_prev * ES));
      const uint32_t base = k * (uint32_t)kTile;  // unit-relative first element of the tile
      for (uint32_t j0 = threadIdx.x; j0 < tile_cnt; j0 += 4 * kThreads) {
        uint32_t raw[4], e[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const uint32_t j = j0 + (uint32_t)t * kThreads;
          const uint32_t q = tile_first + (j < tile_cnt ? j : 0u);
          raw[t] = ES == 4 ? ((const uint32_t*)vals)[q] : (uint32_t)((const uint16_t*)vals)[q];
          e[t] = j < tile_cnt ? idx[q] - base : (uint32_t)kTile;
        }
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          if (e[t] >= (uint32_t)kTile) continue;
          Raw8<DT>* grp = &P[e[t] >> 3];
          const int i = (int)(e[t] & 7u);
          lds_set<DT>(grp, i, acc ? raw_bits<DT>(round_to<DT>(from_raw<DT>(lds_elem<DT>(grp, i)) + from_raw<DT>(raw[t])))
                                  : raw[t]);
        }
      }
    };

    uint32_t lane_nnz = 0;
#pragma unroll 4
    for (int g = 0; g < GP; ++g) {
      const Raw8<DT> x = load(ring(c, 1), g);
      P[slot(g)] = x;
      if constexpr (kH16) lane_nnz += nonzeros_h16x8(x.w[0]);
      else lane_nnz += nonzeros<DT>(unpack8<DT>(x), nvof(g));
    }
    for (int h = 1; h <= N; ++h) {
      uint8_t* msg = msg1 + (uint64_t)(h - 1) * hstride;
      if (h > 1) {
        // receiver of message h-1 (rank c+h): its own copy plus the decoded message
        wave_stores_done();
        lane_nnz = 0;
        const int r = ring(c, h);
        if (sp_prev) {
          // the receiver's copy, then the entries (see the allgather below)
#pragma unroll 4
          for (int g = 0; g < GP; ++g) P[slot(g)] = load(r, g);
          __syncthreads();
          scatter_sparse(msg - hstride, true);
          __syncthreads();
#pragma unroll 4
          for (int g = 0; g < GP; ++g) {
            if constexpr (kH16) lane_nnz += nonzeros_h16x8(P[slot(g)].w[0]);
            else lane_nnz += nonzeros<DT>(unpack8<DT>(P[slot(g)]), nvof(g));
          }
        } else {
#pragma unroll 2
          for (int g = 0; g < GP; ++g) {
            const Raw8<DT> p = decode_own(msg - hstride, g, load(r, g), true);
            P[slot(g)] = p;
            if constexpr (kH16) lane_nnz += nonzeros_h16x8(p.w[0]);
            else lane_nnz += nonzeros<DT>(unpack8<DT>(p), nvof(g));
          }
        }
      }
      uint32_t tile_nnz, unused;
      block_sum2(lane_nnz, 0u, &tile_nnz, &unused);
      const uint64_t fi = (uint64_t)(h - 1) * nunits + uid;
      auto write_bfp = [&]() {
        uint8_t* payload = msg + 16;
        if (k == 0 && threadIdx.x < eb - nb) payload[nb + threadIdx.x] = 0;  // exponent padding
#pragma unroll 2
        for (int g = 0; g < GP; ++g) {
          if constexpr (kH16) {
            const H16Code q = enc_h16x8(P[slot(g)].w[0], mbits);
            const int nv = nvof(g);
            if (nv == 0) continue;
            const uint64_t o = off(g);
            if ((threadIdx.x & 15u) == 0) payload[o / 128] = (uint8_t)q.E;
            uint8_t* mp = payload + eb + (mbits > 4 ? o : o / 2);
            if (nv == 8) {
              if (mbits > 4) *(u32x2*)mp = q.bytes;
              else *(uint32_t*)mp = q.bytes[0];
            } else if (mbits > 4) {
              for (int i = 0; i < nv; ++i) mp[i] = (uint8_t)(q.bytes[i >> 2] >> (8 * (i & 3)));
            } else {
              for (int i = 0; i < (nv + 1) / 2; ++i) mp[i] = (uint8_t)(q.bytes[0] >> (8 * i));
            }
          } else {
            encode_group<DT, LPB>(unpack8<DT>(P[slot(g)]), nvof(g), off(g), payload, payload + eb, lpb, mbits, qmax);
          }
        }
      };
      auto write_sparse = [&](uint32_t total) {
        // non-zeros of the unit's tiles before this one
        uint32_t before_part = 0;
        for (uint32_t j = threadIdx.x; j < k; j += kThreads) {
          uint32_t v = 0;
          for (uint32_t it = 0; (v = ld_agent32(&a.tilecnt[fi * a.kmax + j])) == 0u; ++it) {
            if (it >= kSpinLimit || ((it & 255u) == 255u && ld_agent32(a.abort) != 0u)) {
              __hip_atomic_store(a.abort, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
              v = 1;
              break;
            }
            __builtin_amdgcn_s_sleep(2);
          }
          before_part += v - 1;
        }
        uint32_t before;
        block_sum2(before_part, 0u, &before, &unused);
        uint8_t* vals = msg + spoff;
        uint32_t* idx = (uint32_t*)(msg + spoff + round16((uint64_t)total * ES));
        uint32_t rel = 0;  // entries of this tile written so far
        for (int g = 0; g < GP; ++g) {
          const G8 x = unpack8<DT>(P[slot(g)]);
          uint32_t m = nz_mask<DT>(x, nvof(g));
          uint32_t gtot;
          const uint32_t lpos = rel + block_exclusive_scan((uint32_t)__builtin_popcount(m), &gtot);
          uint32_t q = before + lpos;
          const uint32_t o = (uint32_t)off(g);
          for (; m; m &= m - 1, ++q) {  // ascending element order
            const int i = __builtin_ctz(m);
            const uint32_t raw = lds_elem<DT>(&P[slot(g)], i);
            if constexpr (ES == 4) ((uint32_t*)vals)[q] = raw;
            else ((uint16_t*)vals)[q] = (uint16_t)raw;
            idx[q] = o + (uint32_t)i;
          }
          rel += gtot;
        }
        tile_first = before;
        tile_cnt = rel;
        if (k == 0 && threadIdx.x < 16) {
          // zero padding between the values and the indices
          const uint64_t pad0 = spoff + (uint64_t)total * ES, pad1 = spoff + round16((uint64_t)total * ES);
          if (pad0 + threadIdx.x < pad1) msg[pad0 + threadIdx.x] = 0;
        }
      };
      // A tile whose own zeros would leave its unit BFP writes its BFP part
      // while its count's add is in flight and learns the unit's decision
      // afterwards: most messages are BFP, and the add's round trip then
      // overlaps the write.  If the unit goes sparse after all, the tile
      // writes its sparse part too (into the slot's sparse body, which the
      // BFP area does not overlap).  Other tiles learn the decision first.
      const uint64_t tlen = ulen - (uint64_t)k * kTile < kTile ? ulen - (uint64_t)k * kTile : kTile;
      const bool spec = (double)(tlen - tile_nnz) <= (double)a.theta * (double)tlen;  // uniform
      uint32_t kind = 0, total = 0;  // thread 0
      bool known = false;
      if (threadIdx.x == 0) {
        // zeros > theta * len fails for every running sum at or past lim_nnz
        const double lim = (double)a.theta * (double)ulen;
        st_agent32(&a.tilecnt[fi * a.kmax + k], tile_nnz + 1);
        const uint64_t old = __hip_atomic_fetch_add(&a.unitw[fi], (1ull << 32) | (uint64_t)tile_nnz,
                                                    __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const uint32_t arrived = (uint32_t)(old >> 32) + 1u, sum = (uint32_t)old + tile_nnz;
        if ((double)(ulen - sum) <= lim) {
          // BFP: zeros only shrink as counts arrive.  The add that crossed publishes it.
          if (!((double)(ulen - (uint32_t)old) <= lim)) st_agent64(&a.decw[fi], 1ull);
          known = true;
        } else if (arrived >= Ku) {
          // the last count, and the threshold never crossed: sparse, with the exact total
          kind = 1;
          total = sum;
          st_agent64(&a.decw[fi], ((uint64_t)sum << 8) | 2ull);
          known = true;
        }
      }
      if (spec) write_bfp();
      if (threadIdx.x == 0) {
        if (!known) {
          // wait for the tile that crosses the threshold or for the last one
          for (uint32_t it = 0;; ++it) {
            const uint64_t d = ld_agent64(&a.decw[fi]);
            if (d != 0) {
              kind = (d & 0xffu) == 2u ? 1u : 0u;
              total = (uint32_t)(d >> 8);
              break;
            }
            if (it >= kSpinLimit || ((it & 255u) == 255u && ld_agent32(a.abort) != 0u)) {
              __hip_atomic_store(a.abort, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
              break;
            }
            __builtin_amdgcn_s_sleep(2);
          }
        }
        s_dec[0] = kind;
        s_dec[1] = total;
      }
      __syncthreads();
      const bool sparse = s_dec[0] != 0;
      total = s_dec[1];
      if (k == 0 && threadIdx.x == 0) {
        uint32_t* hdr = (uint32_t*)msg;
        hdr[0] = sparse ? total : 0u;
        hdr[1] = sparse ? 1u : 0u;
        hdr[2] = (uint32_t)ulen;
        hdr[3] = 0u;
        const uint64_t bytes = sparse ? 16 + round16((uint64_t)total * ES) + 4ull * total
                                      : 16 + bfp_msg_bytes(ulen, (int)block, mbits);
        // message h < N goes from rank c+h to c+h+1; message N (the owner's)
        // is relayed around the ring, from c+s-1 to c+s for s = 1..N-1
        const int s0 = h < N ? h : 1, s1 = h < N ? h : N - 1;
        for (int s = s0; s <= s1; ++s) {
          const int from = h < N ? ring(c, s) : ring(c, s - 1);
          const int to = from + 1 == N ? 0 : from + 1;
          atomicAdd((unsigned long long*)&a.traffic[from], (unsigned long long)bytes);
          atomicAdd((unsigned long long*)&a.traffic[kMaxRanks + to], (unsigned long long)bytes);
        }
      }
      if (sparse) write_sparse(total);
      else if (!spec) write_bfp();
      sp_prev = sparse;
      tot_prev = total;
    }
    // allgather: every rank (owner included) stores the owner's message decoded
    wave_stores_done();
    const uint8_t* last = msg1 + (uint64_t)(N - 1) * hstride;
    if (sp_prev) {
      // zeros, then the entries (written by every wavefront of the workgroup:
      // the barrier orders their completed stores before these loads)
      Raw8<DT> z;
#pragma unroll
      for (int w = 0; w < (int)(sizeof(z) / 16); ++w) z.w[w] = (u32x4){0u, 0u, 0u, 0u};
#pragma unroll 4
      for (int g = 0; g < GP; ++g) P[slot(g)] = z;
      __syncthreads();
      scatter_sparse(last, false);
      __syncthreads();
    }
#pragma unroll 2
    for (int g = 0; g < GP; ++g) {
      const int nv = nvof(g);
      const Raw8<DT> yr = sp_prev ? P[slot(g)] : decode_own(last, g, Raw8<DT>{}, false);
      if (full) {
        // write-through stores over the tile's range in each rank
        const uint64_t t0 = ulo + (uint64_t)k * kTile;
        for (int d = 0; d < N; ++d)
          store_raw8_wt<DT>(wt_range(a.bufs.p[d] + t0 * ES, (uint32_t)(kTile * ES)), (uint32_t)((ulo + off(g) - t0) * ES), yr);
      } else if (nv > 0) {
        const G8 y = unpack8<DT>(yr);
        for (int d = 0; d < N; ++d) store_part8<DT>(a.bufs.p[d], ulo + off(g), nv, y);
      }
    }
    // the next unit's first hop reuses s_dec, P and the scans' LDS
    // only after barriers every lane passes after its last read of them
    __syncthreads();
  }
}

__global__ void zero_u64_kernel(uint64_t* p, uint64_t n) {
  for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (uint64_t)gridDim.x * blockDim.x)
    p[i] = 0;
}

// 8-element groups per lane: tiles of 16384 binary16 / bfloat16 elements
// or 8192 binary32 elements (32 KiB of partials in LDS; with the small
// static arrays four workgroups fit in a CU's 160 KiB, not five).
// Measured on MI355X (N = 8 x 64M fp16, 4 MiB units, ranks 0-3 95% zeros):
// 0.888 ms with the binary32 codec and each lane decoding its own sparse
// entries one dependent load at a time, 0.845 ms with the packed binary16
// codec (77 instead of 112 VGPRs), 0.786 ms with the workgroup decoding the
// sparse entries together, 0.764 ms with a dense tile writing its BFP part
// before it learns the unit's decision.  Per hop of a unit (timestamps of the first
// unit of each tile): decode 7-10 us, learning the decision 2.4-3.3 us
// (BFP) or 7-12 us (sparse: every count must be in), message write 3-7 us;
// the allgather 34 us.  Holding the next receiver's copy in
// registers during the message write needs 140-250 VGPRs (half the
// occupancy).  Loading the next receiver's copy straight into a second LDS
// buffer a hop ahead (global_load_lds) measured slower, 0.965 ms at 8192-
// element tiles and 1.21 ms at 16384: the extra buffer halves the units the
// chip holds at once, and the rounds of hops cost more than the latency it
// hides.  Unrolling the decode loop 4-fold instead of 2 changed nothing.
// Other measured variants: a decision word per tile (256 bytes apart, so no
// two waiting tiles read one word) 0.789 ms, no gain; two units per
// workgroup half a hop apart (8192-element tiles) 0.810 ms, because the
// count's atomic round trip still holds the workgroup before the other
// unit's work; the same with the tiles reading the arrival word for the
// decision instead of a decision word 1.39 ms (the reads queue with the
// adds on that word); 32768-element tiles (two workgroups per CU) 1.07 ms,
// 12288-element tiles (six per CU) 0.89 ms; a unit's BFP allgather spread
// over the workgroup's next unit, one group per hop between the count and
// the decision, 0.787 ms (no gain); counting one hop ahead (the next
// receiver's copy loaded into the partials while the message is written,
// its count taken with the message as it will decode, so the gang's counts
// gather during the receive) 0.851 ms: a sparse unit still waits for the
// gang's slowest count, which the short sparse receive does not cover, and
// the copy's loads no longer overlap the message's.  Hops split in two
// phases (count and publish; then decide and write), a workgroup carrying
// several units with their phases interleaved so that one unit's decision
// gathers while the workgroup works on another: with the partials
// recomputed in the second phase instead of held, 1.20 ms at two units and
// 1.08 ms at four (the second read comes from DRAM: 2.47 GB read per call
// against 1.36 GB); with each unit's partials held in its share of the
// LDS, 0.883 ms at two units (8192-element tiles) and 2.27 ms at four
// (4096): a unit's tiles multiply, and with them the counts, the adds and
// the look-back reads.  Loading the first two groups of the receiver's
// copy before the wait for the message stores: 0.771 against 0.760 ms
// (96 VGPRs; all eight groups: 215).  A tile whose own count is sparse
// writing its entries before the decision as well (indices at a fixed
// offset, so that only the header waits for the unit's total): 0.764-0.771
// against 0.764-0.768 ms.  Odd gangs starting 3, 6 or 12 us late, so that
// their decision waits would fall in the other gangs' decodes: 0.761-0.764,
// 0.761-0.764 and 0.768 ms against 0.758-0.760 (the gangs do not leave
// the memory idle together; each unit's chain of hops is the bound).
template <int DT>
struct SpGroups {
  static constexpr int value = DT == DT_F32 ? 4 : 8;
};

uint64_t sp_tile_elems(int dt) { return (uint64_t)kThreads * kGroupElems * (dt == DT_F32 ? 4 : 8); }

template <int DT, int LPB>
const void* sp_kernel() {
  return (const void*)sparse_pipe_kernel<DT, LPB, SpGroups<DT>::value>;
}

size_t sp_lds_for(int dt) {
  return dt == DT_F32 ? sp_lds_bytes<DT_F32, SpGroups<DT_F32>::value>() : sp_lds_bytes<DT_F16, SpGroups<DT_F16>::value>();
}

// The pipelined sparse ring is built for the pages' 128-element BFP block
// (16 lanes per block); other blocks run the staged schedule.
const void* sp_kernel_for(int dt) {
  switch (dt) {
    case DT_F32: return sp_kernel<DT_F32, 16>();
    case DT_F16: return sp_kernel<DT_F16, 16>();
    default: return sp_kernel<DT_BF16, 16>();
  }
}

// Units in flight: whole gangs of kmax workgroups that fit on the device at
// once (0 when one unit's tiles cannot all be resident).
hipError_t sp_gangs(const void* fn, size_t lds, uint64_t kmax, uint64_t nunits, uint64_t* gangs) {
  int dev = 0, cus = 0, per_cu = 0;
  hipError_t e;
  if ((e = hipGetDevice(&dev)) != hipSuccess) return e;
  if ((e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess) return e;
  if ((e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, kThreads, lds)) != hipSuccess) return e;
  const uint64_t capacity = (uint64_t)cus * (uint64_t)per_cu;
  uint64_t g = kmax ? capacity / kmax : 0;
  if (g > nunits) g = nunits;
  // as few gangs as give the same number of rounds of units (each round
  // runs its hops in lock step, so a last, partly filled round costs a full one)
  if (g > 0) {
    const uint64_t rounds = (nunits + g - 1) / g;
    g = (nunits + rounds - 1) / rounds;
  }
  *gangs = g;
  return hipSuccess;
}

}  // namespace

uint64_t sparse_pipe_tiles_per_unit(uint64_t unit_elems, int dt) {
  const uint64_t tile = sp_tile_elems(dt);
  return (unit_elems + tile - 1) / tile;
}

hipError_t launch_sparse_pipe(const RankPtrs& bufs, int n, uint64_t count, uint64_t L, uint64_t U, uint64_t upc,
                              uint64_t slot, uint8_t* slots, uint64_t* flags, uint64_t nflag_words,
                              uint64_t* traffic, int dt, int block, int mbits, float theta, hipStream_t stream) {
  if (L == 0 || count == 0) return hipSuccess;
  const uint64_t nunits = (uint64_t)n * upc;
  const uint64_t kmax = sparse_pipe_tiles_per_unit(U, dt);
  if (block != 128) return hipErrorInvalidValue;
  const void* fn = sp_kernel_for(dt);
  uint64_t gangs = 0;
  const size_t lds = sp_lds_for(dt);
  hipError_t e = sp_gangs(fn, lds, kmax, nunits, &gangs);
  if (e != hipSuccess) return e;
  if (gangs == 0) return hipErrorCooperativeLaunchTooLarge;  // checked before anything is enqueued
  // counters, arrival words, per-tile words and the abort word start at zero
  hipLaunchKernelGGL(zero_u64_kernel, dim3(64), dim3(256), 0, stream, traffic, (uint64_t)2 * kMaxRanks);
  hipLaunchKernelGGL(zero_u64_kernel, dim3(1024), dim3(256), 0, stream, flags, nflag_words);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  SpPipeArgs a;
  a.bufs = bufs;
  a.slots = slots;
  a.unitw = flags;
  a.decw = flags + (uint64_t)n * nunits;
  a.tilecnt = (uint32_t*)(flags + 2 * (uint64_t)n * nunits);
  a.abort = (uint32_t*)(flags + nflag_words - 1);
  a.traffic = traffic;
  a.count = count;
  a.L = L;
  a.U = U;
  a.upc = upc;
  a.slot = slot;
  a.kmax = (uint32_t)kmax;
  a.gangs = (uint32_t)gangs;
  a.nranks = n;
  a.lpb = block / 8;
  a.mbits = mbits;
  a.theta = theta;
  void* args[] = {&a};
  if ((e = hipLaunchCooperativeKernel(fn, dim3((unsigned)(gangs * kmax)), dim3(kThreads), args, (unsigned)lds,
                                      stream)) !=
      hipSuccess)
    return e;
  return launch_status(stream);
}

bool sparse_pipe_fits(int n, uint64_t upc, uint64_t U, int dt, int block) {
  uint64_t gangs = 0;
  return block == 128 && sp_gangs(sp_kernel_for(dt), sp_lds_for(dt), sparse_pipe_tiles_per_unit(U, dt), (uint64_t)n * upc,
                  &gangs) ==
             hipSuccess &&
         gangs > 0;
}

// Words of the flag area: per (hop, unit) one arrival word and one decision
// word, then per (hop, unit, tile) one 32-bit count (rounded up to whole
// words), then the abort word.
uint64_t sparse_pipe_flag_words(int n, uint64_t upc, uint64_t U, int dt) {
  const uint64_t nunits = (uint64_t)n * upc, kmax = sparse_pipe_tiles_per_unit(U, dt);
  return 2 * (uint64_t)n * nunits + ((uint64_t)n * nunits * kmax + 1) / 2 + 1;
}

}  // namespace rar
