// Device helpers shared by the gate/up kernels that work on 32-row halves
// of 64-row slabs: the expert block of one projection (from its directory
// record), column chunking, LDS staging with 16-byte global_load_lds, the
// SWAR plane decode and the transpose reduction.
//
// BitsMoE blog note, Methodology: "second split" (expert output = sum over
// components of magnitude * z_k * quantized unit direction) and "execution"
// (components of one width stored together, plane by plane).
#pragma once
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.h"
#include "format.h"

namespace bitsmoe {
namespace slab {

constexpr int kSlabRows = 32;  // rows of one half-slab

typedef __attribute__((address_space(3))) void lds_void;

// One projection's expert block, uniform across the work-group (SGPRs).
struct Proj {
  const uint8_t* blk;
  uint32_t mps, nq, n16, a_off, s_off, m_off, p_off, f_off;
  uint32_t c01, c23, c45;  // column counts of widths 1..8, two per word
  bool ok;
};

// First column and first mask of each 1..8-bit width group.
struct HGeo {
  uint32_t gcol[kNumQGroups + 1], gmask[kNumQGroups + 1];
};

__device__ __forceinline__ int hwidth(int g) { return g < 4 ? g + 1 : (g == 4 ? 6 : 8); }

__device__ __forceinline__ HGeo hgeo(const Proj& p) {
  const uint32_t c[kNumQGroups] = {p.c01 & 0xFFFFu, p.c01 >> 16, p.c23 & 0xFFFFu,
                                   p.c23 >> 16,     p.c45 & 0xFFFFu, p.c45 >> 16};
  HGeo G;
  G.gcol[0] = 0;
  G.gmask[0] = 0;
#pragma unroll
  for (int g = 0; g < kNumQGroups; ++g) {
    G.gcol[g + 1] = G.gcol[g] + c[g];
    G.gmask[g + 1] = G.gmask[g] + c[g] * (uint32_t)hwidth(g);
  }
  return G;
}

// Directory record of expert e (uniform) of one blob, read with scalar loads
// from e clamped into [0, E) (always inside the directory).
__device__ __forceinline__ DirRec load_rec_s(const uint8_t* blob, int e, int E) {
  typedef __attribute__((address_space(4))) const uint32_t CU32;
  const int ec = e < 0 ? 0 : (e >= E ? E - 1 : e);
  CU32* rp = (CU32*)(blob + kHeaderBytes + (size_t)ec * kDirRecBytes);
  union {
    uint32_t v[16];
    DirRec r;
  } u;
#pragma unroll
  for (int i = 0; i < 16; ++i) u.v[i] = rp[i];
  return u.r;
}

// The expert block described by record d, checked against header h.
__device__ __forceinline__ Proj make_proj(const uint8_t* blob, uint64_t bytes, int e,
                                          const DirRec& d, const HdrF& h, const GateUpArgs& a) {
  Proj p;
  p.ok = check_dir(h, d, bytes, e, a.E, a.dout, a.r);
  p.blk = blob + (p.ok ? d.block_offset : 0);
  p.mps = p.ok ? d.masks_per_slab : 0u;
  p.nq = p.ok ? d.n_q : 0u;
  p.n16 = p.ok ? d.n_16 : 0u;
  p.a_off = d.a_off;
  p.s_off = d.s_off;
  p.m_off = d.m_off;
  p.p_off = d.planes_off;
  p.f_off = d.f16_off;
  p.c01 = p.ok ? (uint32_t)d.count[0] | ((uint32_t)d.count[1] << 16) : 0u;
  p.c23 = p.ok ? (uint32_t)d.count[2] | ((uint32_t)d.count[3] << 16) : 0u;
  p.c45 = p.ok ? (uint32_t)d.count[4] | ((uint32_t)d.count[5] << 16) : 0u;
  return p;
}

// First mask of 1..8-bit column c (c = n_q gives masks_per_slab).
__device__ __forceinline__ uint32_t hmask_of(const HGeo& G, uint32_t c) {
  uint32_t m = G.gmask[kNumQGroups];
#pragma unroll
  for (int g = kNumQGroups - 1; g >= 0; --g)
    if (c < G.gcol[g + 1]) m = G.gmask[g] + (c - G.gcol[g]) * (uint32_t)hwidth(g);
  return m;
}

// Arena units (u64) of columns [0, c): masks, then 8 per fp16 column.
__device__ __forceinline__ uint32_t hpos(const Proj& p, const HGeo& G, uint32_t c) {
  return c <= p.nq ? hmask_of(G, c) : p.mps + 8u * (c - p.nq);
}

// End of the chunk that starts at column c0 (columns in blob order), for
// arenas of MaxM u64 (+2) and MaxC columns (+16).
template <int MaxM, int MaxC>
__device__ __forceinline__ uint32_t hchunk_end(const Proj& p, const HGeo& G, uint32_t c0) {
  const uint32_t n = p.nq + p.n16;
  uint32_t c1 = min(n, c0 + (uint32_t)MaxC - 16u);
  const uint32_t b0 = hpos(p, G, c0) & ~1u;
  while (c1 > c0 + 1 && hpos(p, G, c1) - b0 > (uint32_t)MaxM - 2u) c1 = c0 + (c1 - c0) / 2;
  return c1;
}

__device__ __forceinline__ void hstage16(void* dst, const void* src, uint32_t n, int lp,
                                         int lane, int nl) {
  const uint8_t* s = static_cast<const uint8_t*>(src);
  uint8_t* d = static_cast<uint8_t*>(dst);
  for (int i = lp; i < (int)n; i += nl)
    __builtin_amdgcn_global_load_lds(static_cast<const void*>(s + 16 * (size_t)i),
                                     (lds_void*)(d + 16 * (size_t)(i - lane)), 16, 0, 0);
}

__device__ __forceinline__ uint32_t hunits(uint32_t lo, uint32_t hi, uint32_t epu) {
  return hi > lo ? (hi - (lo & ~(epu - 1)) + epu - 1) / epu : 0u;
}

// LDS arenas of one projection.
struct Arena {
  uint64_t* M;   // plane masks, then the fp16 half-columns (8 u64 each)
  uint16_t* K;   // k indices
  float* A;      // magnitudes (coefficients once z is known)
  uint16_t* S;   // fp16 scales
  uint16_t* Mo;  // fp16 offsets
};

// Chunk [c0, c1) of projection p of slab `slab`, half `hh`, staged by nl
// lanes (lp = 0..nl-1): masks of the 1..8-bit columns from an even start,
// then the fp16 half-columns (64 bytes each) behind them.
__device__ __forceinline__ void hstage_chunk(const Arena& L, const Proj& p, uint32_t c0,
                                             uint32_t c1, int slab, int hh, uint32_t dout_pad,
                                             int lp, int lane, int nl) {
  const HGeo G = hgeo(p);
  const uint32_t q0 = min(c0, p.nq), q1 = min(c1, p.nq);
  const uint32_t base = (uint32_t)slab * p.mps;
  const uint32_t ma0 = (base + hmask_of(G, q0)) & ~1u;
  const uint32_t mu = q1 > q0 ? hunits(ma0, base + hmask_of(G, q1), 2) : 0u;
  hstage16(L.M, reinterpret_cast<const uint64_t*>(p.blk + p.p_off) + ma0, mu, lp, lane,
           nl);
  const uint16_t* kidx = reinterpret_cast<const uint16_t*>(p.blk);
  hstage16(L.K, kidx + (c0 & ~7u), hunits(c0, c1, 8), lp, lane, nl);
  hstage16(L.A, reinterpret_cast<const float*>(p.blk + p.a_off) + (c0 & ~3u),
           hunits(c0, c1, 4), lp, lane, nl);
  hstage16(L.S, reinterpret_cast<const uint16_t*>(p.blk + p.s_off) + (q0 & ~7u),
           hunits(q0, q1, 8), lp, lane, nl);
  hstage16(L.Mo, reinterpret_cast<const uint16_t*>(p.blk + p.m_off) + (q0 & ~7u),
           hunits(q0, q1, 8), lp, lane, nl);
  const uint32_t f0 = max(c0, p.nq) - p.nq, f1 = max(c1, p.nq) - p.nq;
  if (f1 > f0) {
    const uint8_t* fb = p.blk + p.f_off + ((size_t)slab * 64 + (size_t)hh * kSlabRows) * 2;
    uint8_t* dst = reinterpret_cast<uint8_t*>(L.M + 2 * mu);
    const int n = (int)(f1 - f0) * 4;
    for (int u = lp; u < n; u += nl) {
      const uint8_t* src = fb + (size_t)(f0 + (u >> 2)) * dout_pad * 2u + (u & 3) * 16;
      __builtin_amdgcn_global_load_lds(static_cast<const void*>(src),
                                       (lds_void*)(dst + 16 * (size_t)(u - lane)), 16, 0, 0);
    }
  }
}

__device__ __forceinline__ int hwave_bmax(int b) {
  if (__any(b > 6)) return 8;
  if (__any(b > 4)) return 6;
  if (__any(b > 3)) return 4;
  if (__any(b > 2)) return 3;
  if (__any(b > 1)) return 2;
  return __any(b > 0) ? 1 : 0;
}

// One 1..8-bit column of width b <= B over 32 rows: plane word j is the
// 32-bit half of mask j; bits are spread into byte codes, coef * code added.
template <int B>
__device__ __forceinline__ void column32(const uint32_t* words, int b, float coef,
                                         float (&acc)[kSlabRows]) {
  uint32_t w[B];
#pragma unroll
  for (int j = 0; j < B; ++j) w[j] = j < b ? words[2 * j] : 0u;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    uint32_t c = 0;
#pragma unroll
    for (int j = 0; j < B; ++j) {
      const uint32_t x = __builtin_amdgcn_ubfe(w[j], 4 * i, 4);
      c |= ((x * 0x00204081u) & 0x01010101u) << j;
    }
    acc[4 * i + 0] = fmaf(coef, (float)(c & 0xFFu), acc[4 * i + 0]);
    acc[4 * i + 1] = fmaf(coef, (float)((c >> 8) & 0xFFu), acc[4 * i + 1]);
    acc[4 * i + 2] = fmaf(coef, (float)((c >> 16) & 0xFFu), acc[4 * i + 2]);
    acc[4 * i + 3] = fmaf(coef, (float)(c >> 24), acc[4 * i + 3]);
  }
}

template <int O>
__device__ __forceinline__ void hstep(float (&v)[kSlabRows], bool up) {
#pragma unroll
  for (int i = 0; i < O; ++i) {
    const float send = up ? v[i] : v[i + O];
    const float keep = up ? v[i + O] : v[i];
    v[i] = keep + __shfl_xor(send, O, kWave);
  }
}

// Lanes l and l + 32 end with the sum over all 64 lanes of v[l & 31].
__device__ __forceinline__ float htranspose_sum(float (&v)[kSlabRows], int lane) {
  hstep<16>(v, (lane & 16) != 0);
  hstep<8>(v, (lane & 8) != 0);
  hstep<4>(v, (lane & 4) != 0);
  hstep<2>(v, (lane & 2) != 0);
  hstep<1>(v, (lane & 1) != 0);
  return v[0] + __shfl_xor(v[0], 32, kWave);
}


}  // namespace slab
}  // namespace bitsmoe
