// Device helpers shared by the MFMA gate/up kernels that work on 32-row
// segment records: one projection's expert block (from its directory record),
// block geometry, chunking, LDS staging with 16-byte global_load_lds, the
// plane decode that turns plane words into fp16 MFMA operands, and the
// v_mfma_f32_16x16x32_f16 step.
//
// BitsMoE blog note, Methodology: "second split" (an expert's output is the
// sum over components of magnitude * z_k * quantized unit direction) and
// "execution" (components of one width stored together, plane by plane).
//
// The apply is a contraction over slots (K): Y[row, n] = sum_slot code[row,
// slot] * coef[slot, n], with n the token columns.  Codes are the A operand
// (16 rows x 32 slots per instruction; lane l holds row l % 16 and slots
// 8 (l / 16) .. + 7, i.e. two 4-slot blocks), the fp16 coefficients the B
// operand (lane l holds token l % 16, the same 8 slots).  Coefficients are
// split into fp16 hi + lo parts of c * 2^S, so each K step is two MFMAs and
// the result carries ~22 bits of the coefficient; codes (<= 255) and fp16
// column values are exact in fp16 and every product is exact in fp32.
#pragma once
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.h"
#include "format.h"
#include "kernels.h"

namespace bitsmoe {
namespace seg {

typedef __attribute__((address_space(3))) void lds_void;
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));

constexpr int kBlkPerK = 8;  // 4-slot blocks per 32-slot K step
constexpr int kPW = 4;       // waves per projection sharing a segment's K steps

// Global-memory pointer types: loads through them are global (or buffer)
// loads counted only on the vector memory counter.  A pointer rebuilt from
// integers (as the uniform copies below are) would otherwise be a generic
// one, whose flat loads the compiler must also wait for before any LDS or
// scalar result is used.
typedef __attribute__((address_space(1))) const uint16_t gu16;
typedef __attribute__((address_space(1))) const uint32_t gu32;
typedef __attribute__((address_space(1))) const float gf32;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(1))) const u32x4 gv4;

// 16-byte global load (p 16-byte aligned).
template <typename T>
__device__ __forceinline__ uint4 ld16(const T* p) {
  const u32x4 v = *(const gv4*)p;
  return make_uint4(v.x, v.y, v.z, v.w);
}

// One projection's expert block, uniform across the work-group (SGPRs).
struct SegProj {
  const gu16* kidx;
  const gf32* A;
  const gu16* S;
  const gu16* M;
  const gu32* planes;  // segment 0's record
  uint32_t seg_words, n_slot, n_qslot, n_blk;
  uint32_t b1, b2, b3, b4, b5, b6;  // first block of groups 1..6 (widths 2,3,4,6,8,16)
  uint32_t w1, w2, w3, w4, w5, w6;  // first word of groups 1..6 inside a segment record
  float cmax;
  bool ok;
};

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

__device__ __forceinline__ SegProj make_seg(const uint8_t* blob, uint64_t bytes, int e,
                                            const DirRec& d, const HdrF& h, int E, int dout,
                                            int r) {
  SegProj p;
  p.ok = check_dir(h, d, bytes, e, E, dout, r);
  // A record that fails the check gives counts of 0 (no loop reads an
  // array) and a block at the blob base: kidx is then the blob base, and the
  // one reader that loads without looking at the counts (load_meta) takes
  // every array from there (the 128-byte header covers its loads at index
  // 0).  The other arrays' offsets are taken unchecked here, so that forming
  // them does not wait for the check.
  const uint64_t blk = reinterpret_cast<uint64_t>(blob) + (p.ok ? d.block_offset : 0);
  p.kidx = (const gu16*)blk;
  p.A = (const gf32*)(blk + d.a_off);
  p.S = (const gu16*)(blk + d.s_off);
  p.M = (const gu16*)(blk + d.m_off);
  p.planes = (const gu32*)(blk + d.planes_off);
  const SlotGeo geo = slot_geo(d.count);
  uint32_t nb[kNumGroups];
#pragma unroll
  for (int g = 0; g < kNumGroups; ++g) nb[g] = p.ok ? geo.nb[g] : 0u;
  uint32_t bs[kNumGroups + 1], ws[kNumGroups + 1];
  bs[0] = 0;
  ws[0] = 0;
#pragma unroll
  for (int g = 0; g < kNumGroups; ++g) {
    bs[g + 1] = bs[g] + nb[g];
    ws[g + 1] = ws[g] + 4u * nb[g] * (uint32_t)kGroupWidth[g];
  }
  p.b1 = bs[1]; p.b2 = bs[2]; p.b3 = bs[3]; p.b4 = bs[4]; p.b5 = bs[5]; p.b6 = bs[6];
  p.w1 = ws[1]; p.w2 = ws[2]; p.w3 = ws[3]; p.w4 = ws[4]; p.w5 = ws[5]; p.w6 = ws[6];
  p.n_blk = bs[kNumGroups];
  p.seg_words = ws[kNumGroups];
  p.n_slot = 4u * p.n_blk;
  p.n_qslot = 4u * bs[kNumQGroups];
  p.cmax = p.ok ? d.cmax : 0.f;
  return p;
}

__device__ __forceinline__ uint32_t rfl(uint32_t v) { return __builtin_amdgcn_readfirstlane(v); }

// Work-group barrier that orders LDS accesses only.  Unlike __syncthreads it
// does not make the wave wait for its outstanding global loads, including
// global_load_lds copies into LDS: a caller that needs those copies landed
// waits for them itself (s_waitcnt) before the barrier.
__device__ __forceinline__ void lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

template <typename T>
__device__ __forceinline__ T* rfl_ptr(T* p) {
  const uint64_t v = (uint64_t)p;
  return (T*)(((uint64_t)rfl((uint32_t)(v >> 32)) << 32) | rfl((uint32_t)v));
}

// The record is the same for every lane; this keeps it in scalar registers
// so that loops over blocks and K steps stay uniform branches.
__device__ __forceinline__ SegProj uniform_seg(const SegProj& p) {
  SegProj q;
  q.kidx = rfl_ptr(p.kidx);
  q.A = rfl_ptr(p.A);
  q.S = rfl_ptr(p.S);
  q.M = rfl_ptr(p.M);
  q.planes = rfl_ptr(p.planes);
  q.seg_words = rfl(p.seg_words);
  q.n_slot = rfl(p.n_slot);
  q.n_qslot = rfl(p.n_qslot);
  q.n_blk = rfl(p.n_blk);
  q.b1 = rfl(p.b1); q.b2 = rfl(p.b2); q.b3 = rfl(p.b3);
  q.b4 = rfl(p.b4); q.b5 = rfl(p.b5); q.b6 = rfl(p.b6);
  q.w1 = rfl(p.w1); q.w2 = rfl(p.w2); q.w3 = rfl(p.w3);
  q.w4 = rfl(p.w4); q.w5 = rfl(p.w5); q.w6 = rfl(p.w6);
  q.cmax = __uint_as_float(rfl(__float_as_uint(p.cmax)));
  q.ok = rfl(p.ok ? 1u : 0u) != 0u;
  return q;
}

// Group of block b (0..6; blocks at or beyond n_blk report group 6).
__device__ __forceinline__ int block_group(const SegProj& p, uint32_t b) {
  return (b >= p.b1) + (b >= p.b2) + (b >= p.b3) + (b >= p.b4) + (b >= p.b5) + (b >= p.b6);
}

__device__ __forceinline__ int group_width(int g) {
  return g < 4 ? g + 1 : (g == 4 ? 6 : (g == 5 ? 8 : 16));
}

// First word of block b inside a segment record (b = n_blk gives seg_words).
__device__ __forceinline__ uint32_t block_word(const SegProj& p, uint32_t b) {
  if (b >= p.n_blk) return p.seg_words;
  const int g = block_group(p, b);
  uint32_t bs = 0, ws = 0;
  if (g == 1) { bs = p.b1; ws = p.w1; }
  if (g == 2) { bs = p.b2; ws = p.w2; }
  if (g == 3) { bs = p.b3; ws = p.w3; }
  if (g == 4) { bs = p.b4; ws = p.w4; }
  if (g == 5) { bs = p.b5; ws = p.w5; }
  if (g == 6) { bs = p.b6; ws = p.w6; }
  return ws + (b - bs) * 4u * (uint32_t)group_width(g);
}

// End of the chunk of blocks that starts at block b0 (a multiple of 8):
// whole K steps whose words fit an arena of max_words (>= 512) words.
__device__ __forceinline__ uint32_t chunk_end(const SegProj& p, uint32_t b0, uint32_t max_words) {
  if (b0 >= p.n_blk) return p.n_blk;
  const uint32_t w0 = block_word(p, b0);
  if (p.seg_words - w0 <= max_words) return p.n_blk;
  // steps of 8 blocks; one step takes at most 8 * 64 words, so one always fits
  uint32_t lo = 1, hi = min((p.n_blk - b0 + kBlkPerK - 1) / kBlkPerK, max_words / 32u);
  while (hi > lo) {
    const uint32_t mid = (lo + hi + 1) / 2;
    if (block_word(p, min(b0 + kBlkPerK * mid, p.n_blk)) - w0 <= max_words)
      lo = mid;
    else
      hi = mid - 1;
  }
  return min(b0 + kBlkPerK * lo, p.n_blk);
}

// Copy n16 16-byte units from src to the LDS arena dst with nl lanes
// (lp = 0..nl-1; each wave writes the 1 KB behind its first lane's unit).
__device__ __forceinline__ void stage16(void* dst, const gu32* src, uint32_t n16, int lp,
                                        int lane, int nl) {
  typedef __attribute__((address_space(1))) void gvoid;
  const uint64_t s = (uint64_t)src;
  uint8_t* d = static_cast<uint8_t*>(dst);
  for (int i = lp; i < (int)n16; i += nl)
    __builtin_amdgcn_global_load_lds((gvoid*)(s + 16 * (uint64_t)i),
                                     (lds_void*)(d + 16 * (size_t)(i - lane)), 16, 0, 0);
}

// The 4 codes of octet row rho in one block of width W <= 8, one per byte
// (byte u = slot u): bit 8 u + rho of plane word j is bit j of the code, so
// rotating word j right by rho - j (mod 32) puts every byte's bit on bit j
// of that byte (a 4-byte mask keeps them): one v_alignbit_b32 and one
// v_and_or_b32 per plane.
template <int W>
__device__ __forceinline__ uint32_t row_codes4(const uint32_t (&w)[W], int rho) {
  uint32_t c = 0;
#pragma unroll
  for (int j = 0; j < W; ++j)
    c |= __builtin_amdgcn_alignbit(w[j], w[j], (uint32_t)(rho - j) & 31u) & (0x01010101u << j);
  return c;
}

// 4 byte codes -> two fp16 pairs, exact: bytes become (1024 + q) by a byte
// permute under the exponent byte 0x64, then 1024 is subtracted.
__device__ __forceinline__ void codes_to_f16(uint32_t c, uint32_t& lo, uint32_t& hi) {
  const h2 k1024 = {(_Float16)1024.0f, (_Float16)1024.0f};
  const uint32_t a = __builtin_amdgcn_perm(0x64646464u, c, 0x04010400u);
  const uint32_t b = __builtin_amdgcn_perm(0x64646464u, c, 0x04030402u);
  lo = __builtin_bit_cast(uint32_t, __builtin_bit_cast(h2, a) - k1024);
  hi = __builtin_bit_cast(uint32_t, __builtin_bit_cast(h2, b) - k1024);
}

__device__ __forceinline__ f4 mfma(h8 a, h8 b, f4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ h8 h8_of(uint4 v) { return __builtin_bit_cast(h8, v); }

// Scale exponent S for coefficients bounded by x * y (x, y >= 0):
// |c| 2^S < 2^14 (0 when the bound is 0 or not finite).
__device__ __forceinline__ int coef_shift(float x, float y) {
  if (!(x > 0.f) || !(y > 0.f) || !(x < 3.0e38f) || !(y < 3.0e38f)) return 0;
  int ex, ey;
  (void)frexpf(x, &ex);
  (void)frexpf(y, &ey);
  return 14 - ex - ey;
}

// hi + lo fp16 parts of c * 2^S.
__device__ __forceinline__ void split_coef(float c, int S, _Float16& hi, _Float16& lo) {
  const float v = ldexpf(c, S);
  hi = (_Float16)v;
  lo = (_Float16)(v - (float)hi);
}

// Words [0, W) of a block's row octet, read with the widest LDS loads the
// alignment allows (oct points at word oct_index * W of a 16-byte aligned
// block record).
template <int W>
__device__ __forceinline__ void load_oct(const uint32_t* oct, uint32_t (&w)[W]) {
  if constexpr (W == 2 || W == 6) {
#pragma unroll
    for (int i = 0; i < W / 2; ++i) {
      const uint2 v = reinterpret_cast<const uint2*>(oct)[i];
      w[2 * i] = v.x;
      w[2 * i + 1] = v.y;
    }
  } else if constexpr (W == 4 || W == 8) {
#pragma unroll
    for (int i = 0; i < W / 4; ++i) {
      const uint4 v = reinterpret_cast<const uint4*>(oct)[i];
      w[4 * i] = v.x;
      w[4 * i + 1] = v.y;
      w[4 * i + 2] = v.z;
      w[4 * i + 3] = v.w;
    }
  } else {
#pragma unroll
    for (int i = 0; i < W; ++i) w[i] = oct[i];
  }
}

// A operands of a K step whose 8 blocks all have width W <= 8: this lane's
// two blocks start at rec (block 2 kg of the step) and rec + 4 W.
template <int W>
__device__ __forceinline__ void a_tiles_uniform(const uint32_t* rec, int m, h8& a0, h8& a1) {
  const int rho = m & 7, o = m >> 3;
  uint32_t v[2][4];
#pragma unroll
  for (int tile = 0; tile < 2; ++tile) {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      uint32_t w[W];
      load_oct<W>(rec + 4 * W * t + (2 * tile + o) * W, w);
      codes_to_f16(row_codes4<W>(w, rho), v[tile][2 * t], v[tile][2 * t + 1]);
    }
  }
  union {
    uint32_t u[4];
    h8 h;
  } o0, o1;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    o0.u[i] = v[0][i];
    o1.u[i] = v[1][i];
  }
  a0 = o0.h;
  a1 = o1.h;
}

// A operands of a K step of 16-bit blocks: fp16 values read directly.
__device__ __forceinline__ void a_tiles_f16(const uint32_t* rec, int m, h8& a0, h8& a1) {
  const int o = m >> 3, r = m & 7;
  uint2 v[2][2];
#pragma unroll
  for (int tile = 0; tile < 2; ++tile)
#pragma unroll
    for (int t = 0; t < 2; ++t)
      v[tile][t] = *reinterpret_cast<const uint2*>(rec + 64 * t + (2 * tile + o) * 16 + 2 * r);
  union {
    uint2 u[2];
    h8 h;
  } o0, o1;
  o0.u[0] = v[0][0];
  o0.u[1] = v[0][1];
  o1.u[0] = v[1][0];
  o1.u[1] = v[1][1];
  a0 = o0.h;
  a1 = o1.h;
}

// B operand (fp16 hi and lo coefficients) of one lane for K step kb.
__device__ __forceinline__ void b_operand(const _Float16* chi, const _Float16* clo, int cstride,
                                          uint32_t s0, int nt, uint32_t kb, int m, int kg,
                                          uint4& vh, uint4& vl) {
  vh = make_uint4(0, 0, 0, 0);
  vl = make_uint4(0, 0, 0, 0);
  if (m < nt) {
    const uint32_t so = (uint32_t)m * cstride + 32u * kb + 8u * kg - s0;
    vh = *reinterpret_cast<const uint4*>(chi + so);
    vl = *reinterpret_cast<const uint4*>(clo + so);
  }
}

__device__ __forceinline__ void mfma4(const h8& a0, const h8& a1, const uint4& vh, const uint4& vl,
                                      f4& acc0, f4& acc1) {
  const h8 bh = h8_of(vh), bl = h8_of(vl);
  acc0 = mfma(a0, bh, acc0);
  acc1 = mfma(a1, bh, acc1);
  acc0 = mfma(a0, bl, acc0);
  acc1 = mfma(a1, bl, acc1);
}

// K steps kb = kfirst, kfirst + nw, ... < kend, all of width W (W = 16:
// fp16 values).  rec0: record of block 2 kg of step kfirst.  The next
// step's words and coefficients are loaded before this step is decoded.
template <int W>
__device__ __forceinline__ void ksteps_uniform(const uint32_t* rec0, uint32_t kfirst, uint32_t kend,
                                               const _Float16* chi, const _Float16* clo,
                                               int cstride, uint32_t s0, int nt, int m, int kg,
                                               f4& acc0, f4& acc1) {
  if (kfirst >= kend) return;
  constexpr uint32_t nw = kPW;
  const uint32_t rstep = nw * kBlkPerK * 4u * (W == 16 ? 16u : (uint32_t)W);
  if constexpr (W == 16) {
#pragma unroll 2
    for (uint32_t kb = kfirst; kb < kend; kb += nw, rec0 += rstep) {
      uint4 vh, vl;
      b_operand(chi, clo, cstride, s0, nt, kb, m, kg, vh, vl);
      h8 a0, a1;
      a_tiles_f16(rec0, m, a0, a1);
      mfma4(a0, a1, vh, vl, acc0, acc1);
    }
  } else {
#pragma unroll 2
    for (uint32_t kb = kfirst; kb < kend; kb += nw, rec0 += rstep) {
      uint4 vh, vl;
      b_operand(chi, clo, cstride, s0, nt, kb, m, kg, vh, vl);
      h8 a0, a1;
      a_tiles_uniform<W>(rec0, m, a0, a1);
      mfma4(a0, a1, vh, vl, acc0, acc1);
    }
  }
}

// The steps of one width group inside [kb0, kb1) that this wave owns
// (kb = kb0 + wp mod 4): bs, be are the group's first and end blocks (whole
// K steps), ws its first word.
template <int W>
__device__ __forceinline__ void group_steps(const uint32_t* base, uint32_t bs, uint32_t be,
                                            uint32_t ws, uint32_t kb0, uint32_t kb1, int wp,
                                            const _Float16* chi, const _Float16* clo,
                                            int cstride, uint32_t s0, int nt, int m, int kg,
                                            f4& acc0, f4& acc1) {
  const uint32_t ks = max(bs / kBlkPerK, kb0), ke = min(be / kBlkPerK, kb1);
  const uint32_t kf = ks + ((kb0 + (uint32_t)wp - ks) & (uint32_t)(kPW - 1));
  if (kf >= ke) return;
  constexpr uint32_t bw = 4u * (W == 16 ? 16u : (uint32_t)W);  // words per block
  const uint32_t* rec0 = base + ws + (kBlkPerK * kf - bs) * bw + 2u * bw * (uint32_t)kg;
  ksteps_uniform<W>(rec0, kf, ke, chi, clo, cstride, s0, nt, m, kg, acc0, acc1);
}

// This wave's K steps of one segment: kb = kb0 + wp, kb0 + wp + 4, ... < kb1
// (acc0 gets rows 0-15, acc1 rows 16-31, column n = token n).
//  base: word 0 of the segment record (the staged chunk holds these steps)
//  chi, clo: fp16 coefficient parts, token n's slot s at n * cstride + s - s0
//  nt:   tokens (columns) present; lanes of other columns use zero operands
// Width groups are padded to whole 32-slot steps, so every step has one
// width: each group runs a tight loop with its width as a constant.
__device__ __forceinline__ void mfma_ksteps(const SegProj& p, const uint32_t* base,
                                            const _Float16* chi, const _Float16* clo,
                                            int cstride, uint32_t s0, int nt, uint32_t kb0,
                                            uint32_t kb1, int wp, int lane, f4& acc0,
                                            f4& acc1) {
  const int m = lane & 15, kg = lane >> 4;
  kb0 = rfl(kb0);
  kb1 = rfl(kb1);
  group_steps<1>(base, 0u, p.b1, 0u, kb0, kb1, wp, chi, clo, cstride, s0, nt, m, kg, acc0, acc1);
  group_steps<2>(base, p.b1, p.b2, p.w1, kb0, kb1, wp, chi, clo, cstride, s0, nt, m, kg, acc0, acc1);
  group_steps<3>(base, p.b2, p.b3, p.w2, kb0, kb1, wp, chi, clo, cstride, s0, nt, m, kg, acc0, acc1);
  group_steps<4>(base, p.b3, p.b4, p.w3, kb0, kb1, wp, chi, clo, cstride, s0, nt, m, kg, acc0, acc1);
  group_steps<6>(base, p.b4, p.b5, p.w4, kb0, kb1, wp, chi, clo, cstride, s0, nt, m, kg, acc0, acc1);
  group_steps<8>(base, p.b5, p.b6, p.w5, kb0, kb1, wp, chi, clo, cstride, s0, nt, m, kg, acc0, acc1);
  group_steps<16>(base, p.b6, p.n_blk, p.w6, kb0, kb1, wp, chi, clo, cstride, s0, nt, m, kg, acc0, acc1);
}

// The same K steps with the B operand read straight from the tile's
// coefficient tables in global memory (no LDS copy, no chunk barriers): bh
// and bl point at this lane's 16-byte piece of step 0 (token row m, slots
// 8 kg .. + 7), step kb at + 32 kb.  Each step's B is loaded two steps ahead
// of its products.  Rows past the tile's tokens may hold anything finite:
// they only feed output columns that are never stored.
template <int W>
__device__ __forceinline__ void ksteps_gb(const uint32_t* rec0, uint32_t kfirst, uint32_t kend,
                                          const _Float16* bh, const _Float16* bl, int m,
                                          f4& acc0, f4& acc1) {
  if (kfirst >= kend) return;
  constexpr uint32_t nw = kPW;
  const uint32_t rstep = nw * kBlkPerK * 4u * (W == 16 ? 16u : (uint32_t)W);
  const uint4 zero = make_uint4(0, 0, 0, 0);
  uint4 h0 = *reinterpret_cast<const uint4*>(bh + 32u * kfirst), l0 = *reinterpret_cast<const uint4*>(bl + 32u * kfirst);
  uint4 h1 = zero, l1 = zero;
  if (kfirst + nw < kend) {
    h1 = *reinterpret_cast<const uint4*>(bh + 32u * (kfirst + nw));
    l1 = *reinterpret_cast<const uint4*>(bl + 32u * (kfirst + nw));
  }
#pragma unroll 1
  for (uint32_t kb = kfirst; kb < kend; kb += nw, rec0 += rstep) {
    const uint4 vh = h0, vl = l0;
    h0 = h1;
    l0 = l1;
    if (kb + 2u * nw < kend) {
      h1 = *reinterpret_cast<const uint4*>(bh + 32u * (kb + 2u * nw));
      l1 = *reinterpret_cast<const uint4*>(bl + 32u * (kb + 2u * nw));
    }
    h8 a0, a1;
    if constexpr (W == 16)
      a_tiles_f16(rec0, m, a0, a1);
    else
      a_tiles_uniform<W>(rec0, m, a0, a1);
    mfma4(a0, a1, vh, vl, acc0, acc1);
  }
}

template <int W>
__device__ __forceinline__ void group_steps_gb(const uint32_t* base, uint32_t bs, uint32_t be,
                                               uint32_t ws, uint32_t kb0, uint32_t kb1, int wp,
                                               const _Float16* bh, const _Float16* bl, int m,
                                               int kg, f4& acc0, f4& acc1) {
  const uint32_t ks = max(bs / kBlkPerK, kb0), ke = min(be / kBlkPerK, kb1);
  const uint32_t kf = ks + ((kb0 + (uint32_t)wp - ks) & (uint32_t)(kPW - 1));
  if (kf >= ke) return;
  constexpr uint32_t bw = 4u * (W == 16 ? 16u : (uint32_t)W);  // words per block
  const uint32_t* rec0 = base + ws + (kBlkPerK * kf - bs) * bw + 2u * bw * (uint32_t)kg;
  ksteps_gb<W>(rec0, kf, ke, bh, bl, m, acc0, acc1);
}

// This wave's K steps kb0 + wp, kb0 + wp + 4, ... < kb1 of one segment with
// B from the coefficient tables (acc0 rows 0-15, acc1 rows 16-31, column n =
// token n); base: word 0 of the segment record (the staged chunk holds
// these steps).
__device__ __forceinline__ void mfma_ksteps_gb(const SegProj& p, const uint32_t* base,
                                               const _Float16* bh, const _Float16* bl,
                                               uint32_t kb0, uint32_t kb1, int wp, int lane,
                                               f4& acc0, f4& acc1) {
  const int m = lane & 15, kg = lane >> 4;
  kb0 = rfl(kb0);
  kb1 = rfl(kb1);
  group_steps_gb<1>(base, 0u, p.b1, 0u, kb0, kb1, wp, bh, bl, m, kg, acc0, acc1);
  group_steps_gb<2>(base, p.b1, p.b2, p.w1, kb0, kb1, wp, bh, bl, m, kg, acc0, acc1);
  group_steps_gb<3>(base, p.b2, p.b3, p.w2, kb0, kb1, wp, bh, bl, m, kg, acc0, acc1);
  group_steps_gb<4>(base, p.b3, p.b4, p.w3, kb0, kb1, wp, bh, bl, m, kg, acc0, acc1);
  group_steps_gb<6>(base, p.b4, p.b5, p.w4, kb0, kb1, wp, bh, bl, m, kg, acc0, acc1);
  group_steps_gb<8>(base, p.b5, p.b6, p.w5, kb0, kb1, wp, bh, bl, m, kg, acc0, acc1);
  group_steps_gb<16>(base, p.b6, p.n_blk, p.w6, kb0, kb1, wp, bh, bl, m, kg, acc0, acc1);
}

// The same for nb (up to kMaxNB) tiles of one expert: each step's A operands are
// decoded once and multiplied with every tile's B; tile t's lane piece of
// step 0 is at thi / tlo + boff[t], step kb at + 32 kb.  Each tile's B of
// the next step is loaded right after this step's products with it.
constexpr int kMaxNB = 2;

template <int W>
__device__ __forceinline__ void ksteps_gbn(const uint32_t* rec0, uint32_t kfirst, uint32_t kend,
                                           const _Float16* thi, const _Float16* tlo,
                                           const uint32_t (&boff)[kMaxNB], int nb, int m,
                                           f4 (&acc0)[kMaxNB], f4 (&acc1)[kMaxNB]) {
  if (kfirst >= kend) return;
  constexpr uint32_t nw = kPW;
  const uint32_t rstep = nw * kBlkPerK * 4u * (W == 16 ? 16u : (uint32_t)W);
  uint4 vh[kMaxNB], vl[kMaxNB];
#pragma unroll
  for (int t = 0; t < kMaxNB; ++t) {
    vh[t] = vl[t] = make_uint4(0, 0, 0, 0);
    if (t < nb) {
      vh[t] = *reinterpret_cast<const uint4*>(thi + boff[t] + 32u * kfirst);
      vl[t] = *reinterpret_cast<const uint4*>(tlo + boff[t] + 32u * kfirst);
    }
  }
#pragma unroll 1
  for (uint32_t kb = kfirst; kb < kend; kb += nw, rec0 += rstep) {
    h8 a0, a1;
    if constexpr (W == 16)
      a_tiles_f16(rec0, m, a0, a1);
    else
      a_tiles_uniform<W>(rec0, m, a0, a1);
    const bool more = kb + nw < kend;
#pragma unroll
    for (int t = 0; t < kMaxNB; ++t) {
      if (t < nb) {
        mfma4(a0, a1, vh[t], vl[t], acc0[t], acc1[t]);
        if (more) {
          vh[t] = *reinterpret_cast<const uint4*>(thi + boff[t] + 32u * (kb + nw));
          vl[t] = *reinterpret_cast<const uint4*>(tlo + boff[t] + 32u * (kb + nw));
        }
      }
    }
  }
}

template <int W>
__device__ __forceinline__ void group_steps_gbn(const uint32_t* base, uint32_t bs, uint32_t be,
                                                uint32_t ws, uint32_t kb0, uint32_t kb1, int wp,
                                                const _Float16* thi, const _Float16* tlo,
                                                const uint32_t (&boff)[kMaxNB], int nb, int m,
                                                int kg, f4 (&acc0)[kMaxNB], f4 (&acc1)[kMaxNB]) {
  const uint32_t ks = max(bs / kBlkPerK, kb0), ke = min(be / kBlkPerK, kb1);
  const uint32_t kf = ks + ((kb0 + (uint32_t)wp - ks) & (uint32_t)(kPW - 1));
  if (kf >= ke) return;
  constexpr uint32_t bw = 4u * (W == 16 ? 16u : (uint32_t)W);  // words per block
  const uint32_t* rec0 = base + ws + (kBlkPerK * kf - bs) * bw + 2u * bw * (uint32_t)kg;
  ksteps_gbn<W>(rec0, kf, ke, thi, tlo, boff, nb, m, acc0, acc1);
}

__device__ __forceinline__ void mfma_ksteps_gbn(const SegProj& p, const uint32_t* base,
                                                const _Float16* thi, const _Float16* tlo,
                                                const uint32_t (&boff)[kMaxNB], int nb,
                                                uint32_t kb0, uint32_t kb1, int wp, int lane,
                                                f4 (&acc0)[kMaxNB], f4 (&acc1)[kMaxNB]) {
  const int m = lane & 15, kg = lane >> 4;
  kb0 = rfl(kb0);
  kb1 = rfl(kb1);
  group_steps_gbn<1>(base, 0u, p.b1, 0u, kb0, kb1, wp, thi, tlo, boff, nb, m, kg, acc0, acc1);
  group_steps_gbn<2>(base, p.b1, p.b2, p.w1, kb0, kb1, wp, thi, tlo, boff, nb, m, kg, acc0, acc1);
  group_steps_gbn<3>(base, p.b2, p.b3, p.w2, kb0, kb1, wp, thi, tlo, boff, nb, m, kg, acc0, acc1);
  group_steps_gbn<4>(base, p.b3, p.b4, p.w3, kb0, kb1, wp, thi, tlo, boff, nb, m, kg, acc0, acc1);
  group_steps_gbn<6>(base, p.b4, p.b5, p.w4, kb0, kb1, wp, thi, tlo, boff, nb, m, kg, acc0, acc1);
  group_steps_gbn<8>(base, p.b5, p.b6, p.w5, kb0, kb1, wp, thi, tlo, boff, nb, m, kg, acc0, acc1);
  group_steps_gbn<16>(base, p.b6, p.n_blk, p.w6, kb0, kb1, wp, thi, tlo, boff, nb, m, kg, acc0,
                      acc1);
}

// ---------------------------------------------------------------------------
// Integer apply for one token column (the one-launch kernel).
//
// Coefficients of 1..8-bit slots become integers v = rint(c 2^S) with
// |v| < 2^30 (S from the largest such |c| of the projection), stored as four
// signed 8-bit digits v = sum_n 2^(8 n) d_n (each in [-128, 127]); v keeps
// the full float precision of every c within 2^6 of that maximum.  With one
// token, the B operand's 16 columns carry the four digit rows (column n =
// digit n, columns 4..15 zero), so one v_mfma_i32_16x16x64_i8 per 16-row
// tile applies a 64-slot step: the decoded code bytes are the A operand as
// they come out of the plane decode, and every product and sum is exact in
// int32 (|code| <= 128, |digit| <= 128, <= 4.4k slots).  The columns are
// folded once per unit: y = sum_n 2^(8 n) C[., n].  Width-8 codes (0..255)
// enter as code - 128; the caller adds back 128 * sum of their v.  16-bit
// slots have a scale S16 of their own and use v_mfma_f32_16x16x32_f16 with
// the fp16 hi and lo parts of v 2^-16 in columns 0 and 1.  Lane l holds row
// l % 16 of a tile and the slots of one quarter (l / 16) of the step, in A
// and B alike, so the contraction covers the whole step.
typedef int i32x4 __attribute__((ext_vector_type(4)));
constexpr int kDigits = 4;

// S for coefficients bounded by mx: |c| 2^S < 2^30 (0 when mx is 0 or not
// finite).
__device__ __forceinline__ int digit_shift(float mx) {
  if (!(mx > 0.f) || !(mx < 3.0e38f)) return 0;
  int e;
  (void)frexpf(mx, &e);
  return 30 - e;
}

// The four digit bytes of v in one word (byte n = digit n): adding 0x80 to
// every byte lets the carries of a 32-bit add perform the balanced
// base-256 split, and the xor recentres each byte (|v| <= 2^30).
__device__ __forceinline__ uint32_t digit_bytes(int v) {
  return ((uint32_t)v + 0x80808080u) ^ 0x80808080u;
}

// 4 x 4 byte transpose: words a, b, c, d (one slot each, byte n = digit n)
// become rows r[n] = digit n of (a, b, c, d) in bytes 0..3.
__device__ __forceinline__ void transpose4(uint32_t a, uint32_t b, uint32_t c, uint32_t d,
                                           uint32_t (&r)[4]) {
  const uint32_t ab_lo = __builtin_amdgcn_perm(b, a, 0x05010400u);  // a0 b0 a1 b1
  const uint32_t ab_hi = __builtin_amdgcn_perm(b, a, 0x07030602u);  // a2 b2 a3 b3
  const uint32_t cd_lo = __builtin_amdgcn_perm(d, c, 0x05010400u);
  const uint32_t cd_hi = __builtin_amdgcn_perm(d, c, 0x07030602u);
  r[0] = __builtin_amdgcn_perm(cd_lo, ab_lo, 0x05040100u);
  r[1] = __builtin_amdgcn_perm(cd_lo, ab_lo, 0x07060302u);
  r[2] = __builtin_amdgcn_perm(cd_hi, ab_hi, 0x05040100u);
  r[3] = __builtin_amdgcn_perm(cd_hi, ab_hi, 0x07060302u);
}

__device__ __forceinline__ i32x4 mfma_i8(i32x4 a, i32x4 b, i32x4 c) {
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}

// A operand of tile `tile` (rows 16 tile .. + 15) for this lane's 4 blocks of
// width W <= 8 starting at `rec` (block record words, 4 W per block).
template <int W>
__device__ __forceinline__ i32x4 a_i8(const uint32_t* rec, int m, int tile) {
  i32x4 a;
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    uint32_t w[W];
    load_oct<W>(rec + 4 * W * d + (2 * tile + (m >> 3)) * W, w);
    uint32_t c = row_codes4<W>(w, m & 7);
    if constexpr (W == 8) c ^= 0x80808080u;  // code - 128 in every byte
    a[d] = (int)c;
  }
  return a;
}

// Steps of one width group W <= 8 inside K32 range [s, e) (K32 index k =
// slots 32 k .. + 31): 64-slot steps from s, the wave taking the steps i
// with (i + off) % 4 == wp; a trailing half step (e - s odd) uses zero codes
// and digits in its upper lanes and reads nothing there.  Block b's record:
// base + ws + (b - bs) 4 W.  lb: digit rows, row n at lb + n * ldig.
template <int W>
__device__ __forceinline__ void i8_group(const uint32_t* base, uint32_t bs, uint32_t ws,
                                         uint32_t s, uint32_t e, uint32_t off, int wp,
                                         const int8_t* lb, uint32_t ldig, int lane,
                                         i32x4& acc0, i32x4& acc1) {
  if (e <= s) return;
  const int m = lane & 15, g = lane >> 4;
  const uint32_t n64 = (e - s + 1) / 2;
  const uint32_t i0 = ((uint32_t)wp + 4u - (off & 3u)) & 3u;
  const i32x4 zero = {0, 0, 0, 0};
  const int8_t* lbn = lb + (m & 3) * ldig;  // this lane's digit row (columns >= 4: zero)
#pragma unroll 1
  for (uint32_t i = i0; i < n64; i += 4) {
    const uint32_t k = s + 2 * i;
    const bool valid = g < 2 || k + 1 < e;
    i32x4 b = zero, a0 = zero, a1 = zero;
    if (valid) {
      const i32x4 bv = *reinterpret_cast<const i32x4*>(lbn + 32u * k + 16u * (uint32_t)g);
      b = m < kDigits ? bv : zero;
      const uint32_t* rec = base + ws + (8u * k + 4u * (uint32_t)g - bs) * 4u * W;
      a0 = a_i8<W>(rec, m, 0);
      a1 = a_i8<W>(rec, m, 1);
    }
    acc0 = mfma_i8(a0, b, acc0);
    acc1 = mfma_i8(a1, b, acc1);
  }
}

// 16-bit group steps [s, e) (K32) on the fp16 path: A = the stored fp16
// values, B column 0 = hi and column 1 = lo fp16 parts of v 2^-16 rebuilt
// from v's digits (|v 2^-16| < 2^14 stays in fp16 range; hi + lo keeps 22
// bits of v): the sums are in units of 2^(16 - S16).
__device__ __forceinline__ void f16_group(const uint32_t* base, uint32_t bs, uint32_t ws,
                                          uint32_t s, uint32_t e, uint32_t off, int wp,
                                          const int8_t* lb, uint32_t ldig, int lane, f4& acc0,
                                          f4& acc1) {
  if (e <= s) return;
  const int m = lane & 15, kg = lane >> 4;
  const uint32_t i0 = ((uint32_t)wp + 4u - (off & 3u)) & 3u;
#pragma unroll 1
  for (uint32_t k = s + i0; k < e; k += 4) {
    uint4 bv = make_uint4(0, 0, 0, 0);
    if (m < 2) {
      const uint32_t so = 32u * k + 8u * (uint32_t)kg;
      uint2 q[kDigits];
#pragma unroll
      for (int l = 0; l < kDigits; ++l) q[l] = *reinterpret_cast<const uint2*>(lb + l * ldig + so);
      union {
        _Float16 h[8];
        uint4 u;
      } hv;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int sh = 8 * (j & 3);
        float fv = 0.f;
#pragma unroll
        for (int l = kDigits - 1; l >= 0; --l)
          // sign extension through int8_t: the sbfe builtin's result was
          // converted as unsigned by this compiler
          fv = fv * 256.f + (float)(int)(int8_t)((j < 4 ? q[l].x : q[l].y) >> sh);
        fv *= 1.52587890625e-05f;  // 2^-16, exact
        const _Float16 hi = (_Float16)fv;
        hv.h[j] = m == 0 ? hi : (_Float16)(fv - (float)hi);
      }
      bv = hv.u;
    }
    h8 a0, a1;
    a_tiles_f16(base + ws + (8u * k + 2u * (uint32_t)kg - bs) * 64u, m, a0, a1);
    const h8 b = h8_of(bv);
    acc0 = mfma(a0, b, acc0);
    acc1 = mfma(a1, b, acc1);
  }
}

// This wave's share of the K32 steps [kb0, kb1) of a segment (the staged
// chunk holds them; base: word 0 of the segment record).  Integer sums go
// to acc_t (tile t, column n = digit n, units of 2^(8 n - S)), fp16-column
// sums to acc16_t (column 0 hi, 1 lo, units of 2^(16 - S16)).  Steps are
// dealt to the waves round-robin across groups.
__device__ __forceinline__ void i8_ksteps(const SegProj& p, const uint32_t* base,
                                          const int8_t* lb, uint32_t ldig, uint32_t kb0,
                                          uint32_t kb1, int wp, int lane, i32x4& acc_0,
                                          i32x4& acc_1, f4& acc16_0, f4& acc16_1) {
  kb0 = rfl(kb0);
  kb1 = rfl(kb1);
  const uint32_t gb[kNumGroups + 1] = {0u, p.b1, p.b2, p.b3, p.b4, p.b5, p.b6, p.n_blk};
  const uint32_t gw[kNumGroups] = {0u, p.w1, p.w2, p.w3, p.w4, p.w5, p.w6};
  uint32_t off = 0;
#pragma unroll
  for (int g = 0; g < kNumGroups; ++g) {
    const uint32_t s = max(gb[g] / kBlkPerK, kb0), e = min(gb[g + 1] / kBlkPerK, kb1);
    const uint32_t n = e > s ? e - s : 0u;
    switch (g) {
      case 0: i8_group<1>(base, gb[g], gw[g], s, e, off, wp, lb, ldig, lane, acc_0, acc_1); break;
      case 1: i8_group<2>(base, gb[g], gw[g], s, e, off, wp, lb, ldig, lane, acc_0, acc_1); break;
      case 2: i8_group<3>(base, gb[g], gw[g], s, e, off, wp, lb, ldig, lane, acc_0, acc_1); break;
      case 3: i8_group<4>(base, gb[g], gw[g], s, e, off, wp, lb, ldig, lane, acc_0, acc_1); break;
      case 4: i8_group<6>(base, gb[g], gw[g], s, e, off, wp, lb, ldig, lane, acc_0, acc_1); break;
      case 5: i8_group<8>(base, gb[g], gw[g], s, e, off, wp, lb, ldig, lane, acc_0, acc_1); break;
      default:
        f16_group(base, gb[g], gw[g], s, e, off, wp, lb, ldig, lane, acc16_0, acc16_1);
        break;
    }
    off += g < kNumGroups - 1 ? (n + 1) / 2 : n;
  }
}

}  // namespace seg
}  // namespace bitsmoe
