// Slot metadata of a one-launch gate/up kernel: each lane of a projection's
// 256 lanes holds the component index k, magnitude a and fp16 scale s and
// offset m of its slots in registers, loaded with 16-byte global loads and
// unpacked only where the coefficients are formed.
//
// BitsMoE blog note, Methodology, "second split": the coefficient of slot
// (column) k of expert e is a_{e,k} z_k, folded with the column's scale and
// offset of the quantized unit direction.
#pragma once
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "seg_common.h"

namespace bitsmoe {
namespace seg {

// Slot metadata of one lane: kFSper = 8 V + 1 slots, the 8 V contiguous
// slots 8 V lp .. 8 V lp + 8 V - 1 (read with 16-byte loads) and the tail
// slot 2048 V + lp (n_slot <= r + 7 * 31 < 2048 V + 256).  The raw loaded
// words are kept as they are and unpacked only where the coefficients are
// formed, so that nothing before that point waits for these loads.
template <int kFSper>
struct SlotMeta {
  static constexpr int V = (kFSper - 1) / 8;
  uint4 kq[V], a0[V], a1[V], sq[V], mq[V];  // kidx, a (2 x 4), s, m of 8 slots each
  uint32_t kt, at, st, mt;                  // the tail slot
};
template <int kFSper>
__device__ __forceinline__ uint32_t meta_slot(int lp, int i) {
  constexpr int V = SlotMeta<kFSper>::V;
  return i < 8 * V ? (uint32_t)(8 * V * lp + i) : (uint32_t)(2048 * V + lp);
}
// Every load is issued unconditionally (an index past the array is replaced
// by 0, inside the expert block) and through a global address (the
// descriptor's pointers are global ones); a load inside a branch, or a flat
// load (which also counts on the LDS counter), would make the wave wait for
// all of its outstanding loads right there.  A 16-byte vector that starts
// inside an array ends at most 28 bytes past it, still inside the expert
// block (the next array, or the planes and the block's 16-byte tail).
// A descriptor whose record failed its check has counts of 0, so every index
// is 0, and its arrays are all taken from kidx, the blob base then.
template <int kFSper>
__device__ __forceinline__ void load_meta(const SegProj& p, int lp, SlotMeta<kFSper>& md) {
  constexpr int V = SlotMeta<kFSper>::V;
  static_assert(kFSper == 8 * V + 1, "8 V contiguous slots and one tail slot");
  const gf32* A = p.ok ? p.A : (const gf32*)p.kidx;
  const gu16* S = p.ok ? p.S : p.kidx;
  const gu16* M = p.ok ? p.M : p.kidx;
  const uint32_t s0 = 8u * V * (uint32_t)lp;
#pragma unroll
  for (int v = 0; v < V; ++v) {
    const uint32_t sv = s0 + 8u * v;
    const uint32_t iq = sv < p.n_slot ? sv : 0u, ia = sv + 4 < p.n_slot ? sv + 4 : 0u;
    const uint32_t is = sv < p.n_qslot ? sv : 0u;
    md.kq[v] = ld16(p.kidx + iq);
    md.a0[v] = ld16(A + iq);
    md.a1[v] = ld16(A + ia);
    md.sq[v] = ld16(S + is);
    md.mq[v] = ld16(M + is);
  }
  const uint32_t sl = 2048u * V + (uint32_t)lp;
  const uint32_t ic = sl < p.n_slot ? sl : 0u, iq = sl < p.n_qslot ? sl : 0u;
  // 16-bit values through the aligned 32-bit word that holds them (the half
  // is picked where they are used)
  md.kt = *(const gu32*)(p.kidx + (ic & ~1u));
  md.at = *(const gu32*)(A + ic);
  md.st = *(const gu32*)(S + (iq & ~1u));
  md.mt = *(const gu32*)(M + (iq & ~1u));
}
// Slot i of the lane (see SlotMeta): component index k, magnitude a and
// fp16 s, m as floats; slots past the arrays give k = 0, a = 0, s = 1, m = 0.
template <int kFSper>
__device__ __forceinline__ void meta_get(const SlotMeta<kFSper>& md, int lp, int i,
                                         uint32_t n_slot, uint32_t n_qslot, uint32_t& k,
                                         float& a, float& sv, float& mv) {
  constexpr int V = SlotMeta<kFSper>::V;
  const uint32_t sl = meta_slot<kFSper>(lp, i);
  uint32_t kk, aa, ss, mm;
  if (i < 8 * V) {
    const int v = i >> 3, j = i & 7;
    const uint32_t kw[4] = {md.kq[v].x, md.kq[v].y, md.kq[v].z, md.kq[v].w};
    const uint32_t sw[4] = {md.sq[v].x, md.sq[v].y, md.sq[v].z, md.sq[v].w};
    const uint32_t mw[4] = {md.mq[v].x, md.mq[v].y, md.mq[v].z, md.mq[v].w};
    const uint32_t aw[8] = {md.a0[v].x, md.a0[v].y, md.a0[v].z, md.a0[v].w,
                            md.a1[v].x, md.a1[v].y, md.a1[v].z, md.a1[v].w};
    const uint32_t sh = 16 * (j & 1);
    kk = (kw[j >> 1] >> sh) & 0xFFFFu;
    ss = (sw[j >> 1] >> sh) & 0xFFFFu;
    mm = (mw[j >> 1] >> sh) & 0xFFFFu;
    aa = aw[j];
  } else {
    const uint32_t sh = 16 * (sl & 1);  // the tail slot's half of the loaded words
    kk = (md.kt >> sh) & 0xFFFFu;
    aa = md.at;
    ss = (md.st >> sh) & 0xFFFFu;
    mm = (md.mt >> sh) & 0xFFFFu;
  }
  k = sl < n_slot ? kk : 0u;
  a = sl < n_slot ? __uint_as_float(aa) : 0.f;
  sv = sl < n_qslot ? __half2float(__ushort_as_half((unsigned short)ss)) : 1.f;
  mv = sl < n_qslot ? __half2float(__ushort_as_half((unsigned short)mm)) : 0.f;
}

}  // namespace seg
}  // namespace bitsmoe
