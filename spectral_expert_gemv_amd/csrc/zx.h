// z = Phi^T x produced inside a one-launch gate/up kernel and exchanged
// between its work-groups.
//
// BitsMoE blog note, Methodology, "first split": z = Phi^T x does not depend
// on the expert, so it is formed once per token and every routed expert
// reuses it.  In a one-launch kernel every work-group produces a run of z
// rows and every work-group that applies an expert needs all of them, so the
// values are exchanged through device memory:
//  * the producing waves publish each value as one 64-bit word (float bits |
//    launch tag << 32) into the launch's buffer of a ring (the tag picks
//    it), then add one to a hint counter without waiting for the stores; the
//    counters are cumulative over launches, so after the launch with tag g
//    their sum is g times the number of producing waves (modulo 2^32);
//  * a consumer polls the hint counters (bounded), then copies the token's
//    words into LDS with ordinary (L2-shared) loads and re-reads, with
//    device-coherent loads and bounded, any word whose tag is not yet there.
// All waits are bounded by the launch's spin limit: a time-out is reported to
// the caller (its rows become NaN) and the kernel still exits.
#pragma once
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.h"
#include "kernels.h"

namespace bitsmoe {
namespace zx {

typedef _Float16 hh2 __attribute__((ext_vector_type(2)));

constexpr int kPre = 4;          // Phi^T rows a producing wave loads up front
constexpr int kHint = 64;        // hint counters (one per 64th of the producing waves)
constexpr int kHintStride = 32;  // u32 between counters (one 128-byte line each)

__device__ __forceinline__ float fdot8(uint4 a, uint4 b, float acc) {
  const hh2* ha = reinterpret_cast<const hh2*>(&a);
  const hh2* hb = reinterpret_cast<const hh2*>(&b);
#pragma unroll
  for (int i = 0; i < 4; ++i) acc = __builtin_amdgcn_fdot2(ha[i], hb[i], acc, false);
  return acc;
}

// This lane's partial dot product of one Phi^T row (p: this lane's NU
// 16-byte units of the first NU * 512 inputs) with token tt's x, over all din
// inputs (units past NU * 512 are loaded here, a batch of 4 at a time).
template <int NU>
__device__ __forceinline__ float zpart(const FusedArgs& s, const uint4* prow, const uint4 (&p)[NU],
                                       const uint4 (&xv)[NU], int tt, int lane) {
  const uint4* xt = s.x + (size_t)tt * s.din8;
  float acc = 0.f;
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    const int i = lane + u * kWave;
    if (i < s.din8) acc = fdot8(p[u], tt == 0 ? xv[u] : xt[i], acc);
  }
  for (int i0 = NU * kWave; i0 < s.din8; i0 += 4 * kWave) {
    uint4 q4[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = i0 + lane + u * kWave;
      q4[u] = i < s.din8 ? prow[i] : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = i0 + lane + u * kWave;
      if (i < s.din8) acc = fdot8(q4[u], xt[i], acc);
    }
  }
  return acc;
}

__device__ __forceinline__ void publish_z(uint64_t* zt, int r, int tt, int n, float v,
                                          uint32_t tag) {
  const uint64_t w = ((uint64_t)tag << 32) | __float_as_uint(v);
  __hip_atomic_store(&zt[(size_t)tt * 2 * r + n], w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// One transposing exchange of a kPre-value reduction: lanes with bit O set
// keep the upper half of the values, the others the lower half.
template <int O>
__device__ __forceinline__ void tstep(float (&v)[kPre], bool up) {
#pragma unroll
  for (int i = 0; i < O; ++i) {
    const float send = up ? v[i] : v[i + O];
    const float keep = up ? v[i + O] : v[i];
    v[i] = keep + __shfl_xor(send, O, kWave);
  }
}

// A producing wave owns z rows [n0, n0 + nrw) of every token.  The loads of
// its first kPre Phi^T rows (NU 16-byte units a lane: the whole row for din
// <= NU * 512) and of x go out first, in straight-line code (so that they
// stay together and ahead of anything that depends on a load); z_finish then
// reduces the kPre partial sums together (2 transposing exchanges leave row
// lane & 3 in every lane, 4 more finish the sum) and lane i publishes row i.
// Rows beyond the first kPre follow kPre at a time, each batch's loads all
// issued before any is used.
template <int NU>
struct PhiRegs {
  uint4 pv[kPre][NU];
  uint4 xv[NU];
};

template <int NU>
__device__ __forceinline__ void phi_rows(const FusedArgs& s, int n0, int nrw, int j0, int lane,
                                         uint4 (&pv)[kPre][NU]) {
  const int R = 2 * s.g.r;
#pragma unroll
  for (int j = 0; j < kPre; ++j) {
    const int n = (j0 + j < nrw && n0 + j0 + j < R) ? n0 + j0 + j : 0;
    const uint4* prow = s.phi_t + (size_t)n * s.din8;
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const int i = lane + u * kWave;
      pv[j][u] = i < s.din8 ? prow[i] : make_uint4(0, 0, 0, 0);
    }
  }
}

template <int NU>
__device__ __forceinline__ void phi_issue(const FusedArgs& s, int n0, int nrw, int lane,
                                          PhiRegs<NU>& q) {
  phi_rows<NU>(s, n0, nrw, 0, lane, q.pv);
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    const int i = lane + u * kWave;
    q.xv[u] = i < s.din8 ? s.x[i] : make_uint4(0, 0, 0, 0);
  }
}

// z of rows n0 + j0 .. + kPre - 1 (those below nrw and R) for every token,
// from their loaded units pv, published by lanes 0 .. kPre - 1.
template <int NU>
__device__ __forceinline__ void z_batch(const FusedArgs& s, uint64_t* zt, int n0, int nrw, int j0,
                                        int lane, uint32_t tag, const uint4 (&pv)[kPre][NU],
                                        const uint4 (&xv)[NU]) {
  static_assert(kPre == 4, "the transposing reduction is written for 4 rows");
  const int R = 2 * s.g.r;
  // (T >= 1: a do-while leaves no path on which the x and Phi^T loads are
  // still outstanding when the hint increment is issued, which would make the
  // compiler wait for every store first)
  int tt = 0;
  do {
    float v[kPre];
#pragma unroll
    for (int j = 0; j < kPre; ++j) {
      const int n = (j0 + j < nrw && n0 + j0 + j < R) ? n0 + j0 + j : 0;
      v[j] = zpart<NU>(s, s.phi_t + (size_t)n * s.din8, pv[j], xv, tt, lane);
    }
    tstep<2>(v, (lane & 2) != 0);
    tstep<1>(v, (lane & 1) != 0);
    float z = v[0];
#pragma unroll
    for (int off = 4; off < kWave; off <<= 1) z += __shfl_xor(z, off, kWave);
    const int j = lane & 3;
    if (lane < kPre && j0 + j < nrw && n0 + j0 + j < R) publish_z(zt, s.g.r, tt, n0 + j0 + j, z, tag);
  } while (++tt < s.T);
}

template <int NU>
__device__ __forceinline__ void z_finish(const FusedArgs& s, uint64_t* zt, int n0, int nrw,
                                         int lane, uint32_t tag, const PhiRegs<NU>& q) {
  const int R = 2 * s.g.r;
  z_batch<NU>(s, zt, n0, nrw, 0, lane, tag, q.pv, q.xv);
  for (int j0 = kPre; j0 < nrw && n0 + j0 < R; j0 += kPre) {  // rows beyond the first kPre
    uint4 pv[kPre][NU];
    phi_rows<NU>(s, n0, nrw, j0, lane, pv);
    z_batch<NU>(s, zt, n0, nrw, j0, lane, tag, pv, q.xv);
  }
}

// Counts the producing wave `pw` on its hint counter (after its z stores
// were issued: the hint may run ahead of them, and a reader that comes too
// early finds old tags and re-reads those words).
__device__ __forceinline__ void hint_add(const FusedArgs& s, int pw, int lane) {
  if (lane == 0)
    __hip_atomic_fetch_add(s.hint + kHintStride * (pw & (kHint - 1)), 1u, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
}

// Bounded wait until the hint counters say that every producing wave of this
// launch has published: the counters are never reset, so after the launch
// with tag g their sum is g times the number of producing waves (modulo
// 2^32).  Lane i reads counter i; 64 counters on separate lines keep the
// producers' increments from contending.  Only a hint: the tags decide.  At
// most spin / 64 polls; false when the count was not reached.
__device__ __forceinline__ bool wait_hint(const uint32_t* hint, uint32_t target, uint32_t spin) {
  const int lane = threadIdx.x & (kWave - 1);
  uint32_t polls = 0;
  while (true) {
    const uint32_t c =
        __hip_atomic_load(hint + kHintStride * lane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const uint32_t tot = wave_sum_u32_dpp(c);  // modulo 2^32, like the target
    if ((int32_t)(tot - target) >= 0) return true;
    if (++polls >= spin / 64) return false;
    __builtin_amdgcn_s_sleep(4);
  }
}

// One more wait of this launch gave up (uniform condition; lane 0 counts
// it): the host reads the cumulative count, so a time-out that turned rows
// into NaN is never silent.
__device__ __forceinline__ void count_timeout(const FusedArgs& s, bool gave_up, int lane) {
  if (gave_up && lane == 0)
    __hip_atomic_fetch_add(s.timeouts, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The token's R tagged z words, copied into LDS as floats by the NT lanes of
// the work-group with coalesced loads (PER words per lane, NT * PER >= R).
// The first read is an ordinary (L2-cached) load, issued once the hint
// counters say that every producer's z stores have completed, so the
// work-groups of one XCD share one fetch; words whose tag is not there (a
// line an L2 kept from an older launch) are re-read with device-coherent
// loads until it is, at most `spin` rounds.  zmax gets this lane's largest
// |z|.  Returns false on a time-out (a spin limit of 0 gives up at once).
template <int NT, int PER>
__device__ __forceinline__ bool stage_z(const uint64_t* src, int R, uint32_t tag, float* Z,
                                        uint32_t spin, float& zmax) {
  uint64_t zw[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int i = (int)threadIdx.x + NT * j;
    zw[j] = i < R ? src[i] : ((uint64_t)tag << 32);
  }
  uint32_t spins = 0;
  while (true) {
    bool ready = true;
#pragma unroll
    for (int j = 0; j < PER; ++j) ready &= (uint32_t)(zw[j] >> 32) == tag;
    if (__all(ready) || spins >= spin) break;
    __builtin_amdgcn_s_sleep(2);
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int i = (int)threadIdx.x + NT * j;
      if ((uint32_t)(zw[j] >> 32) != tag)
        zw[j] = __hip_atomic_load(src + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    ++spins;
  }
  float mx = 0.f;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int i = (int)threadIdx.x + NT * j;
    const float v = __uint_as_float((uint32_t)zw[j]);
    if (i < R) Z[i] = v;
    mx = fmaxf(mx, i < R ? fabsf(v) : 0.f);
  }
  zmax = mx;
  return spins < spin;
}

}  // namespace zx
}  // namespace bitsmoe
