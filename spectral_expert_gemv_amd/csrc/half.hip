// One-launch gate/up kernel: one 512-lane work-group per (token, slot,
// 32-row half of a 64-row slab), both projections, placed XCD-aware.
//
// BitsMoE blog note, Methodology: "first split" (z = Phi^T x once per token,
// reused by every routed expert), "second split" (an expert's output is the
// sum over components of magnitude * z_k * quantized unit direction) and
// "execution" (components of one width stored together, plane by plane).
// h = SiLU(y_gate) * y_up.
//
// gfx950 mapping.
//  * Work units.  Unit (q, half) with q = slab * pairs + pair covers 32 rows
//    of one (token, slot) pair for both projections, so SiLU * mul needs no
//    other work-group.  Units go to XCD q % 8: both halves of a slab (which
//    read the same 64-row plane masks) and, when there are at least 8 pairs,
//    every slab of a pair (which read the same column metadata) share one
//    L2, so HBM delivers those bytes once.  Work-group b runs on XCD b % 8
//    and takes that XCD's units b / 8, b / 8 + G / 8, ...
//  * Every wave first issues the loads of its 2r / (8 G) Phi^T rows; waves
//    0-3 then read the routed id and the gate directory record (waves 4-7:
//    up) with scalar loads and copy the slab's plane masks, column metadata
//    and fp16 half-columns into LDS with 16-byte global_load_lds.  Once its
//    loads are in, each wave computes its z rows (v_dot2_f32_f16, wave
//    reduction) and publishes each value as a 64-bit word (float bits |
//    epoch tag << 32) with one device-coherent store.
//  * Every work-group then loads the token's 2 r tagged z words (coalesced,
//    waiting for tags that are not there yet) into LDS.
//  * Decode: waves 0-3 take the gate columns, waves 4-7 the up columns, one
//    column per lane and round.  coef = a s z_k; the 32 bits of each plane
//    are spread into byte codes with SWAR arithmetic (a 4-bit field times
//    0x00204081 puts bit n at bit 8n) and coef * code is added to 32 row
//    registers; sum a m z_k is summed apart.  fp16 columns add coef * value.
//  * Each wave reduces its lanes with a transpose reduction (32 exchanges),
//    the 4 waves of a projection are added through LDS, and wave 0 writes
//    SiLU(gate) * up for the 32 rows.
// Layers whose slab does not fit the LDS arenas are processed in column
// chunks.  Groups wait for other groups' z, so the host launches at most as
// many groups as can be resident at once; all waits are bounded (time-out
// gives NaN rows, the kernel still exits).  The last group of the grid
// advances the epoch.
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include "device_common.h"
#include "format.h"
#include "kernels.h"
#include "slab_common.h"

namespace bitsmoe {
namespace {

using namespace slab;

constexpr int kHWaves = 8;
constexpr int kHThreads = kHWaves * kWave;  // 512
constexpr int kHProj = 256;                 // lanes per projection (waves 0-3 gate, 4-7 up)
constexpr int kHPW = kHWaves / 2;           // waves per projection
constexpr int kHRows = kSlabRows;
constexpr int kHMaxM = 5120;  // u64 per projection per chunk: masks, then 8 per fp16 column
constexpr int kHMaxC = 2048;  // columns per projection per chunk
constexpr int kHPre = 2;      // Phi^T rows a wave loads up front
constexpr uint32_t kHSpin = 1u << 20;
constexpr int kHZPer = 2 * kHalfMaxR / kHThreads;  // z words per lane

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

struct __align__(16) HalfLds {
  uint64_t M[2][kHMaxM + 2];
  float A[2][kHMaxC + 8];
  uint16_t K[2][kHMaxC + 16];
  uint16_t S[2][kHMaxC + 16];
  uint16_t Mo[2][kHMaxC + 16];
  float Z[2 * kHalfMaxR];
  float red[2][kHPW][kHRows];
  float bias[2][kHPW];
  uint32_t ok[2][kHPW];
  int nch[2];
};

__device__ __forceinline__ float hdot8(uint4 a, uint4 b, float acc) {
  const half2_t* ha = reinterpret_cast<const half2_t*>(&a);
  const half2_t* hb = reinterpret_cast<const half2_t*>(&b);
#pragma unroll
  for (int i = 0; i < 4; ++i) acc = __builtin_amdgcn_fdot2(ha[i], hb[i], acc, false);
  return acc;
}

__device__ __forceinline__ float hsettle(const uint64_t* p, uint64_t w, uint32_t tag,
                                         bool active) {
  bool ready = !active || (uint32_t)(w >> 32) == tag;
  uint32_t spins = 0;
  while (!__all(ready) && spins < kHSpin) {
    __builtin_amdgcn_s_sleep(1);
    if (!ready) {
      w = __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      ready = (uint32_t)(w >> 32) == tag;
    }
    ++spins;
  }
  if (!active) return 0.f;
  return ready ? __uint_as_float((uint32_t)w) : __builtin_nanf("");
}

// Every wave: z rows gw, gw + nw, ... of every token, published tagged.
__device__ __forceinline__ void hproduce_z(const HalfArgs& s, int gw, int nw, int lane,
                                           uint32_t tag, uint4 (&pv)[kHPre][4],
                                           uint4 (&xv)[4]) {
  const int R = 2 * s.g.r;
  for (int q = 0; gw + q * nw < R; ++q) {
    const int n = gw + q * nw;
    const uint4* prow = s.phi_t + (size_t)n * s.din8;
    uint4 p0[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = lane + u * kWave;
      if (q == 0) p0[u] = pv[0][u];
      else if (q == 1) p0[u] = pv[1][u];
      else p0[u] = i < s.din8 ? prow[i] : make_uint4(0, 0, 0, 0);
    }
    for (int tt = 0; tt < s.T; ++tt) {
      const uint4* xt = s.x + (size_t)tt * s.din8;
      float acc = 0.f;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int i = lane + u * kWave;
        if (i < s.din8) acc = hdot8(p0[u], tt == 0 ? xv[u] : xt[i], acc);
      }
      for (int i0 = 4 * kWave; i0 < s.din8; i0 += 4 * kWave) {  // din > 2048
        uint4 q4[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int i = i0 + lane + u * kWave;
          q4[u] = i < s.din8 ? prow[i] : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int i = i0 + lane + u * kWave;
          if (i < s.din8) acc = hdot8(q4[u], xt[i], acc);
        }
      }
      acc = wave_sum(acc);
      if (lane == 0) {
        const uint64_t w = ((uint64_t)tag << 32) | __float_as_uint(acc);
        __hip_atomic_store(&s.zt[(size_t)tt * R + n], w, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
}

__global__ __launch_bounds__(kHThreads) void k_gateup_half(HalfArgs s) {
  extern __shared__ __align__(16) uint8_t lds_raw[];
  HalfLds& L = *reinterpret_cast<HalfLds*>(lds_raw);
  const GateUpArgs& a = s.g;
  const int lane = threadIdx.x & (kWave - 1);
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int pj = wv >= kHPW ? 1 : 0;           // waves 0-3 gate, 4-7 up
  const int lp = (int)threadIdx.x & (kHProj - 1);
  const int R = 2 * a.r;
  const uint32_t G = (uint32_t)s.grid;
  const int np = a.npairs;
  const int Q = np * a.n_slabs;                // (pair, slab) units, q = slab * np + pair
  const int xcd = blockIdx.x & 7;
  const int per_xcd = (int)G >> 3;
  const uint32_t dout_pad = (uint32_t)a.n_slabs * 64u;
  const uint32_t tag =
      __hip_atomic_load(s.epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1u;

  const int gw = (int)blockIdx.x * kHWaves + wv;
  const int nw = (int)G * kHWaves;
  uint4 pv[kHPre][4];
  uint4 xv[4];

  int zt_cached = -1;  // token whose z is in L.Z
  bool first = true;
  for (int j = (int)blockIdx.x >> 3;; j += per_xcd) {
    const int q = 8 * (j >> 1) + xcd;
    const bool have = q < Q;
    if (!have && !first) break;
    const int hh = j & 1;
    const int pair = have ? q % np : 0;
    const int slab = have ? q / np : 0;
    const int t = pair / a.ktop;
    // ---- phase A: routed id, then the directory record (scalar loads); on
    // the first unit the Phi^T rows are issued right behind the record, so
    // the record is ahead of the Phi^T stream in the memory queues ----
    const int e = have ? __builtin_amdgcn_readfirstlane(a.ids[pair]) : 0;
    const uint8_t* blob = pj ? a.blob_u : a.blob_g;
    const DirRec drec = load_rec_s(blob, e, a.E);
    const HdrF hdr = load_hdr(blob);
    if (first) {
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int qq = 0; qq < kHPre; ++qq) {
        const int n = gw + qq * nw;
        const uint4* prow = s.phi_t + (size_t)(n < R ? n : 0) * s.din8;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int i = lane + u * kWave;
          pv[qq][u] = (n < R && i < s.din8) ? prow[i] : make_uint4(0, 0, 0, 0);
        }
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int i = lane + u * kWave;
        xv[u] = i < s.din8 ? s.x[i] : make_uint4(0, 0, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    const Proj P = make_proj(blob, pj ? a.bytes_u : a.bytes_g, e, drec, hdr, a);
    const HGeo Gm = hgeo(P);
    const uint32_t ncol = have ? P.nq + P.n16 : 0u;
    // chunk counts of both projections (they advance together)
    {
      int nc = 0;
      for (uint32_t c = 0; c < ncol; c = hchunk_end<kHMaxM, kHMaxC>(P, Gm, c)) ++nc;
      if (threadIdx.x == (unsigned)(pj * kHProj)) L.nch[pj] = nc;
    }
    __syncthreads();
    const int nch = max(L.nch[0], L.nch[1]);
    float acc[kHRows];
    float biasv = 0.f;
    bool good = P.ok;
    uint32_t c0 = 0;
    for (int ch = 0; ch < max(nch, 1); ++ch) {
      const uint32_t c1 = c0 < ncol ? hchunk_end<kHMaxM, kHMaxC>(P, Gm, c0) : c0;
      // ---- phase B: stage this projection's chunk (its 8 waves) ----
      if (c1 > c0) {
        const Arena ar = {&L.M[pj][0], &L.K[pj][0], &L.A[pj][0], &L.S[pj][0], &L.Mo[pj][0]};
        hstage_chunk(ar, P, c0, c1, slab, hh, dout_pad, lp, lane, kHProj);
      }
      // ---- first pass only: this wave's z rows, once its loads are in ----
      if (first && ch == 0) {
        __builtin_amdgcn_s_waitcnt(0);
        hproduce_z(s, gw, nw, lane, tag, pv, xv);
      }
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if (!have) break;
      // ---- phase C: the token's z into LDS (coalesced, tags checked) ----
      if (t != zt_cached) {
        const uint64_t* src = s.zt + (size_t)t * R;
        uint64_t zw[kHZPer];
#pragma unroll
        for (int u = 0; u < kHZPer; ++u) {
          const int i = (int)threadIdx.x + kHThreads * u;
          zw[u] = i < R ? __hip_atomic_load(src + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                        : 0ull;
        }
#pragma unroll
        for (int u = 0; u < kHZPer; ++u) {
          const int i = (int)threadIdx.x + kHThreads * u;
          if (u * kHThreads >= R) break;
          const float z = hsettle(src + i, zw[u], tag, i < R);
          if (i < R) L.Z[i] = z;
        }
        zt_cached = t;
        __syncthreads();
      }
      // ---- phase D: decode this projection's columns of the chunk ----
      if (ch == 0) {
#pragma unroll
        for (int i = 0; i < kHRows; ++i) acc[i] = 0.f;
      }
      {
        const uint32_t q0 = min(c0, P.nq), q1 = min(c1, P.nq);
        const uint32_t ma0 = ((uint32_t)slab * P.mps + hmask_of(Gm, q0)) & ~1u;
        const uint32_t mu = q1 > q0 ? hunits(ma0, (uint32_t)slab * P.mps + hmask_of(Gm, q1), 2)
                                    : 0u;
        const int n_items = (int)(c1 - c0);
        const int nqi = (int)(q1 - q0);
        const float* zrow = &L.Z[pj ? a.r : 0];
        const uint32_t* Mw = reinterpret_cast<const uint32_t*>(&L.M[pj][0]);
#pragma unroll 1
        for (int r0 = 0; r0 < n_items; r0 += kHProj) {
          const int it = r0 + (((r0 / kHProj) & 1) ? kHProj - 1 - lp : lp);
          const bool live = it < n_items;
          const uint32_t c = c0 + (uint32_t)(live ? it : 0);
          const uint32_t kk = live ? L.K[pj][c - (c0 & ~7u)] : 0u;
          good &= kk < (uint32_t)a.r;
          const float z = live ? zrow[kk < (uint32_t)a.r ? kk : 0u] : 0.f;
          const float av = live ? L.A[pj][c - (c0 & ~3u)] : 0.f;
          const float az = av * z;
          good &= !live || z == z;
          const bool isq = live && it < nqi;
          if (__any(isq)) {
            int grp = 0;
#pragma unroll
            for (int gg = 1; gg < kNumQGroups; ++gg) grp += c >= Gm.gcol[gg] ? 1 : 0;
            uint32_t gc = Gm.gcol[0], gm = Gm.gmask[0];
#pragma unroll
            for (int gg = 1; gg < kNumQGroups; ++gg) {
              if (grp == gg) {
                gc = Gm.gcol[gg];
                gm = Gm.gmask[gg];
              }
            }
            const int b = isq ? hwidth(grp) : 0;
            float coef = 0.f;
            uint32_t mi = 0;
            if (isq) {
              const uint32_t si = c - (q0 & ~7u);
              coef = az * __half2float(__ushort_as_half(L.S[pj][si]));
              biasv += az * __half2float(__ushort_as_half(L.Mo[pj][si]));
              mi = (uint32_t)slab * P.mps + gm + (c - gc) * (uint32_t)b - ma0;
            }
            const uint32_t* wp = Mw + 2 * mi + hh;
            switch (hwave_bmax(b)) {
              case 1: column32<1>(wp, b, coef, acc); break;
              case 2: column32<2>(wp, b, coef, acc); break;
              case 3: column32<3>(wp, b, coef, acc); break;
              case 4: column32<4>(wp, b, coef, acc); break;
              case 6: column32<6>(wp, b, coef, acc); break;
              case 8: column32<8>(wp, b, coef, acc); break;
              default: break;
            }
          }
          const bool isf = live && it >= nqi;
          if (__any(isf)) {
            const float coef = isf ? az : 0.f;
            const uint4* fv =
                reinterpret_cast<const uint4*>(&L.M[pj][2 * mu + 8 * (isf ? it - nqi : 0)]);
#pragma unroll
            for (int qq = 0; qq < 4; ++qq) {
              const uint4 v4 = fv[qq];
              const __half2* h2 = reinterpret_cast<const __half2*>(&v4);
#pragma unroll
              for (int u = 0; u < 4; ++u) {
                const float2 f2 = __half22float2(h2[u]);
                acc[8 * qq + 2 * u] = fmaf(coef, f2.x, acc[8 * qq + 2 * u]);
                acc[8 * qq + 2 * u + 1] = fmaf(coef, f2.y, acc[8 * qq + 2 * u + 1]);
              }
            }
          }
        }
      }
      __syncthreads();  // the arenas are restaged by the next chunk
      c0 = c1;
    }
    if (!have) break;
    // ---- phase E: row sums, SiLU * mul ----
    {
      const float v = htranspose_sum(acc, lane);
      const float bw = wave_sum(biasv);
      const bool wok = __all(good);
      const int wp = wv & (kHPW - 1);
      if (lane < kHRows) L.red[pj][wp][lane] = v;
      if (lane == 0) {
        L.bias[pj][wp] = bw;
        L.ok[pj][wp] = wok;
      }
    }
    __syncthreads();
    if (wv == 0 && lane < kHRows) {
      float gsum = 0.f, usum = 0.f;
      bool ok = true;
#pragma unroll
      for (int w = 0; w < kHPW; ++w) {
        gsum += L.red[0][w][lane] + L.bias[0][w];
        usum += L.red[1][w][lane] + L.bias[1][w];
        ok = ok && L.ok[0][w] && L.ok[1][w];
      }
      const int row = slab * 64 + hh * kHRows + lane;
      if (row < a.dout)
        a.h[(size_t)pair * a.dout + row] = ok ? silu_mul(gsum, usum) : __builtin_nanf("");
    }
    __syncthreads();  // red and nch are reused by the next unit
    first = false;
  }

  // ---- grid arrival: the last group advances the epoch ----
  if (threadIdx.x == 0) {
    const uint32_t n =
        __hip_atomic_fetch_add(s.arrive, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (n == G - 1) {
      __hip_atomic_store(s.arrive, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(s.epoch, tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

}  // namespace

size_t half_lds_bytes() { return sizeof(HalfLds); }

int half_grid() {
  static int grid[64];
  static bool done[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  if (!done[dev]) {
    int cus = 0, nb = 0;
    (void)hipFuncSetAttribute((const void*)k_gateup_half,
                              hipFuncAttributeMaxDynamicSharedMemorySize,
                              (int)sizeof(HalfLds));
    (void)hipGetLastError();
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, k_gateup_half, kHThreads,
                                                     sizeof(HalfLds)) != hipSuccess)
      return 0;
    // one group per compute unit, all resident at once, a multiple of 8
    grid[dev] = (nb >= 1 && cus >= 8) ? (cus & ~7) : 0;
    done[dev] = true;
  }
  return grid[dev];
}

void launch_gateup_half(const HalfArgs& s, hipStream_t st) {
  hipLaunchKernelGGL(k_gateup_half, dim3((unsigned)s.grid), dim3(kHThreads), sizeof(HalfLds),
                     st, s);
}

}  // namespace bitsmoe
