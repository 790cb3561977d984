// Route grouping and the grouped gate/up expert kernel (token batches).
//
// BitsMoE blog note, Methodology: "first split" (z = Phi^T x is computed once
// per token and reused by every expert the token is routed to), "second
// split" (expert output = sum over components of magnitude * z_k * quantized
// unit direction) and "execution" (components of one width stored together,
// plane by plane).  Grouping the batch's (token, slot) pairs by expert
// extends the first split's reuse across tokens: an expert's planes are read
// from HBM and decoded once per batch instead of once per routed token.
//
// k_route_group (one work-group): counting sort of the T*k pairs by expert
// id -- LDS histogram, block scan, scatter -- into per-expert pair lists
// (groups in ascending expert id; the order of pairs inside a group does not
// affect any result).  Pairs whose id lies outside [0, E) get NaN rows.
//
// k_gateup_grouped: one 512-lane work-group per (group, 64-row slab, 32-row
// half), both projections (waves 0-3 gate, 4-7 up), placed XCD-aware like
// the one-launch kernel.  The slab's plane masks and metadata are staged in
// LDS once (column chunks if they do not fit); the group's pairs are then
// taken NT (up to 2) at a time: their z rows (from the projection launch) go to LDS,
// and each lane spreads a column's plane bits into byte codes once and adds
// coef_t * code for all NT tokens.  A transpose reduction per token, the 4
// waves of a projection through LDS, and SiLU * mul finish each pair.
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include "device_common.h"
#include "format.h"
#include "kernels.h"
#include "slab_common.h"

namespace bitsmoe {
namespace {

using namespace slab;

// ------------------------------------------------------------ route groups
constexpr int kRThreads = 1024;

__global__ __launch_bounds__(kRThreads) void k_route_group(const int32_t* __restrict__ ids,
                                                           int P, int E, int dout,
                                                           float* __restrict__ h,
                                                           RouteLists rl) {
  extern __shared__ uint32_t cnt[];  // E counters, then E cursors
  uint32_t* cur = cnt + E;
  __shared__ uint32_t part[kRThreads], dpart[kRThreads];
  const int tid = threadIdx.x;
  for (int i = tid; i < E; i += kRThreads) cnt[i] = 0;
  __syncthreads();
  for (int p = tid; p < P; p += kRThreads) {
    const int e = ids[p];
    if (e >= 0 && e < E) atomicAdd(&cnt[e], 1u);
  }
  __syncthreads();
  // block scan over E: each thread owns a contiguous run of counters
  const int per = (E + kRThreads - 1) / kRThreads;
  const int e0 = min(E, tid * per), e1 = min(E, e0 + per);
  uint32_t sum = 0, nd = 0;
  for (int e = e0; e < e1; ++e) {
    sum += cnt[e];
    nd += cnt[e] > 0 ? 1u : 0u;
  }
  part[tid] = sum;
  dpart[tid] = nd;
  __syncthreads();
  for (int d = 1; d < kRThreads; d <<= 1) {
    const uint32_t a = tid >= d ? part[tid - d] : 0u;
    const uint32_t b = tid >= d ? dpart[tid - d] : 0u;
    __syncthreads();
    part[tid] += a;
    dpart[tid] += b;
    __syncthreads();
  }
  uint32_t off = part[tid] - sum, g = dpart[tid] - nd;
  for (int e = e0; e < e1; ++e) {
    const uint32_t c = cnt[e];
    cur[e] = off;
    if (c > 0) {
      rl.gexp[g] = e;
      rl.goff[g] = (int)off;
      ++g;
    }
    off += c;
  }
  if (tid == kRThreads - 1) {
    const uint32_t ng = dpart[tid];
    rl.goff[ng] = (int)part[tid];
    rl.ngroups[0] = (int)ng;
  }
  __syncthreads();
  for (int p = tid; p < P; p += kRThreads) {
    const int e = ids[p];
    if (e >= 0 && e < E) {
      rl.pairs[atomicAdd(&cur[e], 1u)] = p;
    } else {
      for (int i = 0; i < dout; ++i) h[(size_t)p * dout + i] = __builtin_nanf("");
    }
  }
}

// ------------------------------------------------------- grouped gate/up
constexpr int kGWaves = 8;
constexpr int kGThreads = kGWaves * kWave;  // 512
constexpr int kGProj = 256;                 // lanes per projection
constexpr int kGPW = kGWaves / 2;           // waves per projection
constexpr int kGMaxM = 5120;                // u64 per projection per chunk
constexpr int kGMaxC = 2048;                // columns per projection per chunk
constexpr int kGZ = 8192;                   // z floats staged per token batch
constexpr int kGMaxNT = 2;

struct __align__(16) GroupLds {
  uint64_t M[2][kGMaxM + 2];
  float A[2][kGMaxC + 8];
  uint16_t K[2][kGMaxC + 16];
  uint16_t S[2][kGMaxC + 16];
  uint16_t Mo[2][kGMaxC + 16];
  float Z[kGZ];
  float red[2][kGPW][kGMaxNT][kSlabRows];
  float bias[2][kGPW][kGMaxNT];
  uint32_t ok[2][kGPW];
  int nch[2];
};

// One column of width b <= B over 32 rows for NT tokens: the codes are
// spread once and converted once; coef[t] * code is added for every token.
template <int B, int NT>
__device__ __forceinline__ void column32n(const uint32_t* words, int b, const float (&coef)[NT],
                                          float (&acc)[NT][kSlabRows]) {
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
    const float f[4] = {(float)(c & 0xFFu), (float)((c >> 8) & 0xFFu),
                        (float)((c >> 16) & 0xFFu), (float)(c >> 24)};
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[t][4 * i + r] = fmaf(coef[t], f[r], acc[t][4 * i + r]);
  }
}

template <int NT>
__global__ __launch_bounds__(kGThreads) void k_gateup_grouped(GroupArgs s) {
  extern __shared__ __align__(16) uint8_t lds_raw[];
  GroupLds& L = *reinterpret_cast<GroupLds*>(lds_raw);
  const GateUpArgs& a = s.g;
  const int lane = threadIdx.x & (kWave - 1);
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int pj = wv >= kGPW ? 1 : 0;  // waves 0-3 gate, 4-7 up
  const int lp = (int)threadIdx.x & (kGProj - 1);
  const int R = 2 * a.r;
  const uint32_t dout_pad = (uint32_t)a.n_slabs * 64u;

  // unit (group, slab, half); XCD q % 8 shared by both halves of a slab
  const int Q = s.gmax * a.n_slabs;
  const int b = blockIdx.x;
  const int j = b >> 3;
  const int q = 8 * (j >> 1) + (b & 7);
  if (q >= Q) return;
  const int hh = j & 1;
  const int gi = q % s.gmax, slab = q / s.gmax;
  if (gi >= s.rl.ngroups[0]) return;
  const int e = __builtin_amdgcn_readfirstlane(s.rl.gexp[gi]);
  const int p0 = __builtin_amdgcn_readfirstlane(s.rl.goff[gi]);
  const int p1 = __builtin_amdgcn_readfirstlane(s.rl.goff[gi + 1]);

  const uint8_t* blob = pj ? a.blob_u : a.blob_g;
  const Proj P = make_proj(blob, pj ? a.bytes_u : a.bytes_g, e, load_rec_s(blob, e, a.E),
                           load_hdr(blob), a);
  const HGeo Gm = hgeo(P);
  const uint32_t ncol = P.nq + P.n16;
  {
    int nc = 0;
    for (uint32_t c = 0; c < ncol; c = hchunk_end<kGMaxM, kGMaxC>(P, Gm, c)) ++nc;
    if (threadIdx.x == (unsigned)(pj * kGProj)) L.nch[pj] = nc;
  }
  __syncthreads();
  const int nch = max(L.nch[0], L.nch[1]);
  const Arena ar = {&L.M[pj][0], &L.K[pj][0], &L.A[pj][0], &L.S[pj][0], &L.Mo[pj][0]};
  const uint32_t* Mw = reinterpret_cast<const uint32_t*>(&L.M[pj][0]);
  const float* Asrc = &L.A[pj][0];

  for (int t0 = p0; t0 < p1; t0 += NT) {
    const int nt = min(NT, p1 - t0);
    float acc[NT][kSlabRows];
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int i = 0; i < kSlabRows; ++i) acc[t][i] = 0.f;
    float biasv[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) biasv[t] = 0.f;
    bool good = P.ok;
    // z rows of this batch's tokens: Z[t][0, 2r) -- 16-byte loads, all
    // issued before the first is used
    {
      const float4* zsrc[NT];
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const int pair = __builtin_amdgcn_readfirstlane(s.rl.pairs[t0 + (t < nt ? t : 0)]);
        zsrc[t] = reinterpret_cast<const float4*>(s.z + (size_t)(pair / a.ktop) * R);
      }
      constexpr int kPer = kGZ / 4 / kGThreads;  // float4 per lane at most
      const int n4 = R / 4;                     // float4 per token (R = 2r, r % 4 == 0)
      float4 v[kPer];
#pragma unroll
      for (int u = 0; u < kPer; ++u) {
        const int i = (int)threadIdx.x + kGThreads * u;
        const int t = i >= n4 ? 1 : 0;
        v[u] = (i < nt * n4 && t < NT) ? zsrc[t < NT ? t : 0][i - t * n4]
                                        : make_float4(0.f, 0.f, 0.f, 0.f);
      }
#pragma unroll
      for (int u = 0; u < kPer; ++u) {
        const int i = (int)threadIdx.x + kGThreads * u;
        if (i < nt * n4) reinterpret_cast<float4*>(L.Z)[i] = v[u];
      }
    }
    uint32_t c0 = 0;
    for (int ch = 0; ch < max(nch, 1); ++ch) {
      const uint32_t c1 = c0 < ncol ? hchunk_end<kGMaxM, kGMaxC>(P, Gm, c0) : c0;
      // the slab is staged once when it fits one chunk
      const bool restage = nch > 1 || t0 == p0;
      if (restage && c1 > c0) hstage_chunk(ar, P, c0, c1, slab, hh, dout_pad, lp, lane, kGProj);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      const uint32_t q0 = min(c0, P.nq), q1 = min(c1, P.nq);
      const uint32_t ma0 = ((uint32_t)slab * P.mps + hmask_of(Gm, q0)) & ~1u;
      const uint32_t mu =
          q1 > q0 ? hunits(ma0, (uint32_t)slab * P.mps + hmask_of(Gm, q1), 2) : 0u;
      const int n_items = (int)(c1 - c0);
      const int nqi = (int)(q1 - q0);
      const float* zrow = &L.Z[pj ? a.r : 0];
#pragma unroll 1
      for (int r0 = 0; r0 < n_items; r0 += kGProj) {
        const int it = r0 + (((r0 / kGProj) & 1) ? kGProj - 1 - lp : lp);
        const bool live = it < n_items;
        const uint32_t c = c0 + (uint32_t)(live ? it : 0);
        const uint32_t kk = live ? L.K[pj][c - (c0 & ~7u)] : 0u;
        good &= kk < (uint32_t)a.r;
        const uint32_t kc = kk < (uint32_t)a.r ? kk : 0u;
        const float av = live ? Asrc[c - (c0 & ~3u)] : 0.f;
        float az[NT];
#pragma unroll
        for (int t = 0; t < NT; ++t) az[t] = (live && t < nt) ? av * zrow[t * R + kc] : 0.f;
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
          const int bw = isq ? hwidth(grp) : 0;
          float coef[NT];
          uint32_t mi = 0;
          if (isq) {
            const uint32_t si = c - (q0 & ~7u);
            const float sv = __half2float(__ushort_as_half(L.S[pj][si]));
            const float mv = __half2float(__ushort_as_half(L.Mo[pj][si]));
#pragma unroll
            for (int t = 0; t < NT; ++t) {
              coef[t] = az[t] * sv;
              biasv[t] += az[t] * mv;
            }
            mi = (uint32_t)slab * P.mps + gm + (c - gc) * (uint32_t)bw - ma0;
          } else {
#pragma unroll
            for (int t = 0; t < NT; ++t) coef[t] = 0.f;
          }
          const uint32_t* wp = Mw + 2 * mi + hh;
          switch (hwave_bmax(bw)) {
            case 1: column32n<1, NT>(wp, bw, coef, acc); break;
            case 2: column32n<2, NT>(wp, bw, coef, acc); break;
            case 3: column32n<3, NT>(wp, bw, coef, acc); break;
            case 4: column32n<4, NT>(wp, bw, coef, acc); break;
            case 6: column32n<6, NT>(wp, bw, coef, acc); break;
            case 8: column32n<8, NT>(wp, bw, coef, acc); break;
            default: break;
          }
        }
        const bool isf = live && it >= nqi;
        if (__any(isf)) {
          const uint4* fv =
              reinterpret_cast<const uint4*>(&L.M[pj][2 * mu + 8 * (isf ? it - nqi : 0)]);
#pragma unroll
          for (int qq = 0; qq < 4; ++qq) {
            const uint4 v4 = fv[qq];
            const __half2* h2 = reinterpret_cast<const __half2*>(&v4);
#pragma unroll
            for (int u = 0; u < 4; ++u) {
              const float2 f2 = __half22float2(h2[u]);
#pragma unroll
              for (int t = 0; t < NT; ++t) {
                const float cf = isf ? az[t] : 0.f;
                acc[t][8 * qq + 2 * u] = fmaf(cf, f2.x, acc[t][8 * qq + 2 * u]);
                acc[t][8 * qq + 2 * u + 1] = fmaf(cf, f2.y, acc[t][8 * qq + 2 * u + 1]);
              }
            }
          }
        }
      }
      __syncthreads();  // arenas are restaged by the next chunk or batch
      c0 = c1;
    }
    // row sums of each token, SiLU * mul
    const int wp = wv & (kGPW - 1);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const float v = htranspose_sum(acc[t], lane);
      const float bw = wave_sum(biasv[t]);
      if (lane < kSlabRows) L.red[pj][wp][t][lane] = v;
      if (lane == 0) L.bias[pj][wp][t] = bw;
    }
    {
      const bool wok = __all(good);
      if (lane == 0) L.ok[pj][wp] = wok;
    }
    __syncthreads();
    if (wv == 0 && lane < kSlabRows) {
      bool ok = true;
#pragma unroll
      for (int w = 0; w < kGPW; ++w) ok = ok && L.ok[0][w] && L.ok[1][w];
      const int row = slab * 64 + hh * kSlabRows + lane;
      for (int t = 0; t < nt; ++t) {
        float gsum = 0.f, usum = 0.f;
#pragma unroll
        for (int w = 0; w < kGPW; ++w) {
          gsum += L.red[0][w][t][lane] + L.bias[0][w][t];
          usum += L.red[1][w][t][lane] + L.bias[1][w][t];
        }
        const int pair = s.rl.pairs[t0 + t];
        if (row < a.dout)
          a.h[(size_t)pair * a.dout + row] = ok ? silu_mul(gsum, usum) : __builtin_nanf("");
      }
    }
    __syncthreads();  // red, Z are reused by the next batch
  }
}

}  // namespace

size_t grouped_lds_bytes() { return sizeof(GroupLds); }

int grouped_tokens_per_batch(int r) {
  const int nt = kGZ / (2 * r);
  return nt >= kGMaxNT ? kGMaxNT : (nt >= 1 ? 1 : 0);
}

int launch_route_group(const int32_t* ids, int P, int E, int dout, float* h,
                       const RouteLists& rl, hipStream_t st) {
  hipLaunchKernelGGL(k_route_group, dim3(1), dim3(kRThreads), (size_t)2 * E * sizeof(uint32_t),
                     st, ids, P, E, dout, h, rl);
  return 0;
}

int launch_gateup_grouped(const GroupArgs& s, hipStream_t st) {
  static bool attr_done[64];
  int dev = 0;
  if (hipGetDevice(&dev) == hipSuccess && dev >= 0 && dev < 64 && !attr_done[dev]) {
    (void)hipFuncSetAttribute((const void*)k_gateup_grouped<1>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)sizeof(GroupLds));
    (void)hipFuncSetAttribute((const void*)k_gateup_grouped<2>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)sizeof(GroupLds));
    (void)hipGetLastError();
    attr_done[dev] = true;
  }
  // units rounded up so that both halves of every slab exist: 2 * 8 * ceil(Q / 8)
  const long long Q = (long long)s.gmax * s.g.n_slabs;
  const long long blocks = 16 * ((Q + 7) / 8);
  const dim3 grid((unsigned)blocks);
  switch (grouped_tokens_per_batch(s.g.r)) {
    case 2: hipLaunchKernelGGL(k_gateup_grouped<2>, grid, dim3(kGThreads), sizeof(GroupLds), st, s); break;
    case 1: hipLaunchKernelGGL(k_gateup_grouped<1>, grid, dim3(kGThreads), sizeof(GroupLds), st, s); break;
    default: return -1;
  }
  return 0;
}

}  // namespace bitsmoe
