// Gate/up expert kernel with LDS staging (z computed by a previous launch).
//
// BitsMoE blog note, Methodology: "first split" (z = Phi^T x once per token,
// shared by the routed experts), "second split" (expert output = sum over
// components of magnitude * z_k * quantized unit direction) and "execution"
// (components of one width stored together, by bit plane).
// h = SiLU(y_gate) * y_up.
//
// gfx950 mapping.  One work-group of 8 waves owns 32 rows (half of a 64-row
// slab) of one (token, slot): waves 0-3 the gate projection, waves 4-7 the
// up projection, 256 lanes each, so SiLU * mul needs no other group.
//  1. Staging: the slab's plane masks and the column metadata (k index, a,
//     s, m) are copied into LDS with 16-byte global_load_lds -- asynchronous,
//     no registers, one round trip.
//  2. z: each lane gathers z_k for its columns (all loads issued together)
//     and stores coef = a * s * z_k in LDS; the row-independent offset
//     sum a * m * z_k is reduced apart.
//  3. Columns are dealt to lanes; a lane reads its column's plane words from
//     LDS, spreads the 32 row bits of each plane into byte codes with SWAR
//     arithmetic (a 4-bit field times 0x00204081 puts bit n at bit 8n) and
//     adds coef * code to 32 row registers.  Row sums go through LDS.
// Columns are processed in chunks that fit the LDS budget.
//
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include "device_common.h"
#include "format.h"
#include "kernels.h"

namespace bitsmoe {
namespace {

constexpr int kSWaves = 8;
constexpr int kSThreads = kSWaves * kWave;  // 512
constexpr int kGL = 256;                    // lanes per projection group
constexpr int kRowsS = 32;
constexpr int kPitchS = kRowsS + 1;
constexpr int kMaxM = 6144;                 // staged plane masks (u64) per projection
constexpr int kMaxC = 2048;                 // staged columns per projection
constexpr int kZIt = kMaxC / kGL;           // z gathers per lane per chunk

typedef __attribute__((address_space(3))) void lds_void;

// LDS layout (dynamic), per projection:
//   masks u64[kMaxM + 2] | kidx u16[kMaxC + 16] | a f32[kMaxC + 8] (later coef)
//   | s u16[kMaxC + 16] | m u16[kMaxC + 16]
// Each array is staged from a 16-byte aligned source start, so it holds a
// few leading elements before the chunk's first one (the *0 offsets).
constexpr int kMaskCap = kMaxM + 2, kU16Cap = kMaxC + 16, kF32Cap = kMaxC + 8;
constexpr size_t kLdsProj =
    (size_t)kMaskCap * 8 + (size_t)kU16Cap * 2 * 3 + (size_t)kF32Cap * 4;
constexpr size_t kLdsBytes = 2 * kLdsProj;

struct Lds {
  uint64_t* masks;
  uint16_t* kidx;
  float* a;
  uint16_t* s;
  uint16_t* m;
};

__device__ __forceinline__ Lds lds_of(uint8_t* base, int p) {
  uint8_t* b = base + (size_t)p * kLdsProj;
  Lds l;
  l.masks = reinterpret_cast<uint64_t*>(b);
  b += (size_t)kMaskCap * 8;
  l.kidx = reinterpret_cast<uint16_t*>(b);
  b += (size_t)kU16Cap * 2;
  l.a = reinterpret_cast<float*>(b);
  b += (size_t)kF32Cap * 4;
  l.s = reinterpret_cast<uint16_t*>(b);
  b += (size_t)kU16Cap * 2;
  l.m = reinterpret_cast<uint16_t*>(b);
  return l;
}

// Asynchronous copy of n 16-byte units from a 16-byte aligned src to dst.
// Lanes of a wave write consecutive units, so the LDS base of each
// instruction (dst + 16 (i - lane)) is uniform across the wave.
__device__ __forceinline__ void stage16(void* dst, const void* src, int n, int lp, int lane) {
  const uint8_t* s = static_cast<const uint8_t*>(src);
  uint8_t* d = static_cast<uint8_t*>(dst);
  for (int i = lp; i < n; i += kGL)
    __builtin_amdgcn_global_load_lds(static_cast<const void*>(s + 16 * (size_t)i),
                                     (lds_void*)(d + 16 * (size_t)(i - lane)), 16, 0, 0);
}

// Widths of the 1..8-bit groups without a memory table (g in 0..5).
__device__ __forceinline__ int width_of(int g) { return g < 4 ? g + 1 : (g == 4 ? 6 : 8); }

// Largest width present in the wave (b in {0,1,2,3,4,6,8}), by ballots.
__device__ __forceinline__ int wave_bmax(int b) {
  if (__any(b > 6)) return 8;
  if (__any(b > 4)) return 6;
  if (__any(b > 3)) return 4;
  if (__any(b > 2)) return 3;
  if (__any(b > 1)) return 2;
  return __any(b > 0) ? 1 : 0;
}

// Reads B plane words (the 32-bit half hw of each mask) of a column of width
// b <= B from LDS, spreads them into 32 byte codes and adds coef * code.
template <int B>
__device__ __forceinline__ void column(const uint32_t* words, int b, float coef,
                                       float (&acc)[kRowsS]) {
  uint32_t w[B];
#pragma unroll
  for (int j = 0; j < B; ++j) {
    const uint32_t v = words[2 * (j < b ? j : (b > 0 ? b - 1 : 0))];
    w[j] = j < b ? v : 0u;
  }
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

__global__ __launch_bounds__(kSThreads) void k_gateup_staged(StagedArgs s) {
  extern __shared__ __align__(16) uint8_t lds_raw[];
  const GateUpArgs& a = s.g;
  const int n_half = 2 * a.n_slabs;
  const int hs = blockIdx.x % n_half;
  const int pair = blockIdx.x / n_half;
  const int slab = hs >> 1, hw = hs & 1;
  const int lane = threadIdx.x & (kWave - 1);
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int proj = wv >> 2;          // waves 0-3 gate, 4-7 up
  const int lp = threadIdx.x & (kGL - 1);
  const int t = pair / a.ktop;
  const int R = 2 * a.r;

  const int e = a.ids[pair];

  // ---- this projection's expert block ----
  const uint8_t* blob = proj ? a.blob_u : a.blob_g;
  const uint64_t bytes = proj ? a.bytes_u : a.bytes_g;
  DirRec d;
  const bool ok = load_dir(blob, bytes, e, a.E, a.dout, a.r, d);
  const uint8_t* blk = blob + d.block_offset;
  const uint16_t* g_kidx = reinterpret_cast<const uint16_t*>(blk);
  const float* g_a = reinterpret_cast<const float*>(blk + d.a_off);
  const uint16_t* g_s = reinterpret_cast<const uint16_t*>(blk + d.s_off);
  const uint16_t* g_m = reinterpret_cast<const uint16_t*>(blk + d.m_off);
  const uint64_t* g_masks = reinterpret_cast<const uint64_t*>(blk + d.planes_off);
  const uint32_t mps = ok ? d.masks_per_slab : 0u;
  const uint32_t slab_m = (uint32_t)slab * mps;  // first mask of this slab
  uint32_t gcol[kNumQGroups + 1], gmask[kNumQGroups + 1];
  gcol[0] = 0;
  gmask[0] = 0;
#pragma unroll
  for (int g = 0; g < kNumQGroups; ++g) {
    gcol[g + 1] = gcol[g] + (ok ? d.count[g] : 0u);
    gmask[g + 1] = gmask[g] + (ok ? (uint32_t)d.count[g] * width_of(g) : 0u);
  }
  const int n_q = ok ? (int)d.n_q : 0;
  const int n16 = ok ? (int)d.n_16 : 0;
  const float* z_tok = s.z + (size_t)t * R + (proj ? a.r : 0);
  const Lds L = lds_of(lds_raw, proj);
  auto mask_of = [&](int c) -> uint32_t {  // first mask of column c (uniform c)
    uint32_t m = gmask[kNumQGroups];
#pragma unroll
    for (int g = kNumQGroups - 1; g >= 0; --g)
      if ((uint32_t)c < gcol[g + 1]) m = gmask[g] + ((uint32_t)c - gcol[g]) * width_of(g);
    return m;
  };
  auto chunk_end = [&](int c0) -> int {
    int c1 = min(n_q, c0 + kMaxC);
    const uint32_t m0 = mask_of(c0);
    while (c1 > c0 && mask_of(c1) - m0 > (uint32_t)kMaxM - 2) c1 = c0 + (c1 - c0) / 2;
    return c1;
  };

  // ---- 16-bit columns: first batch of loads issued now, used at the end ----
  const uint32_t dout_pad = (uint32_t)a.n_slabs * 64u;
  const __half* F = reinterpret_cast<const __half*>(blk + d.f16_off) + (size_t)slab * 64 +
                    (size_t)hw * kRowsS;
  uint4 fv[4];
  float fa = 0.f;
  uint32_t fk = 0;
  auto f16_issue = [&](int it) {
    const int fc = it * kGL + lp;
    const bool live = fc < n16;
    const int c = n_q + (live ? fc : 0);
    fk = live ? g_kidx[c] : 0u;
    fa = live ? g_a[c] : 0.f;
    const uint4* fp = reinterpret_cast<const uint4*>(F + (size_t)(live ? fc : 0) * dout_pad);
#pragma unroll
    for (int q = 0; q < 4; ++q) fv[q] = live ? fp[q] : make_uint4(0, 0, 0, 0);
  };
  const int n_it16 = (n16 + kGL - 1) / kGL;
  if (n_it16 > 0) f16_issue(0);

  float acc[kRowsS];
#pragma unroll
  for (int i = 0; i < kRowsS; ++i) acc[i] = 0.f;
  float biasv = 0.f;
  bool good = true;

  // chunk counts; both projections run the larger count so barriers match
  int nchunks = 0;
  for (int c0 = 0; c0 < n_q; c0 = chunk_end(c0)) ++nchunks;
  __shared__ int s_nch[2];
  if (lp == 0) s_nch[proj] = nchunks;
  __syncthreads();
  const int nch_all = max(s_nch[0], s_nch[1]);

  int c0 = 0;
  for (int ch = 0; ch < nch_all; ++ch) {
    const int c1 = ch < nchunks ? chunk_end(c0) : c0;
    const int nc = c1 - c0;
    const uint32_t m_lo = mask_of(c0), m_hi = nc > 0 ? mask_of(c1) : m_lo;
    // 16-byte aligned starts: masks by 2, u16 arrays by 8, a by 4
    const uint32_t ma0 = (slab_m + m_lo) & ~1u;
    const int cu0 = c0 & ~7, cf0 = c0 & ~3;
    // ---- 1. stage plane masks and metadata ----
    if (nc > 0) {
      stage16(L.masks, g_masks + ma0, (int)((slab_m + m_hi - ma0 + 1) >> 1), lp, lane);
      const int nu = (c1 - cu0 + 7) >> 3, nf = (c1 - cf0 + 3) >> 2;
      stage16(L.kidx, g_kidx + cu0, nu, lp, lane);
      stage16(L.s, g_s + cu0, nu, lp, lane);
      stage16(L.m, g_m + cu0, nu, lp, lane);
      stage16(L.a, g_a + cf0, nf, lp, lane);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    // ---- 2. z gather (all loads first), coef = a * s * z_k into LDS ----
    const int n_it = (nc + kGL - 1) / kGL;
    {
      uint32_t kc[kZIt];
      float zf[kZIt];
#pragma unroll
      for (int it = 0; it < kZIt; ++it) {
        const int i = it * kGL + lp;
        const bool live = it < n_it && i < nc;
        const uint32_t kk = live ? L.kidx[c0 - cu0 + i] : 0u;
        good &= kk < (uint32_t)a.r;
        kc[it] = kk < (uint32_t)a.r ? kk : 0u;
        zf[it] = live ? z_tok[kc[it]] : 0.f;
      }
#pragma unroll
      for (int it = 0; it < kZIt; ++it) {
        if (it >= n_it) break;
        const int i = it * kGL + lp;
        const bool live = i < nc;
        const float z = zf[it];
        if (live) {
          const float az = L.a[c0 - cf0 + i] * z;
          L.a[c0 - cf0 + i] = az * __half2float(__ushort_as_half(L.s[c0 - cu0 + i]));
          biasv += az * __half2float(__ushort_as_half(L.m[c0 - cu0 + i]));
        }
      }
    }
    __syncthreads();
    // ---- 3. decode and accumulate, lane = column ----
    for (int it = 0; it < n_it; ++it) {
      const int i = it * kGL + lp;
      const int c = c0 + i;
      const bool live = i < nc;
      int g = 0;
#pragma unroll
      for (int gg = 1; gg < kNumQGroups; ++gg) g += (uint32_t)c >= gcol[gg] ? 1 : 0;
      const int b = live ? width_of(g) : 0;
      const int bmax = wave_bmax(b);
      if (bmax == 0) continue;
      uint32_t gc = gcol[0], gm = gmask[0];
#pragma unroll
      for (int gg = 1; gg < kNumQGroups; ++gg) {
        if (g == gg) {
          gc = gcol[gg];
          gm = gmask[gg];
        }
      }
      const uint32_t mi = live ? slab_m + gm + ((uint32_t)c - gc) * b - ma0 : 0u;
      const uint32_t* words = reinterpret_cast<const uint32_t*>(L.masks + mi) + hw;
      const float coef = live ? L.a[c0 - cf0 + i] : 0.f;
      switch (bmax) {
        case 1: column<1>(words, b, coef, acc); break;
        case 2: column<2>(words, b, coef, acc); break;
        case 3: column<3>(words, b, coef, acc); break;
        case 4: column<4>(words, b, coef, acc); break;
        case 6: column<6>(words, b, coef, acc); break;
        default: column<8>(words, b, coef, acc); break;
      }
    }
    __syncthreads();  // LDS is restaged by the next chunk
    c0 = c1;
  }

  // ---- 16-bit columns: fp16 values (loads issued at the start) ----
  for (int it = 0; it < n_it16; ++it) {
    if (it > 0) f16_issue(it);
    const bool live = it * kGL + lp < n16;
    good &= fk < (uint32_t)a.r;
    const uint32_t kc = fk < (uint32_t)a.r ? fk : 0u;
    const float z = live ? z_tok[kc] : 0.f;
    const float az = fa * z;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const __half2* h2 = reinterpret_cast<const __half2*>(&fv[q]);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float2 f2 = __half22float2(h2[u]);
        acc[8 * q + 2 * u] = fmaf(az, f2.x, acc[8 * q + 2 * u]);
        acc[8 * q + 2 * u + 1] = fmaf(az, f2.y, acc[8 * q + 2 * u + 1]);
      }
    }
  }

  // ---- row sums: per wave over its 64 lanes, then per projection ----
  float* red = reinterpret_cast<float*>(lds_raw);  // 8 x 64 x 33 floats
  __shared__ float s_rows[kSWaves][kRowsS];
  __shared__ float s_bias[kSWaves];
  __shared__ int s_ok[kSWaves];
#pragma unroll
  for (int i = 0; i < kRowsS; ++i) red[(wv * kWave + lane) * kPitchS + i] = acc[i];
  {
    const float bsum = wave_sum(biasv);
    const bool wok = ok && __all(good);
    if (lane == 0) {
      s_bias[wv] = bsum;
      s_ok[wv] = wok;
    }
  }
  __syncthreads();
  if (lane < kRowsS) {
    float v = 0.f;
#pragma unroll 8
    for (int l = 0; l < kWave; ++l) v += red[(wv * kWave + l) * kPitchS + lane];
    s_rows[wv][lane] = v;
  }
  __syncthreads();
  if (wv == 0 && lane < kRowsS) {
    float g = 0.f, u = 0.f;
    bool all_ok = true;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      g += s_rows[w][lane] + s_bias[w];
      u += s_rows[4 + w][lane] + s_bias[4 + w];
      all_ok = all_ok && s_ok[w] && s_ok[4 + w];
    }
    const int row = hs * kRowsS + lane;
    if (row < a.dout)
      a.h[(size_t)pair * a.dout + row] = all_ok ? silu_mul(g, u) : __builtin_nanf("");
  }
}

static_assert(kLdsBytes >= (size_t)kSThreads * kPitchS * 4, "reduction fits the staging area");

}  // namespace

size_t staged_lds_bytes() { return kLdsBytes; }

long long staged_blocks(int T, int k, int dout) {
  return (long long)T * k * 2 * ((dout + 63) / 64);
}

int launch_gateup_staged(const StagedArgs& s, hipStream_t st) {
  static bool attr_done[64];
  int dev = 0;
  if (hipGetDevice(&dev) == hipSuccess && dev >= 0 && dev < 64 && !attr_done[dev]) {
    // allow the dynamic LDS size (a no-op where it is already permitted)
    (void)hipFuncSetAttribute((const void*)k_gateup_staged,
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLdsBytes);
    (void)hipGetLastError();
    attr_done[dev] = true;
  }
  const long long blocks = staged_blocks(s.T, s.g.ktop, s.g.dout);
  hipLaunchKernelGGL(k_gateup_staged, dim3((unsigned)blocks), dim3(kSThreads), kLdsBytes, st, s);
  return 0;
}

}  // namespace bitsmoe
