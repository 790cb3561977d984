// Column-parallel expert kernel: y_e = sum_k a_{e,k} z_k p_hat_{e,k} over the
// width-grouped bit planes, then h = SiLU(y_gate) * y_up.
//
// BitsMoE blog note, Methodology: "second split" (the expert output is a sum
// over spectral components of magnitude * shared coordinate * quantized unit
// direction) and "execution" (components of one width stored together, by
// bit plane).
//
// gfx950 mapping.  A work-group owns one 64-row slab of one (token, slot,
// projection) and a share of its columns; each lane takes whole columns.  A
// lane reads its column's b plane masks for the slab (b * 8 contiguous bytes,
// so a wave's loads are fully coalesced), turns the 64-row bit planes into
// 64 byte codes with SWAR arithmetic (4-bit fields spread to bytes by one
// 24-bit multiply), and accumulates coef * code into 64 row registers, coef =
// a * z_k * s.  The offset term sum_k a z m does not depend on the row and is
// reduced once.  Row sums over the lanes go through LDS; partial slabs of the
// work-groups that share a slab are added in a fixed order by the last one to
// arrive (deterministic), which also applies SiLU * mul.
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include "device_common.h"
#include "format.h"
#include "kernels.h"

namespace bitsmoe {
namespace {

constexpr int kSW = 4;                 // waves per work-group
constexpr int kSLanes = kSW * kWave;   // column slots per work-group
constexpr int kPitch = 33;             // LDS row pitch (floats) for 32-row halves

struct Blk {
  const uint16_t* kidx;
  const float* A;
  const __half* S;
  const __half* M;
  const uint64_t* planes;  // this slab's masks
  const __half* F;         // this slab's first row of the 16-bit columns
  uint32_t dout_pad;
};

// 64 byte codes of one column from its B plane masks: codes[i] holds rows
// 4i..4i+3, one byte each.  A 4-bit field x of plane j spreads to the four
// bytes by x * 0x00204081 (bit n lands at bit 8n) and is ORed in at bit j.
template <int B>
__device__ __forceinline__ void decode64(const uint64_t (&m)[8], uint32_t (&codes)[16]) {
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    uint32_t c = 0;
#pragma unroll
    for (int j = 0; j < B; ++j) {
      const uint32_t w = (i < 8) ? (uint32_t)m[j] : (uint32_t)(m[j] >> 32);
      const uint32_t x = __builtin_amdgcn_ubfe(w, (4 * i) & 31, 4);
      c |= ((x * 0x00204081u) & 0x01010101u) << j;
    }
    codes[i] = c;
  }
}

template <int B>
__device__ __forceinline__ void load_masks(const uint64_t* p, uint64_t (&m)[8]) {
#pragma unroll
  for (int j = 0; j < B; ++j) m[j] = p[j];
}

template <int B>
__device__ __forceinline__ void run_cols(float (&acc)[64], float& biasv, bool& good,
                                         const Blk& k, int c_lo, int c_hi, uint32_t gmask,
                                         int gcol, const float* __restrict__ zrow, int r,
                                         int slot) {
  for (int c = c_lo + slot; c < c_hi; c += kSLanes) {
    uint64_t m[8];
    load_masks<B>(k.planes + gmask + (uint32_t)(c - gcol) * B, m);
    uint32_t kk = k.kidx[c];
    good &= kk < (uint32_t)r;
    kk = kk < (uint32_t)r ? kk : 0u;
    const float az = k.A[c] * zrow[kk];
    const float coef = az * __half2float(k.S[c]);
    biasv += az * __half2float(k.M[c]);
    uint32_t codes[16];
    decode64<B>(m, codes);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const uint32_t q = codes[i];
      acc[4 * i + 0] = fmaf(coef, (float)(q & 0xFFu), acc[4 * i + 0]);
      acc[4 * i + 1] = fmaf(coef, (float)((q >> 8) & 0xFFu), acc[4 * i + 1]);
      acc[4 * i + 2] = fmaf(coef, (float)((q >> 16) & 0xFFu), acc[4 * i + 2]);
      acc[4 * i + 3] = fmaf(coef, (float)(q >> 24), acc[4 * i + 3]);
    }
  }
}

__global__ __launch_bounds__(kSLanes) void k_gateup_swar(GateUpArgs a) {
  int idx = blockIdx.x;
  const int part = idx % a.parts;
  idx /= a.parts;
  const int proj = idx & 1;
  idx >>= 1;
  const int slab = idx % a.n_slabs;
  const int pair = idx / a.n_slabs;
  const int slot = threadIdx.x;
  const int lane = threadIdx.x & (kWave - 1);
  const int wv = threadIdx.x >> 6;
  const int t = pair / a.ktop;
  const int e = a.ids[pair];
  const uint8_t* blob = proj ? a.blob_u : a.blob_g;
  const uint64_t bytes = proj ? a.bytes_u : a.bytes_g;
  const float* zrow = a.z + (size_t)t * 2 * a.r + (proj ? a.r : 0);

  float acc[64];
#pragma unroll
  for (int i = 0; i < 64; ++i) acc[i] = 0.f;
  float biasv = 0.f;
  bool good = true;
  DirRec d;
  const bool ok = load_dir(blob, bytes, e, a.E, a.dout, a.r, d);
  if (ok) {
    const uint8_t* blk = blob + d.block_offset;
    Blk k;
    k.kidx = reinterpret_cast<const uint16_t*>(blk);
    k.A = reinterpret_cast<const float*>(blk + d.a_off);
    k.S = reinterpret_cast<const __half*>(blk + d.s_off);
    k.M = reinterpret_cast<const __half*>(blk + d.m_off);
    k.planes = reinterpret_cast<const uint64_t*>(blk + d.planes_off) +
               (size_t)slab * d.masks_per_slab;
    k.dout_pad = (uint32_t)a.n_slabs * 64u;
    k.F = reinterpret_cast<const __half*>(blk + d.f16_off) + (size_t)slab * 64;
    const uint32_t mps = d.masks_per_slab;
    const uint32_t m0 = (uint32_t)((uint64_t)mps * part / a.parts);
    const uint32_t m1 = (uint32_t)((uint64_t)mps * (part + 1) / a.parts);
    uint32_t gcol = 0, gmask = 0;
#pragma unroll
    for (int g = 0; g < kNumQGroups; ++g) {
      const int b = kGroupWidth[g];
      const int n = d.count[g];
      int lo = m0 > gmask ? (int)((m0 - gmask + b - 1) / b) : 0;
      int hi = m1 > gmask ? (int)((m1 - gmask + b - 1) / b) : 0;
      lo = min(lo, n);
      hi = min(hi, n);
      if (hi > lo) {
        const int c_lo = (int)gcol + lo, c_hi = (int)gcol + hi;
        switch (b) {
          case 1: run_cols<1>(acc, biasv, good, k, c_lo, c_hi, gmask, gcol, zrow, a.r, slot); break;
          case 2: run_cols<2>(acc, biasv, good, k, c_lo, c_hi, gmask, gcol, zrow, a.r, slot); break;
          case 3: run_cols<3>(acc, biasv, good, k, c_lo, c_hi, gmask, gcol, zrow, a.r, slot); break;
          case 4: run_cols<4>(acc, biasv, good, k, c_lo, c_hi, gmask, gcol, zrow, a.r, slot); break;
          case 6: run_cols<6>(acc, biasv, good, k, c_lo, c_hi, gmask, gcol, zrow, a.r, slot); break;
          default: run_cols<8>(acc, biasv, good, k, c_lo, c_hi, gmask, gcol, zrow, a.r, slot); break;
        }
      }
      gcol += n;
      gmask += (uint32_t)n * b;
    }
    // 16-bit columns (fp16 values), spread over the parts by column index
    const int n_q = (int)d.n_q, n16 = (int)d.n_16;
    const int f_lo = n16 * part / a.parts, f_hi = n16 * (part + 1) / a.parts;
    for (int f = f_lo + slot; f < f_hi; f += kSLanes) {
      const int c = n_q + f;
      uint32_t kk = k.kidx[c];
      good &= kk < (uint32_t)a.r;
      kk = kk < (uint32_t)a.r ? kk : 0u;
      const float az = k.A[c] * zrow[kk];
      const uint4* fv = reinterpret_cast<const uint4*>(k.F + (size_t)f * k.dout_pad);
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const uint4 v = fv[q];
        const __half2* h2 = reinterpret_cast<const __half2*>(&v);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const float2 f2 = __half22float2(h2[u]);
          acc[8 * q + 2 * u] = fmaf(az, f2.x, acc[8 * q + 2 * u]);
          acc[8 * q + 2 * u + 1] = fmaf(az, f2.y, acc[8 * q + 2 * u + 1]);
        }
      }
    }
  }

  // ---- reduce the 256 column slots to one value per row ----
  __shared__ float s_red[kSW][kWave * kPitch];
  __shared__ float s_wave[kSW][kWave];
  __shared__ float s_bias[kSW];
  __shared__ int s_ok[kSW];
  const float bias = wave_sum(biasv);
  const bool wave_ok = ok && __all(good);
  float row_sum = 0.f;
#pragma unroll
  for (int half = 0; half < 2; ++half) {
#pragma unroll
    for (int i = 0; i < 32; ++i) s_red[wv][lane * kPitch + i] = acc[32 * half + i];
    __syncthreads();
    // lanes 32*half .. 32*half+31 sum rows 32*half + (lane & 31) over the 64 slots
    if ((lane >> 5) == half) {
      const int rr = lane & 31;
      float s = 0.f;
#pragma unroll 8
      for (int l = 0; l < kWave; ++l) s += s_red[wv][l * kPitch + rr];
      row_sum = s;
    }
    __syncthreads();
  }
  s_wave[wv][lane] = row_sum;
  if (lane == 0) {
    s_bias[wv] = bias;
    s_ok[wv] = wave_ok;
  }
  __syncthreads();
  if (wv != 0) return;
  float v = s_wave[0][lane];
  float bsum = s_bias[0];
  bool all_ok = s_ok[0];
#pragma unroll
  for (int w = 1; w < kSW; ++w) {
    v += s_wave[w][lane];
    bsum += s_bias[w];
    all_ok = all_ok && s_ok[w];
  }
  v += bsum;
  const size_t unit = (size_t)pair * a.n_slabs + slab;
  // Cross-work-group combine without cache-wide fences: the partial slab is
  // written with agent-coherent stores and the arrival counter is bumped only
  // after those stores have completed (s_waitcnt 0); the last arriver reads
  // the partials with agent-coherent loads.  No L2 write-back or invalidate
  // is issued, so the fences' cost does not scale with the grid.
  __hip_atomic_store(&a.part[((unit * 2 + proj) * a.parts + part) * kWave + lane],
                     all_ok ? v : __builtin_nanf(""), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __builtin_amdgcn_s_waitcnt(0);
  uint32_t old = 0;
  if (lane == 0)
    old = __hip_atomic_fetch_add(&a.cnt[unit], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  old = __shfl(old, 0, kWave);
  if (old != (uint32_t)(2 * a.parts - 1)) return;
  float g = 0.f, u = 0.f;
  float* pg = a.part + (unit * 2) * a.parts * kWave + lane;
  float* pu = pg + (size_t)a.parts * kWave;
  for (int p = 0; p < a.parts; ++p) {
    g += __hip_atomic_load(pg + p * kWave, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    u += __hip_atomic_load(pu + p * kWave, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  const int row = slab * 64 + lane;
  if (row < a.dout) a.h[(size_t)pair * a.dout + row] = silu_mul(g, u);
  if (lane == 0) __hip_atomic_store(&a.cnt[unit], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace

GateUpPlan gateup_plan(int T, int k, int dout, int r) {
  GateUpPlan p;
  p.n_slabs = (dout + 63) / 64;
  const long long units = (long long)T * k * p.n_slabs * 2;
  long long parts = (768 + units - 1) / units;
  p.parts = (int)(parts < 1 ? 1 : (parts > 8 ? 8 : parts));
  p.z_off = 0;
  p.zt_off = align_up((size_t)T * 2 * r * sizeof(float), 256);
  p.sync_off = align_up(p.zt_off + (size_t)T * 2 * r * sizeof(uint64_t), 256);
  p.part_off = align_up(p.sync_off + 2 * sizeof(uint32_t), 256);
  p.cnt_off = align_up(p.part_off + (size_t)units * p.parts * 64 * sizeof(float), 256);
  p.total = align_up(p.cnt_off + (size_t)T * k * 2 * p.n_slabs * sizeof(uint32_t), 256);
  return p;
}

void launch_gateup_swar(const GateUpArgs& a, hipStream_t s) {
  const long long blocks = (long long)a.npairs * a.n_slabs * 2 * a.parts;
  hipLaunchKernelGGL(k_gateup_swar, dim3((unsigned)blocks), dim3(kSLanes), 0, s, a);
}

}  // namespace bitsmoe
