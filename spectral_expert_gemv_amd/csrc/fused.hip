// One-launch gate/up decode step for small token counts.
//
// BitsMoE blog note, Methodology: "first split" (z = Phi^T x is computed
// once per token and shared by every routed expert), "second split" (each
// expert output is a sum over components of magnitude * z_k * quantized
// unit direction) and "execution" (same-width components stored together by
// bit plane).  h = SiLU(y_gate) * y_up.
//
// gfx950 mapping.  Every work-group plays two roles in one launch:
//  * producer: its waves compute a share of the 2r rows of z (one Phi^T row
//    of din fp16 per wave-row, v_dot2_f32_f16 + wave reduction) and publish
//    each value as a 64-bit word (float bits | epoch tag << 32) with one
//    agent-coherent store -- no fence is needed because a reader that sees
//    the tag sees the value in the same word;
//  * consumer: one 64-row slab of one (token, slot, projection) and a share
//    of its columns, lane = column.  Each lane loads its columns' plane masks
//    (coalesced), turns the 64 row bits of each plane into byte codes with
//    SWAR arithmetic, and only then waits for the z values its columns need;
//    coef * code is accumulated into 64 row registers.
// Row sums are reduced through LDS; the partial slabs of the groups that
// share a slab are combined in a fixed order by the last group to arrive
// (deterministic), which applies SiLU * mul.  The last group of the whole
// grid advances the epoch so that the next call's tags differ.
//
// All groups must be resident at once (a consumer waits for producers):
// the host launches this kernel only when the occupancy query says the grid
// fits, and every wait is bounded -- on time-out the affected rows become NaN
// and the kernel still exits.
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include "device_common.h"
#include "format.h"
#include "kernels.h"

namespace bitsmoe {
namespace {

constexpr int kFW = 4;                 // waves per work-group
constexpr int kFL = kFW * kWave;       // lanes (column slots) per work-group
constexpr int kFPitch = 33;            // LDS pitch (floats) for 32-row halves
constexpr int kFMaxCols = 2;           // columns a lane holds at once
constexpr int kFRowsPerWave = 2;       // z rows a wave loads before its expert work
constexpr uint32_t kSpinLimit = 1u << 20;
static_assert(kFRowsPerWave == 2, "the producer loop selects pv[0] or pv[1]");

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float dot8(uint4 a, uint4 b, float acc) {
  const half2_t* ha = reinterpret_cast<const half2_t*>(&a);
  const half2_t* hb = reinterpret_cast<const half2_t*>(&b);
#pragma unroll
  for (int i = 0; i < 4; ++i) acc = __builtin_amdgcn_fdot2(ha[i], hb[i], acc, false);
  return acc;
}

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

__device__ __forceinline__ void decode_any(int bmax, const uint64_t (&m)[8],
                                           uint32_t (&codes)[16]) {
  switch (bmax) {
    case 1: decode64<1>(m, codes); break;
    case 2: decode64<2>(m, codes); break;
    case 3: decode64<3>(m, codes); break;
    case 4: decode64<4>(m, codes); break;
    case 5:
    case 6: decode64<6>(m, codes); break;
    default: decode64<8>(m, codes); break;
  }
}

__device__ __forceinline__ int wave_max(int v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = max(v, __shfl_xor(v, off, kWave));
  return v;
}

// Waits for the tagged z value at p; returns it, or NaN after the bound.
__device__ __forceinline__ float wait_z(const uint64_t* p, uint32_t tag, bool active) {
  uint64_t w = active ? __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0;
  bool ready = !active || (uint32_t)(w >> 32) == tag;
  uint32_t spins = 0;
  while (!__all(ready) && spins < kSpinLimit) {
    __builtin_amdgcn_s_sleep(2);
    if (!ready) {
      w = __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      ready = (uint32_t)(w >> 32) == tag;
    }
    ++spins;
  }
  if (!active) return 0.f;
  return ready ? __uint_as_float((uint32_t)w) : __builtin_nanf("");
}

__global__ __launch_bounds__(kFL) void k_gateup_fused(FusedArgs f) {
  const GateUpArgs& a = f.g;
  int idx = blockIdx.x;
  const int part = idx % a.parts;
  idx /= a.parts;
  const int proj = idx & 1;
  idx >>= 1;
  const int slab = idx % a.n_slabs;
  const int pair = idx / a.n_slabs;
  const int slot = threadIdx.x;
  const int lane = threadIdx.x & (kWave - 1);
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int t = pair / a.ktop;
  const int R = 2 * a.r;

  // ---- epoch tag of this call (read before any arrival, see the end) ----
  const uint32_t tag =
      __hip_atomic_load(f.epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1u;

  // ---- producer: issue the Phi^T row loads of this wave's z rows ----
  const int gw = blockIdx.x * kFW + wv;
  const int nwaves = gridDim.x * kFW;
  uint4 pv[kFRowsPerWave][4];
  int zrow_n[kFRowsPerWave];
#pragma unroll
  for (int q = 0; q < kFRowsPerWave; ++q) {
    const int n = gw + q * nwaves;
    zrow_n[q] = n;
    if (n < R) {
      const uint4* prow = f.phi_t + (size_t)n * f.din8;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int i = lane + u * kWave;
        pv[q][u] = i < f.din8 ? prow[i] : make_uint4(0, 0, 0, 0);
      }
    }
  }

  // ---- consumer set-up: expert block of this (pair, projection) ----
  const int e = a.ids[pair];
  const uint8_t* blob = proj ? a.blob_u : a.blob_g;
  const uint64_t bytes = proj ? a.bytes_u : a.bytes_g;
  DirRec d;
  const bool ok = load_dir(blob, bytes, e, a.E, a.dout, a.r, d);

  // ---- producer: finish and publish the z rows (T tokens each); rows past
  // the first kFRowsPerWave of this wave are loaded and reduced in turn ----
  for (int q = 0; gw + q * nwaves < R; ++q) {
    const int n = gw + q * nwaves;
    const uint4* prow = f.phi_t + (size_t)n * f.din8;
    uint4 p0[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = lane + u * kWave;
      if (q < kFRowsPerWave) {
        p0[u] = q == 0 ? pv[0][u] : pv[kFRowsPerWave - 1][u];
      } else {
        p0[u] = i < f.din8 ? prow[i] : make_uint4(0, 0, 0, 0);
      }
    }
    for (int tt = 0; tt < f.T; ++tt) {
      const uint4* xt = f.x + (size_t)tt * f.din8;
      float acc = 0.f;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int i = lane + u * kWave;
        if (i < f.din8) acc = dot8(p0[u], xt[i], acc);
      }
      // rows longer than 2048 (din8 > 256): remaining chunks
      for (int i0 = 4 * kWave; i0 < f.din8; i0 += 4 * kWave) {
        uint4 pw[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int i = i0 + lane + u * kWave;
          pw[u] = i < f.din8 ? prow[i] : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int i = i0 + lane + u * kWave;
          if (i < f.din8) acc = dot8(pw[u], xt[i], acc);
        }
      }
      acc = wave_sum(acc);
      if (lane == 0) {
        const uint64_t w = ((uint64_t)tag << 32) | __float_as_uint(acc);
        __hip_atomic_store(&f.zt[(size_t)tt * R + n], w, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }

  // ---- consumer: columns of this part, lane = column ----
  float acc[64];
#pragma unroll
  for (int i = 0; i < 64; ++i) acc[i] = 0.f;
  float biasv = 0.f;
  bool good = true;
  const uint64_t* ztok = f.zt + (size_t)t * R + (proj ? a.r : 0);
  if (ok) {
    const uint8_t* blk = blob + d.block_offset;
    const uint16_t* kidx = reinterpret_cast<const uint16_t*>(blk);
    const float* A = reinterpret_cast<const float*>(blk + d.a_off);
    const __half* S = reinterpret_cast<const __half*>(blk + d.s_off);
    const __half* M = reinterpret_cast<const __half*>(blk + d.m_off);
    const uint64_t* planes =
        reinterpret_cast<const uint64_t*>(blk + d.planes_off) + (size_t)slab * d.masks_per_slab;
    const uint32_t dout_pad = (uint32_t)a.n_slabs * 64u;
    const __half* F = reinterpret_cast<const __half*>(blk + d.f16_off) + (size_t)slab * 64;
    // group boundaries (columns and masks) of the 1..8-bit groups
    uint32_t gcol[kNumQGroups + 1], gmask[kNumQGroups + 1];
    gcol[0] = 0;
    gmask[0] = 0;
#pragma unroll
    for (int g = 0; g < kNumQGroups; ++g) {
      gcol[g + 1] = gcol[g] + d.count[g];
      gmask[g + 1] = gmask[g] + (uint32_t)d.count[g] * kGroupWidth[g];
    }
    // columns whose first mask lies in this part's mask range
    const uint32_t mps = d.masks_per_slab;
    const uint32_t m0 = (uint32_t)((uint64_t)mps * part / a.parts);
    const uint32_t m1 = (uint32_t)((uint64_t)mps * (part + 1) / a.parts);
    // first column whose first mask index is >= mm (groups are in mask order)
    auto first_col = [&](uint32_t mm) -> int {
      int c = (int)gcol[kNumQGroups];
      bool found = false;
#pragma unroll
      for (int g = 0; g < kNumQGroups; ++g) {
        const uint32_t b = kGroupWidth[g];
        const uint32_t off = mm > gmask[g] ? (mm - gmask[g] + b - 1) / b : 0u;
        if (!found && off < d.count[g]) {
          c = (int)(gcol[g] + off);
          found = true;
        }
      }
      return c;
    };
    const int C0 = first_col(m0);
    const int C1 = m1 >= mps ? (int)d.n_q : first_col(m1);

    for (int cb = C0; cb < C1; cb += kFL * kFMaxCols) {
      uint64_t mk[kFMaxCols][8];
      int bw[kFMaxCols];
      int kcol[kFMaxCols];
      float as_[kFMaxCols], am_[kFMaxCols];
#pragma unroll
      for (int q = 0; q < kFMaxCols; ++q) {
        const int c = cb + q * kFL + slot;
        bw[q] = 0;
        kcol[q] = 0;
        as_[q] = 0.f;
        am_[q] = 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) mk[q][j] = 0;
        if (c < C1) {
          int g = 0;
#pragma unroll
          for (int gg = 1; gg < kNumQGroups; ++gg) g += (uint32_t)c >= gcol[gg] ? 1 : 0;
          const int b = kGroupWidth[g];
          bw[q] = b;
          const uint64_t* p = planes + gmask[g] + ((uint32_t)c - gcol[g]) * b;
#pragma unroll
          for (int j = 0; j < 8; ++j)
            if (j < b) mk[q][j] = p[j];
          uint32_t kk = kidx[c];
          good &= kk < (uint32_t)a.r;
          kcol[q] = kk < (uint32_t)a.r ? (int)kk : 0;
          const float av = A[c];
          as_[q] = av * __half2float(S[c]);
          am_[q] = av * __half2float(M[c]);
        }
      }
      uint32_t codes[kFMaxCols][16];
#pragma unroll
      for (int q = 0; q < kFMaxCols; ++q) {
        const int bmax = wave_max(bw[q]);
        if (bmax > 0) decode_any(bmax, mk[q], codes[q]);
      }
#pragma unroll
      for (int q = 0; q < kFMaxCols; ++q) {
        const bool active = bw[q] > 0;
        if (__any(active)) {
          const float zk = wait_z(ztok + kcol[q], tag, active);
          const float coef = as_[q] * zk;
          biasv += am_[q] * zk;
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const uint32_t qq = codes[q][i];
            acc[4 * i + 0] = fmaf(coef, (float)(qq & 0xFFu), acc[4 * i + 0]);
            acc[4 * i + 1] = fmaf(coef, (float)((qq >> 8) & 0xFFu), acc[4 * i + 1]);
            acc[4 * i + 2] = fmaf(coef, (float)((qq >> 16) & 0xFFu), acc[4 * i + 2]);
            acc[4 * i + 3] = fmaf(coef, (float)(qq >> 24), acc[4 * i + 3]);
          }
        }
      }
    }
    // 16-bit columns (fp16 values), spread over the parts by column index
    const int n_q = (int)d.n_q, n16 = (int)d.n_16;
    const int f_lo = n16 * part / a.parts, f_hi = n16 * (part + 1) / a.parts;
    const int n_it = (f_hi - f_lo + kFL - 1) / kFL;  // uniform trip count (waits are wave-wide)
    for (int it = 0; it < n_it; ++it) {
      const int fc = f_lo + it * kFL + slot;
      const bool active = fc < f_hi;
      const int c = active ? n_q + fc : n_q;
      uint32_t kk = active ? kidx[c] : 0u;
      good &= kk < (uint32_t)a.r;
      kk = kk < (uint32_t)a.r ? kk : 0u;
      const float av = active ? A[c] : 0.f;
      uint4 fv[8];
      const uint4* fp = reinterpret_cast<const uint4*>(F + (size_t)(active ? fc : 0) * dout_pad);
#pragma unroll
      for (int q = 0; q < 8; ++q) fv[q] = active ? fp[q] : make_uint4(0, 0, 0, 0);
      const float az = av * wait_z(ztok + kk, tag, active);
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const __half2* h2 = reinterpret_cast<const __half2*>(&fv[q]);
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
  __shared__ float s_red[kFW][kWave * kFPitch];
  __shared__ float s_wave[kFW][kWave];
  __shared__ float s_bias[kFW];
  __shared__ int s_ok[kFW];
  const float bias = wave_sum(biasv);
  const bool wave_ok = ok && __all(good);
  float row_sum = 0.f;
#pragma unroll
  for (int half = 0; half < 2; ++half) {
#pragma unroll
    for (int i = 0; i < 32; ++i) s_red[wv][lane * kFPitch + i] = acc[32 * half + i];
    __syncthreads();
    if ((lane >> 5) == half) {
      const int rr = lane & 31;
      float s = 0.f;
#pragma unroll 8
      for (int l = 0; l < kWave; ++l) s += s_red[wv][l * kFPitch + rr];
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
  for (int w = 1; w < kFW; ++w) {
    v += s_wave[w][lane];
    bsum += s_bias[w];
    all_ok = all_ok && s_ok[w];
  }
  v += bsum;
  const size_t unit = (size_t)pair * a.n_slabs + slab;
  __hip_atomic_store(&a.part[((unit * 2 + proj) * a.parts + part) * kWave + lane],
                     all_ok ? v : __builtin_nanf(""), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __builtin_amdgcn_s_waitcnt(0);
  uint32_t old = 0;
  if (lane == 0)
    old = __hip_atomic_fetch_add(&a.cnt[unit], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  old = __shfl(old, 0, kWave);
  if (old == (uint32_t)(2 * a.parts - 1)) {
    float g = 0.f, u = 0.f;
    float* pg = a.part + (unit * 2) * a.parts * kWave + lane;
    float* pu = pg + (size_t)a.parts * kWave;
    for (int p = 0; p < a.parts; ++p) {
      g += __hip_atomic_load(pg + p * kWave, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      u += __hip_atomic_load(pu + p * kWave, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    const int row = slab * 64 + lane;
    if (row < a.dout) a.h[(size_t)pair * a.dout + row] = silu_mul(g, u);
    if (lane == 0)
      __hip_atomic_store(&a.cnt[unit], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  // ---- grid arrival: the last group advances the epoch for the next call ----
  if (lane == 0) {
    __builtin_amdgcn_s_waitcnt(0);
    const uint32_t n =
        __hip_atomic_fetch_add(f.arrive, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (n == gridDim.x - 1) {
      __hip_atomic_store(f.arrive, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(f.epoch, tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

}  // namespace

int fused_capacity() {
  // work-groups of k_gateup_fused that can be resident at once on the current
  // device (0 if unknown); queried once per device
  static int cap[64];
  static bool done[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  if (!done[dev]) {
    int cus = 0, nb = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, k_gateup_fused, kFL, 0) != hipSuccess)
      return 0;
    cap[dev] = cus * nb;
    done[dev] = true;
  }
  return cap[dev];
}



void launch_gateup_fused(const FusedArgs& f, hipStream_t s) {
  const long long blocks = (long long)f.g.npairs * f.g.n_slabs * 2 * f.g.parts;
  hipLaunchKernelGGL(k_gateup_fused, dim3((unsigned)blocks), dim3(kFL), 0, s, f);
}

}  // namespace bitsmoe
