// Lane-mask expert kernel: y_e = sum_k a_{e,k} z_k p_hat_{e,k} over the
// width-grouped bit planes, then h = SiLU(y_gate) * y_up.
//
// BitsMoE blog note, Methodology: "second split" (y is a sum over spectral
// components of magnitude * shared coordinate * quantized unit direction)
// and "execution" (same-width components packed together by bit plane).
//
// gfx950 mapping.  A wave owns one 64-row slab of one (token, slot,
// projection) and a contiguous run of that slab's plane masks.  Lane t is
// row t.  Each stored plane word pair is a 64-bit lane mask: for plane j of
// a column with coefficient c = a * z_k * s, the rows whose code has bit j
// set receive c, so the slab needs ONE masked v_add_f32 per (column, plane)
// -- the mask goes to EXEC from SGPRs (scalar loads), the coefficient is an
// SGPR operand, and plane j accumulates into its own register (the 2^j
// weights are applied once at the end).  The row-independent offset term
// sum_k a z m is a lane-parallel reduction; 16-bit columns use one FMA per
// element.  Column runs are split over waves and work-groups by mask count;
// partial slabs are combined in a fixed order by the last work-group to
// arrive (deterministic), which also applies SiLU * mul.
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include "device_common.h"
#include "format.h"
#include "kernels.h"

namespace bitsmoe {
namespace {

constexpr int kW = 4;  // waves per work-group

__device__ __forceinline__ float rl(float v, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

// acc[j] += c on the rows set in m[j], j < B.  EXEC is saved, replaced by
// saved & m[j] for each plane, and restored inside the same asm block, so the
// compiler never observes a modified EXEC.  The scalar ANDs write SCC, which
// is declared clobbered.
template <int B>
__device__ __forceinline__ void masked_adds(float (&acc)[8], const uint64_t (&m)[8], float c);

#define BM_PLANE(i) "s_and_b64 exec, %[sv], %[m" #i "]\n\tv_add_f32 %[a" #i "], %[c], %[a" #i "]\n\t"

template <>
__device__ __forceinline__ void masked_adds<1>(float (&acc)[8], const uint64_t (&m)[8], float c) {
  uint64_t sv;
  asm volatile("s_mov_b64 %[sv], exec\n\t" BM_PLANE(0) "s_mov_b64 exec, %[sv]"
               : [a0] "+v"(acc[0]), [sv] "=&s"(sv)
               : [m0] "s"(m[0]), [c] "s"(c)
               : "scc");
}
template <>
__device__ __forceinline__ void masked_adds<2>(float (&acc)[8], const uint64_t (&m)[8], float c) {
  uint64_t sv;
  asm volatile("s_mov_b64 %[sv], exec\n\t" BM_PLANE(0) BM_PLANE(1) "s_mov_b64 exec, %[sv]"
               : [a0] "+v"(acc[0]), [a1] "+v"(acc[1]), [sv] "=&s"(sv)
               : [m0] "s"(m[0]), [m1] "s"(m[1]), [c] "s"(c)
               : "scc");
}
template <>
__device__ __forceinline__ void masked_adds<3>(float (&acc)[8], const uint64_t (&m)[8], float c) {
  uint64_t sv;
  asm volatile("s_mov_b64 %[sv], exec\n\t" BM_PLANE(0) BM_PLANE(1) BM_PLANE(2)
               "s_mov_b64 exec, %[sv]"
               : [a0] "+v"(acc[0]), [a1] "+v"(acc[1]), [a2] "+v"(acc[2]), [sv] "=&s"(sv)
               : [m0] "s"(m[0]), [m1] "s"(m[1]), [m2] "s"(m[2]), [c] "s"(c)
               : "scc");
}
template <>
__device__ __forceinline__ void masked_adds<4>(float (&acc)[8], const uint64_t (&m)[8], float c) {
  uint64_t sv;
  asm volatile("s_mov_b64 %[sv], exec\n\t" BM_PLANE(0) BM_PLANE(1) BM_PLANE(2) BM_PLANE(3)
               "s_mov_b64 exec, %[sv]"
               : [a0] "+v"(acc[0]), [a1] "+v"(acc[1]), [a2] "+v"(acc[2]), [a3] "+v"(acc[3]),
                 [sv] "=&s"(sv)
               : [m0] "s"(m[0]), [m1] "s"(m[1]), [m2] "s"(m[2]), [m3] "s"(m[3]), [c] "s"(c)
               : "scc");
}
template <>
__device__ __forceinline__ void masked_adds<6>(float (&acc)[8], const uint64_t (&m)[8], float c) {
  uint64_t sv;
  asm volatile("s_mov_b64 %[sv], exec\n\t" BM_PLANE(0) BM_PLANE(1) BM_PLANE(2) BM_PLANE(3)
               BM_PLANE(4) BM_PLANE(5) "s_mov_b64 exec, %[sv]"
               : [a0] "+v"(acc[0]), [a1] "+v"(acc[1]), [a2] "+v"(acc[2]), [a3] "+v"(acc[3]),
                 [a4] "+v"(acc[4]), [a5] "+v"(acc[5]), [sv] "=&s"(sv)
               : [m0] "s"(m[0]), [m1] "s"(m[1]), [m2] "s"(m[2]), [m3] "s"(m[3]),
                 [m4] "s"(m[4]), [m5] "s"(m[5]), [c] "s"(c)
               : "scc");
}
template <>
__device__ __forceinline__ void masked_adds<8>(float (&acc)[8], const uint64_t (&m)[8], float c) {
  uint64_t sv;
  asm volatile("s_mov_b64 %[sv], exec\n\t" BM_PLANE(0) BM_PLANE(1) BM_PLANE(2) BM_PLANE(3)
               BM_PLANE(4) BM_PLANE(5) BM_PLANE(6) BM_PLANE(7) "s_mov_b64 exec, %[sv]"
               : [a0] "+v"(acc[0]), [a1] "+v"(acc[1]), [a2] "+v"(acc[2]), [a3] "+v"(acc[3]),
                 [a4] "+v"(acc[4]), [a5] "+v"(acc[5]), [a6] "+v"(acc[6]), [a7] "+v"(acc[7]),
                 [sv] "=&s"(sv)
               : [m0] "s"(m[0]), [m1] "s"(m[1]), [m2] "s"(m[2]), [m3] "s"(m[3]),
                 [m4] "s"(m[4]), [m5] "s"(m[5]), [m6] "s"(m[6]), [m7] "s"(m[7]), [c] "s"(c)
               : "scc");
}
#undef BM_PLANE

// Plane masks are read through the constant address space: the data never
// changes during the kernel, and uniform loads from it become scalar loads
// straight into SGPRs.
typedef const __attribute__((address_space(4))) uint64_t cmask_t;

struct Block {
  const uint16_t* kidx;
  const float* A;
  const __half* S;
  const __half* M;
  const uint64_t* planes;  // this slab's masks
  const __half* F;
  uint32_t dout_pad;
};

// Columns [c_lo, c_hi) of one width group; their masks start at mp.  Masks
// are fetched in batches of U columns (U * B <= 16 masks, 32 SGPRs) so that
// each scalar-load round trip feeds up to 16 masked adds.
template <int B>
__device__ __forceinline__ void run_group(float (&acc)[8], float& biasv, bool& good,
                                          const Block& k, int c_lo, int c_hi,
                                          const uint64_t* __restrict__ mp,
                                          const float* __restrict__ zrow, int r, int lane) {
  constexpr int U = 16 / B;
  for (int cb = c_lo; cb < c_hi; cb += kWave) {
    const int col = cb + lane;
    float coefv = 0.f;
    if (col < c_hi) {
      uint32_t kk = k.kidx[col];
      good &= kk < (uint32_t)r;
      kk = kk < (uint32_t)r ? kk : 0u;
      const float az = k.A[col] * zrow[kk];
      coefv = az * __half2float(k.S[col]);
      biasv += az * __half2float(k.M[col]);
    }
    const int nn = min(kWave, c_hi - cb);
    int ii = 0;
    for (; ii + U <= nn; ii += U) {
      cmask_t* cm = (cmask_t*)mp;
      uint64_t mb[U * B];
#pragma unroll
      for (int q = 0; q < U * B; ++q) mb[q] = cm[q];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        uint64_t m[8];
#pragma unroll
        for (int j = 0; j < B; ++j) m[j] = mb[u * B + j];
        masked_adds<B>(acc, m, rl(coefv, ii + u));
      }
      mp += U * B;
    }
    for (; ii < nn; ++ii) {
      cmask_t* cm = (cmask_t*)mp;
      uint64_t m[8];
#pragma unroll
      for (int j = 0; j < B; ++j) m[j] = cm[j];
      masked_adds<B>(acc, m, rl(coefv, ii));
      mp += B;
    }
  }
}

// Pulls this wave's mask run toward the L2 with wide vector loads issued at
// once (their values are not used), so that the scalar loads that follow
// mostly hit the cache instead of waiting on HBM one batch at a time.
__device__ __forceinline__ void prefetch_run(const uint64_t* p, uint32_t n_masks, int lane) {
  uint64_t x = 0;
  for (uint32_t i = lane; i < n_masks; i += kWave) x ^= p[i];  // exactly the run, no over-read
  asm volatile("" ::"v"(x));
}

__global__ __launch_bounds__(kW * kWave) void k_gateup_exec(GateUpArgs a) {
  int idx = blockIdx.x;
  const int part = idx % a.parts;
  idx /= a.parts;
  const int proj = idx & 1;
  idx >>= 1;
  const int slab = idx % a.n_slabs;
  const int pair = idx / a.n_slabs;
  // wave index is uniform across the wave; tell the compiler so that every
  // per-wave quantity (mask pointers, column ranges) lives in SGPRs
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & (kWave - 1);
  const int t = pair / a.ktop;
  const int e = a.ids[pair];
  const uint8_t* blob = proj ? a.blob_u : a.blob_g;
  const uint64_t bytes = proj ? a.bytes_u : a.bytes_g;
  const float* zrow = a.z + (size_t)t * 2 * a.r + (proj ? a.r : 0);

  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float biasv = 0.f, y16 = 0.f;
  bool good = true;
  DirRec d;
  const bool ok = load_dir(blob, bytes, e, a.E, a.dout, a.r, d);
  if (ok) {
    const uint8_t* blk = blob + d.block_offset;
    Block k;
    k.kidx = reinterpret_cast<const uint16_t*>(blk);
    k.A = reinterpret_cast<const float*>(blk + d.a_off);
    k.S = reinterpret_cast<const __half*>(blk + d.s_off);
    k.M = reinterpret_cast<const __half*>(blk + d.m_off);
    k.planes = reinterpret_cast<const uint64_t*>(blk + d.planes_off) +
               (size_t)slab * d.masks_per_slab;
    k.F = reinterpret_cast<const __half*>(blk + d.f16_off);
    k.dout_pad = (uint32_t)a.n_slabs * 64u;
    const int ns = a.parts * kW;
    const int sub = part * kW + wv;
    const uint32_t mps = d.masks_per_slab;
    const uint32_t m0 = (uint32_t)((uint64_t)mps * sub / ns);
    const uint32_t m1 = (uint32_t)((uint64_t)mps * (sub + 1) / ns);
    if (m1 > m0) prefetch_run(k.planes + m0, m1 - m0, lane);
    uint32_t gcol = 0, gmask = 0;
#pragma unroll
    for (int g = 0; g < kNumQGroups; ++g) {
      const int b = kGroupWidth[g];
      const int n = d.count[g];
      // columns whose first mask lies in [m0, m1)
      int lo = m0 > gmask ? (int)((m0 - gmask + b - 1) / b) : 0;
      int hi = m1 > gmask ? (int)((m1 - gmask + b - 1) / b) : 0;
      lo = min(lo, n);
      hi = min(hi, n);
      if (hi > lo) {
        const uint64_t* mp = k.planes + gmask + (uint32_t)lo * b;
        const int c_lo = (int)gcol + lo, c_hi = (int)gcol + hi;
        switch (b) {
          case 1: run_group<1>(acc, biasv, good, k, c_lo, c_hi, mp, zrow, a.r, lane); break;
          case 2: run_group<2>(acc, biasv, good, k, c_lo, c_hi, mp, zrow, a.r, lane); break;
          case 3: run_group<3>(acc, biasv, good, k, c_lo, c_hi, mp, zrow, a.r, lane); break;
          case 4: run_group<4>(acc, biasv, good, k, c_lo, c_hi, mp, zrow, a.r, lane); break;
          case 6: run_group<6>(acc, biasv, good, k, c_lo, c_hi, mp, zrow, a.r, lane); break;
          default: run_group<8>(acc, biasv, good, k, c_lo, c_hi, mp, zrow, a.r, lane); break;
        }
      }
      gcol += n;
      gmask += (uint32_t)n * b;
    }
    // 16-bit columns: one FMA per element, done by the last sub-part
    if (sub == ns - 1) {
      const int n_q = (int)d.n_q, n_nz = (int)d.n_nz;
      for (int cb = n_q; cb < n_nz; cb += kWave) {
        const int col = cb + lane;
        float azv = 0.f;
        if (col < n_nz) {
          uint32_t kk = k.kidx[col];
          good &= kk < (uint32_t)a.r;
          kk = kk < (uint32_t)a.r ? kk : 0u;
          azv = k.A[col] * zrow[kk];
        }
        const int nn = min(kWave, n_nz - cb);
        for (int ii = 0; ii < nn; ++ii) {
          const float c = rl(azv, ii);
          y16 += c * __half2float(k.F[(size_t)(cb + ii - n_q) * k.dout_pad + slab * 64 + lane]);
        }
      }
    }
  }
  float y = acc[7];
#pragma unroll
  for (int j = 6; j >= 0; --j) y = y * 2.0f + acc[j];
  y += wave_sum(biasv) + y16;
  const bool wave_ok = ok && __all(good);

  __shared__ float s_y[kW][kWave];
  __shared__ int s_ok[kW];
  s_y[wv][lane] = y;
  if (lane == 0) s_ok[wv] = wave_ok;
  __syncthreads();
  if (wv != 0) return;
  float v = s_y[0][lane];
  bool all_ok = s_ok[0];
#pragma unroll
  for (int w = 1; w < kW; ++w) {
    v += s_y[w][lane];
    all_ok = all_ok && s_ok[w];
  }
  const size_t unit = (size_t)pair * a.n_slabs + slab;
  a.part[((unit * 2 + proj) * a.parts + part) * kWave + lane] = all_ok ? v : __builtin_nanf("");
  __threadfence();  // publish the partial slab before arriving
  uint32_t old = 0;
  if (lane == 0) old = atomicAdd(&a.cnt[unit], 1u);
  old = __shfl(old, 0, kWave);
  if (old != (uint32_t)(2 * a.parts - 1)) return;
  __threadfence();  // last to arrive: see every partial
  float g = 0.f, u = 0.f;
  const float* pg = a.part + (unit * 2) * a.parts * kWave + lane;
  const float* pu = pg + (size_t)a.parts * kWave;
  for (int p = 0; p < a.parts; ++p) {
    g += pg[p * kWave];
    u += pu[p * kWave];
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
  long long parts = (1024 + units - 1) / units;
  p.parts = (int)(parts < 1 ? 1 : (parts > 8 ? 8 : parts));
  p.z_off = 0;
  p.part_off = align_up((size_t)T * 2 * r * sizeof(float), 256);
  p.cnt_off = align_up(p.part_off + (size_t)units * p.parts * 64 * sizeof(float), 256);
  p.total = align_up(p.cnt_off + (size_t)T * k * p.n_slabs * sizeof(uint32_t), 256);
  return p;
}

void launch_gateup_exec(const GateUpArgs& a, hipStream_t s) {
  const long long blocks = (long long)a.npairs * a.n_slabs * 2 * a.parts;
  hipLaunchKernelGGL(k_gateup_exec, dim3((unsigned)blocks), dim3(kW * kWave), 0, s, a);
}

}  // namespace bitsmoe
