// FQCM importance and the width allocation under a bit budget.
//
// BitsMoE blog note, Methodology: the FQCM part (routed activation
// importance beta, the loss a^2 beta eps of a width, the gain of a wider
// code per stored bit) and "Usage" (the widths {0,1,2,3,4,6,8,16} chosen for
// all components together under a bit budget).
//
//  * k_fqcm_eps: one wave per column p_{e,k}: eps(0) = ||p||^2, eps(b) the
//    squared error of the format's quantizer at b = 1..8 (fp16 scale and
//    offset, float32 codes; p_hat = m + s q exact in float64) and of the
//    fp16 rounding at 16.  Float64 sums.
//  * k_fqcm_beta: beta_{e,k} = sum over the routed pairs of e, in pair
//    order, of g (z_k z_k), float64; thread (e, k).
//  * k_fqcm_choose: for a multiplier lam, each column takes the width that
//    minimises L(b) + lam (dout b), L(b) = ((a a) beta) eps(b) in float64
//    (ties to the narrower width); the widths are summed exactly.  The host
//    bisects lam over the ordered bit patterns of non-negative doubles for
//    the smallest lam whose total fits the budget (the Lagrangian relaxation
//    of the integer program: exact for the bits it uses).
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>
#include <math.h>
#include <string.h>

#include "bitsmoe.h"
#include "common.h"

#pragma clang fp contract(off)

namespace bitsmoe {
namespace {

constexpr int kNW = 8;  // widths 0, 1, 2, 3, 4, 6, 8, 16
__constant__ int kW[kNW] = {0, 1, 2, 3, 4, 6, 8, 16};
constexpr int kFqThreads = 256;
constexpr int kMaxIters = 80;  // counters: one per bisection step (64 suffice)

__device__ __forceinline__ float min_signed(float v, float o) {
  return (o < v || (o == v && signbit(o))) ? o : v;
}

__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

__device__ __forceinline__ float f16_round(float x) { return __half2float(__float2half_rn(x)); }

__global__ __launch_bounds__(kFqThreads) void k_fqcm_eps(const float* __restrict__ p, int ncol,
                                                         int dout, double* __restrict__ eps) {
  const int lane = (int)threadIdx.x & 63;
  const int c = (int)blockIdx.x * (kFqThreads / 64) + ((int)threadIdx.x >> 6);
  if (c >= ncol) return;
  const float* pc = p + (size_t)c * dout;
  float lo = INFINITY, hi = -INFINITY;
  double sq = 0.0, e16 = 0.0;
  for (int i = lane; i < dout; i += 64) {
    const float v = pc[i];
    lo = min_signed(lo, v);
    hi = fmaxf(hi, v);
    const double d = (double)v;
    sq += d * d;
    const double r = d - (double)f16_round(v);
    e16 += r * r;
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    lo = min_signed(lo, __shfl_xor(lo, o, 64));
    hi = fmaxf(hi, __shfl_xor(hi, o, 64));
  }
  sq = wave_sum_f64(sq);
  e16 = wave_sum_f64(e16);
  double out[kNW];
  out[0] = sq;
  out[7] = e16;
  const float mf = f16_round(lo);
#pragma unroll
  for (int wi = 1; wi < 7; ++wi) {
    const int b = kW[wi];
    const float L = (float)((1 << b) - 1);
    float s = f16_round((hi - lo) / L);
    if (s == 0.0f) s = 1.0f;  // scale rounded to zero: use 1
    double acc = 0.0;
    for (int i = lane; i < dout; i += 64) {
      const float v = pc[i];
      float q = rintf((v - mf) / s);
      q = q < 0.0f ? 0.0f : (q > L ? L : q);
      const double r = (double)v - ((double)mf + (double)s * (double)q);
      acc += r * r;
    }
    out[wi] = wave_sum_f64(acc);
  }
  if (lane < kNW) {
    double o = out[0];
#pragma unroll
    for (int wi = 1; wi < kNW; ++wi) o = lane == wi ? out[wi] : o;
    eps[(size_t)c * kNW + lane] = o;
  }
}

__global__ __launch_bounds__(kFqThreads) void k_fqcm_beta(const float* __restrict__ z,
                                                          int z_stride,
                                                          const int32_t* __restrict__ ids,
                                                          const float* __restrict__ g, int T,
                                                          int k, int E, int r,
                                                          double* __restrict__ beta) {
  const int e = (int)blockIdx.y;
  const int kk = (int)blockIdx.x * kFqThreads + (int)threadIdx.x;
  if (kk >= r) return;
  double acc = 0.0;
  for (int t = 0; t < T; ++t) {
    for (int j = 0; j < k; ++j) {
      if (ids[t * k + j] != e) continue;  // uniform across the work-group
      const double zv = (double)z[(size_t)t * z_stride + kk];
      acc += (double)g[t * k + j] * (zv * zv);
    }
  }
  beta[(size_t)e * r + kk] = acc;
}

__global__ __launch_bounds__(kFqThreads) void k_fqcm_choose(
    const float* __restrict__ a, const double* __restrict__ beta, const double* __restrict__ eps,
    int ncol, double dout, double lam, uint8_t* __restrict__ bits,
    unsigned long long* __restrict__ total) {
  __shared__ unsigned long long part[kFqThreads / 64];
  const int c = (int)blockIdx.x * kFqThreads + (int)threadIdx.x;
  unsigned long long w = 0;
  if (c < ncol) {
    const double av = (double)a[c];
    const double imp = (av * av) * beta[c];
    int best = 0;
    double bc = imp * eps[(size_t)c * kNW];  // width 0 costs no bits
#pragma unroll
    for (int wi = 1; wi < kNW; ++wi) {
      const double cost = imp * eps[(size_t)c * kNW + wi] + lam * (dout * (double)kW[wi]);
      if (cost < bc) {
        bc = cost;
        best = wi;
      }
    }
    w = (unsigned long long)kW[best];
    if (bits) bits[c] = (uint8_t)kW[best];
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) w += __shfl_xor(w, o, 64);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = w;
  __syncthreads();
  if (threadIdx.x == 0) {
    unsigned long long s = 0;
    for (int i = 0; i < kFqThreads / 64; ++i) s += part[i];
    atomicAdd(total, s);
  }
}

__global__ void k_fqcm_zero(unsigned long long* p, int n) {
  const int i = (int)(blockIdx.x * blockDim.x + threadIdx.x);
  if (i < n) p[i] = 0ull;
}

int hip_st(hipError_t err, const char* what) {
  if (err != hipSuccess) return fail(BITSMOE_EHIP, "%s: %s", what, hipGetErrorString(err));
  return BITSMOE_OK;
}

int fq_dims(int E, int r, int dout) {
  if (E <= 0 || r <= 0 || dout <= 0)
    return fail(BITSMOE_ESHAPE, "E=%d r=%d dout=%d must be positive", E, r, dout);
  if ((int64_t)E * r > (1ll << 30)) return fail(BITSMOE_ESHAPE, "E*r too large");
  return BITSMOE_OK;
}

bool al(const void* p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

}  // namespace
}  // namespace bitsmoe

using namespace bitsmoe;

extern "C" {

int bitsmoe_fqcm_distortion(const float* p, int E, int r, int dout, double* eps,
                            bitsmoe_stream_t stream) {
  int st = fq_dims(E, r, dout);
  if (st) return st;
  if (!p || !eps) return fail(BITSMOE_EINVAL, "null pointer argument");
  if (!al(p, 4) || !al(eps, 8)) return fail(BITSMOE_EINVAL, "misaligned p or eps");
  const int ncol = E * r;
  const int per = kFqThreads / 64;
  hipLaunchKernelGGL(k_fqcm_eps, dim3((unsigned)((ncol + per - 1) / per)), dim3(kFqThreads), 0,
                     (hipStream_t)stream, p, ncol, dout, eps);
  return hip_st(hipGetLastError(), "distortion launch");
}

int bitsmoe_fqcm_beta(const float* z, int z_stride, const int32_t* ids, const float* g, int T,
                      int k, int E, int r, double* beta, bitsmoe_stream_t stream) {
  int st = fq_dims(E, r, 1);
  if (st) return st;
  if (!z || !ids || !g || !beta) return fail(BITSMOE_EINVAL, "null pointer argument");
  if (T < 1 || k < 1) return fail(BITSMOE_EINVAL, "T=%d k=%d", T, k);
  if (z_stride < r) return fail(BITSMOE_ESHAPE, "z_stride=%d < r=%d", z_stride, r);
  if (E > 65535) return fail(BITSMOE_ESHAPE, "E=%d exceeds 65535", E);
  if (!al(z, 4) || !al(ids, 4) || !al(g, 4) || !al(beta, 8))
    return fail(BITSMOE_EINVAL, "misaligned pointer");
  hipLaunchKernelGGL(k_fqcm_beta, dim3((unsigned)((r + kFqThreads - 1) / kFqThreads), (unsigned)E),
                     dim3(kFqThreads), 0, (hipStream_t)stream, z, z_stride, ids, g, T, k, E, r,
                     beta);
  return hip_st(hipGetLastError(), "beta launch");
}

int bitsmoe_fqcm_allocate(const float* a, const double* beta, const double* eps, int E, int r,
                          int dout, uint64_t budget_bits, uint8_t* bits, double* lambda,
                          uint64_t* used_bits, void* ws, size_t ws_bytes,
                          bitsmoe_stream_t stream) {
  int st = fq_dims(E, r, dout);
  if (st) return st;
  if (!a || !beta || !eps || !bits || !ws) return fail(BITSMOE_EINVAL, "null pointer argument");
  if (!al(a, 4) || !al(beta, 8) || !al(eps, 8) || !al(ws, 8))
    return fail(BITSMOE_EINVAL, "misaligned pointer");
  if (ws_bytes < BITSMOE_FQCM_WS_BYTES)
    return fail(BITSMOE_ENOSPC, "ws_bytes=%zu < %d", ws_bytes, BITSMOE_FQCM_WS_BYTES);
  const hipStream_t s = (hipStream_t)stream;
  const int ncol = E * r;
  const unsigned grid = (unsigned)((ncol + kFqThreads - 1) / kFqThreads);
  unsigned long long* cnt = (unsigned long long*)ws;
  hipLaunchKernelGGL(k_fqcm_zero, dim3(1), dim3(128), 0, s, cnt, kMaxIters);
  if ((st = hip_st(hipGetLastError(), "counter fill"))) return st;
  int it = 0;
  // total bits of the allocation at lam (one counter per evaluation)
  auto total_at = [&](double lam, uint64_t* out) -> int {
    if (it >= kMaxIters) return fail(BITSMOE_EINVAL, "bisection did not converge");
    hipLaunchKernelGGL(k_fqcm_choose, dim3(grid), dim3(kFqThreads), 0, s, a, beta, eps, ncol,
                       (double)dout, lam, (uint8_t*)nullptr, cnt + it);
    int rc = hip_st(hipGetLastError(), "allocation launch");
    if (rc) return rc;
    unsigned long long v = 0;
    if ((rc = hip_st(hipMemcpyAsync(&v, cnt + it, 8, hipMemcpyDeviceToHost, s), "count copy")) ||
        (rc = hip_st(hipStreamSynchronize(s), "allocation")))
      return rc;
    ++it;
    *out = (uint64_t)v * (uint64_t)dout;
    return BITSMOE_OK;
  };
  uint64_t used = 0;
  double lam = 0.0;
  if ((st = total_at(0.0, &used))) return st;
  if (used > budget_bits) {
    // smallest lam (a non-negative double) whose total fits; +inf always fits
    uint64_t lo = 0, hi = 0x7FF0000000000000ull;
    while (hi - lo > 1) {
      const uint64_t mid = lo + (hi - lo) / 2;
      double lm;
      memcpy(&lm, &mid, 8);
      uint64_t u = 0;
      if ((st = total_at(lm, &u))) return st;
      if (u <= budget_bits)
        hi = mid;
      else
        lo = mid;
    }
    memcpy(&lam, &hi, 8);
  }
  hipLaunchKernelGGL(k_fqcm_choose, dim3(grid), dim3(kFqThreads), 0, s, a, beta, eps, ncol,
                     (double)dout, lam, bits, cnt + (kMaxIters - 1));
  if ((st = hip_st(hipGetLastError(), "allocation launch"))) return st;
  unsigned long long v = 0;
  if ((st = hip_st(hipMemcpyAsync(&v, cnt + (kMaxIters - 1), 8, hipMemcpyDeviceToHost, s),
                   "count copy")) ||
      (st = hip_st(hipStreamSynchronize(s), "allocation")))
    return st;
  if (lambda) *lambda = lam;
  if (used_bits) *used_bits = (uint64_t)v * (uint64_t)dout;
  return BITSMOE_OK;
}

}  // extern "C"
