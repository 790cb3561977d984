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
//  * The integer program's own minimum (the widths of least total loss
//    within the budget) from there: with x the Lagrangian widths, every
//    allocation y within the budget has loss(y) >= D + R(y), where D is the
//    dual bound at lam and R(y) the sum of the reduced costs
//    r_c = (L_c(y_c) + lam dout w(y_c)) - (L_c(x_c) + lam dout w(x_c)) >= 0
//    of the columns it changes.  So an allocation better than one whose
//    loss exceeds D by a gap changes only columns to widths with r <= gap.
//    k_fqcm_cand lists the alternatives with r <= tau; the host solves the
//    budget exactly over the listed columns (a dynamic program over the
//    units they add or free, all other columns fixed at x) and, when the
//    best one's gap to D is <= tau, that allocation is the optimum; else
//    tau becomes that gap and the list is rebuilt (the next round always
//    closes).  tau starts at the largest value whose list stays short.
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>
#include <math.h>
#include <string.h>

#include <algorithm>
#include <vector>

#include "bitsmoe.h"
#include "common.h"

#pragma clang fp contract(off)

namespace bitsmoe {
namespace {

constexpr int kNW = 8;  // widths 0, 1, 2, 3, 4, 6, 8, 16
__constant__ int kW[kNW] = {0, 1, 2, 3, 4, 6, 8, 16};
constexpr int kWh[kNW] = {0, 1, 2, 3, 4, 6, 8, 16};  // the same, for host code
constexpr int kFqThreads = 256;
constexpr int kMaxIters = 80;  // counters: one per bisection step (64 suffice)
// workspace: the bisection counters, the candidate counter, then the
// candidate list and the staging of the changed widths
constexpr size_t kCandCountOff = 8 * kMaxIters;
constexpr size_t kCandOff = 1024;
constexpr uint64_t kCandCap = 65536;      // listed alternatives per round
constexpr uint64_t kCandTarget = 2048;    // list length the first tau aims at
constexpr size_t kStageOff = kCandOff + kCandCap * 16;
constexpr uint64_t kDpCellsMax = 1ull << 28;  // columns x unit states of the exact step
static_assert(kStageOff + kCandCap * 8 <= BITSMOE_FQCM_WS_BYTES, "FQCM workspace");

struct Cand {
  int32_t col;
  int16_t wi;     // width index of the alternative
  int16_t delta;  // its width minus the column's Lagrangian width
  double dL;      // its loss minus the Lagrangian width's loss
};
static_assert(sizeof(Cand) == 16, "Cand layout");

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

// Alternatives of reduced cost <= tau at multiplier lam (x = the widths in
// bits): counted in *count, the first cap written to out (any order).
__global__ __launch_bounds__(kFqThreads) void k_fqcm_cand(
    const float* __restrict__ a, const double* __restrict__ beta, const double* __restrict__ eps,
    int ncol, double dout, double lam, const uint8_t* __restrict__ bits, double tau,
    Cand* __restrict__ out, unsigned long long cap, unsigned long long* __restrict__ count) {
  const int c = (int)blockIdx.x * kFqThreads + (int)threadIdx.x;
  if (c >= ncol) return;
  const double av = (double)a[c];
  const double imp = (av * av) * beta[c];
  int ix = 0;
#pragma unroll
  for (int wi = 1; wi < kNW; ++wi)
    if (kW[wi] == (int)bits[c]) ix = wi;
  // the costs as k_fqcm_choose forms them
  auto cost = [&](int wi) {
    const double l = imp * eps[(size_t)c * kNW + wi];
    return wi == 0 ? l : l + lam * (dout * (double)kW[wi]);
  };
  const double cx = cost(ix), lx = imp * eps[(size_t)c * kNW + ix];
  for (int wi = 0; wi < kNW; ++wi) {
    if (wi == ix) continue;
    const double ci = cost(wi);
    // (a margin of 1e-12 of the costs, so rounding in r never drops one)
    if (!(ci - cx <= tau + 1e-12 * (fabs(ci) + fabs(cx)))) continue;
    const unsigned long long slot = atomicAdd(count, 1ull);
    if (slot < cap) {
      Cand v;
      v.col = c;
      v.wi = (int16_t)wi;
      v.delta = (int16_t)(kW[wi] - kW[ix]);
      v.dL = imp * eps[(size_t)c * kNW + wi] - lx;
      out[slot] = v;
    }
  }
}

// bits[col[i]] = w[i] for i < n (the changes of the exact step)
__global__ void k_fqcm_set(uint8_t* __restrict__ bits, const int32_t* __restrict__ cw, int n) {
  const int i = (int)(blockIdx.x * blockDim.x + threadIdx.x);
  if (i < n) bits[cw[2 * i]] = (uint8_t)cw[2 * i + 1];
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

// Exact budget step over the listed alternatives (sorted by column, then
// width index): the columns listed may take any listed width or keep x, the
// rest keep x; total units added <= room.  Minimises the sum of dL, summed
// in column order; ties go to the narrower width at each column and then to
// the fewest units.  Returns the chosen (column, width) changes and that sum.
int exact_step(const std::vector<Cand>& cand, int64_t room, std::vector<int32_t>& changes,
               double* best_sum, int64_t* units_added) {
  struct Alt {
    int wi, delta;
    double dL;
  };
  std::vector<std::vector<Alt>> cols;
  std::vector<int32_t> col_id;
  for (size_t i = 0; i < cand.size();) {
    size_t j = i;
    std::vector<Alt> alts;
    const int ix = [&] {  // the column's own (Lagrangian) width index
      const int wx = kWh[cand[i].wi] - cand[i].delta;
      for (int w = 0; w < kNW; ++w)
        if (kWh[w] == wx) return w;
      return 0;
    }();
    alts.push_back({ix, 0, 0.0});
    for (; j < cand.size() && cand[j].col == cand[i].col; ++j)
      alts.push_back({cand[j].wi, cand[j].delta, cand[j].dL});
    std::sort(alts.begin(), alts.end(), [](const Alt& p, const Alt& q) { return p.wi < q.wi; });
    cols.push_back(alts);
    col_id.push_back(cand[i].col);
    i = j;
  }
  const size_t C = cols.size();
  std::vector<int64_t> neg(C + 1, 0);  // neg[j]: the most units columns j.. can free
  std::vector<int> up(C, 0);            // the most units column j can add
  for (size_t j = C; j-- > 0;) {
    int m = 0;
    for (const Alt& al : cols[j]) {
      m = std::min(m, al.delta);
      up[j] = std::max(up[j], al.delta);
    }
    neg[j] = neg[j + 1] + m;
  }
  const int64_t lo = neg[0], hi = room - lo;  // state s (units added) in [lo, hi]
  const uint64_t S = (uint64_t)(hi - lo + 1);
  if (C > 0 && (uint64_t)C * S > kDpCellsMax)
    return fail(BITSMOE_ENOSPC, "exact allocation step: %zu columns x %llu unit states "
                "exceed %llu", C, (unsigned long long)S, (unsigned long long)kDpCellsMax);
  const double inf = HUGE_VAL;
  std::vector<double> cur(S, inf), nxt(S);
  std::vector<uint8_t> pick((size_t)C * S, 0);
  cur[(size_t)(0 - lo)] = 0.0;
  int64_t clo = 0;  // states reachable so far: [clo, chi]
  int64_t chi = 0;
  for (size_t j = 0; j < C; ++j) {
    const int64_t nlo = clo + (neg[j] - neg[j + 1]);
    const int64_t nhi = room - neg[j + 1];
    std::fill(nxt.begin(), nxt.end(), inf);
    uint8_t* pj = &pick[j * S];
    for (size_t k = 0; k < cols[j].size(); ++k) {  // narrower widths first: they keep ties
      const Alt& al = cols[j][k];
      for (int64_t s0 = clo; s0 <= chi; ++s0) {
        const double v0 = cur[(size_t)(s0 - lo)];
        if (v0 == inf) continue;
        const int64_t t = s0 + al.delta;
        if (t < nlo || t > nhi) continue;
        const double v = v0 + al.dL;
        if (v < nxt[(size_t)(t - lo)]) {
          nxt[(size_t)(t - lo)] = v;
          pj[t - lo] = (uint8_t)k;
        }
      }
    }
    std::swap(cur, nxt);
    clo = nlo;
    chi = std::min(nhi, chi + up[j]);
  }
  int64_t sb = 0;
  double vb = inf;
  for (int64_t s0 = clo; s0 <= std::min(chi, room); ++s0)  // ties: the fewest units
    if (cur[(size_t)(s0 - lo)] < vb) {
      vb = cur[(size_t)(s0 - lo)];
      sb = s0;
    }
  if (vb == inf) return fail(BITSMOE_EINVAL, "exact allocation step found no allocation");
  // read the choices back: (column, width) for every listed column
  changes.clear();
  int64_t t = sb;
  for (size_t j = C; j-- > 0;) {
    const Alt& al = cols[j][pick[j * S + (size_t)(t - lo)]];
    t -= al.delta;
    changes.push_back(col_id[j]);
    changes.push_back(kWh[al.wi]);
  }
  if (t != 0) return fail(BITSMOE_EINVAL, "exact allocation step: inconsistent choices");
  *best_sum = vb;
  *units_added = sb;
  return BITSMOE_OK;
}

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
                          uint64_t* used_bits, double* lp_gap, void* ws, size_t ws_bytes,
                          bitsmoe_stream_t stream) {
  int st = fq_dims(E, r, dout);
  if (st) return st;
  if (!a || !beta || !eps || !bits || !ws) return fail(BITSMOE_EINVAL, "null pointer argument");
  if (!al(a, 4) || !al(beta, 8) || !al(eps, 8) || !al(ws, 8))
    return fail(BITSMOE_EINVAL, "misaligned pointer");
  if (ws_bytes < BITSMOE_FQCM_WS_BYTES)
    return fail(BITSMOE_ENOSPC, "ws_bytes=%zu < %zu", ws_bytes, (size_t)BITSMOE_FQCM_WS_BYTES);
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
  // the integer program's minimum from the Lagrangian widths (see top)
  const uint64_t umax = budget_bits / (uint64_t)dout;
  const int64_t room = (int64_t)umax - (int64_t)v;  // units x leaves unused
  int64_t units = (int64_t)v;
  double gap = 0.0;
  if (lam > 0.0 && std::isfinite(lam) && room > 0) {
    unsigned long long* ccount = (unsigned long long*)((uint8_t*)ws + kCandCountOff);
    Cand* cbuf = (Cand*)((uint8_t*)ws + kCandOff);
    int32_t* stage = (int32_t*)((uint8_t*)ws + kStageOff);
    // alternatives with reduced cost <= tau (listed when list is true)
    auto list_at = [&](double tau, bool list, uint64_t* n) -> int {
      hipLaunchKernelGGL(k_fqcm_zero, dim3(1), dim3(64), 0, s, ccount, 1);
      hipLaunchKernelGGL(k_fqcm_cand, dim3(grid), dim3(kFqThreads), 0, s, a, beta, eps, ncol,
                         (double)dout, lam, bits, tau, cbuf,
                         list ? (unsigned long long)kCandCap : 0ull, ccount);
      int rc = hip_st(hipGetLastError(), "candidate launch");
      if (rc) return rc;
      unsigned long long cnt_h = 0;
      if ((rc = hip_st(hipMemcpyAsync(&cnt_h, ccount, 8, hipMemcpyDeviceToHost, s),
                       "count copy")) ||
          (rc = hip_st(hipStreamSynchronize(s), "candidates")))
        return rc;
      *n = cnt_h;
      return BITSMOE_OK;
    };
    // tau: the gap of x itself (lam dout room) when its list is short, else
    // the largest double whose list holds at most kCandTarget alternatives
    double tau = lam * ((double)dout * (double)room);
    uint64_t n = 0;
    if ((st = list_at(tau, false, &n))) return st;
    if (n > kCandTarget) {
      uint64_t lo = 0, hi;
      memcpy(&hi, &tau, 8);
      uint64_t nlo = 0;
      if ((st = list_at(0.0, false, &nlo))) return st;
      if (nlo > kCandTarget) {
        hi = 0;
      } else {
        while (hi - lo > 1) {
          const uint64_t mid = lo + (hi - lo) / 2;
          double tm;
          memcpy(&tm, &mid, 8);
          uint64_t nm = 0;
          if ((st = list_at(tm, false, &nm))) return st;
          if (nm <= kCandTarget)
            lo = mid;
          else
            hi = mid;
        }
        hi = lo;
      }
      memcpy(&tau, &hi, 8);
    }
    bool closed = false;
    std::vector<Cand> cand;
    std::vector<int32_t> changes;
    for (int round = 0; round < 3 && !closed; ++round) {
      if ((st = list_at(tau, true, &n))) return st;
      if (n > kCandCap)
        return fail(BITSMOE_ENOSPC, "exact allocation: %llu alternatives within the gap, "
                    "above the %llu listed per round", (unsigned long long)n,
                    (unsigned long long)kCandCap);
      cand.resize(n);
      if (n && ((st = hip_st(hipMemcpyAsync(cand.data(), cbuf, n * sizeof(Cand),
                                            hipMemcpyDeviceToHost, s), "candidate copy")) ||
                (st = hip_st(hipStreamSynchronize(s), "candidates"))))
        return st;
      std::sort(cand.begin(), cand.end(), [](const Cand& p, const Cand& q) {
        return p.col != q.col ? p.col < q.col : p.wi < q.wi;
      });
      double sum = 0.0;
      int64_t added = 0;
      if ((st = exact_step(cand, room, changes, &sum, &added))) return st;
      // the best allocation's distance to the dual bound
      gap = sum + lam * ((double)dout * (double)room);
      if (gap <= tau + 1e-12 * fabs(tau)) {
        closed = true;
        const int nch = (int)(changes.size() / 2);
        if (nch > 0) {
          if ((st = hip_st(hipMemcpyAsync(stage, changes.data(), changes.size() * 4,
                                          hipMemcpyHostToDevice, s), "change copy")))
            return st;
          hipLaunchKernelGGL(k_fqcm_set, dim3((unsigned)((nch + 255) / 256)), dim3(256), 0, s,
                             bits, stage, nch);
          if ((st = hip_st(hipGetLastError(), "change launch")) ||
              (st = hip_st(hipStreamSynchronize(s), "changes")))
            return st;
        }
        units = (int64_t)v + added;
      } else {
        tau = gap;
      }
    }
    if (!closed) return fail(BITSMOE_EINVAL, "exact allocation did not close");
  }
  if (lambda) *lambda = lam;
  if (used_bits) *used_bits = (uint64_t)units * (uint64_t)dout;
  if (lp_gap) *lp_gap = gap;
  return BITSMOE_OK;
}

}  // extern "C"
