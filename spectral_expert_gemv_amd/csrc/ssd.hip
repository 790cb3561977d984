// Shared-basis spectral decomposition (SSD) of one linear type on the GPU.
//
// BitsMoE blog note, Methodology, "first split" (the E expert matrices of a
// linear type stacked and decomposed once, so that all experts share the
// right singular basis Phi) and "second split" (the left factor P_e = U_e
// Sigma normalised per column: W_e = sum_k a_{e,k} p_{e,k} phi_k^T with unit
// p_{e,k}).  Stacking reading: W_cat = [W_1; ...; W_E] ((E dout) x din).
//
// Float64 throughout:
//  * k_ssd_gemm (Gram): G = W_cat^T W_cat (din x din), 64 x 64 tiles with
//    LDS staging; its eigenvectors are the right singular vectors of W_cat
//    and its eigenvalues the squared singular values;
//  * cyclic Jacobi with the round-robin (circle) ordering: in each of the
//    n - 1 rounds of a sweep the n / 2 disjoint pairs rotate at once
//    (angles from the round's start, then one pass that maps every 2 x 2
//    block of G by both of its pairs' rotations and rotates V's columns);
//    sweeps stop when the off-diagonal mass falls below (1e-15 ||G||)^2;
//  * rank the eigenvalues (descending, ties by index), Phi = the leading r
//    eigenvectors, each signed so that its largest-magnitude entry (first
//    such) is positive;
//  * k_ssd_gemm (projection): P = W_cat Phi ((E dout) x r); a_{e,k} = the
//    norm of column k of P_e, p_{e,k} = P_e[:, k] / a_{e,k} (a unit vector
//    e_0 when a = 0).
#include <hip/hip_runtime.h>
#include <math.h>
#include <string.h>

#include "bitsmoe.h"
#include "common.h"

#pragma clang fp contract(off)

namespace bitsmoe {
namespace {

constexpr int kTileM = 64, kTileN = 64, kTileK = 16;

// C (M x N, row-major, float64) = A (M x K) B (K x N).  A and B are read
// through accessors: the Gram reads A = W_cat^T (A[m][k] = W[k][m]) and
// B = W_cat; the projection reads A = W_cat and B = the selected
// eigenvectors (B[k][n] = V[k][order[n]]).
struct GemmArgs {
  const float* W;        // W_cat, rows x din (float32)
  const double* V;       // eigenvectors, din x din
  const int* order;      // eigenvalue rank -> column of V
  double* C;
  int M, N, K, ldw;      // ldw = din
  int mode;              // 0: Gram, 1: projection
};

__device__ __forceinline__ double ga(const GemmArgs& g, int m, int k) {
  return g.mode == 0 ? (double)g.W[(size_t)k * g.ldw + m] : (double)g.W[(size_t)m * g.ldw + k];
}
__device__ __forceinline__ double gb(const GemmArgs& g, int k, int n) {
  return g.mode == 0 ? (double)g.W[(size_t)k * g.ldw + n] : g.V[(size_t)k * g.ldw + g.order[n]];
}

__global__ __launch_bounds__(256) void k_ssd_gemm(GemmArgs g) {
  __shared__ double As[kTileK][kTileM + 1];
  __shared__ double Bs[kTileK][kTileN + 1];
  const int tm = (int)blockIdx.y * kTileM, tn = (int)blockIdx.x * kTileN;
  const int tx = (int)threadIdx.x & 15, ty = (int)threadIdx.x >> 4;  // 16 x 16 threads, 4 x 4 each
  double acc[4][4] = {};
  for (int k0 = 0; k0 < g.K; k0 += kTileK) {
    for (int i = (int)threadIdx.x; i < kTileK * kTileM; i += 256) {
      const int kk = i / kTileM, mm = i % kTileM;
      const int m = tm + mm, k = k0 + kk;
      As[kk][mm] = (m < g.M && k < g.K) ? ga(g, m, k) : 0.0;
      const int n = tn + mm;
      Bs[kk][mm] = (n < g.N && k < g.K) ? gb(g, k, n) : 0.0;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < kTileK; ++kk) {
      double av[4], bv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        av[i] = As[kk][ty * 4 + i];
        bv[i] = Bs[kk][tx * 4 + i];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] += av[i] * bv[j];
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int m = tm + ty * 4 + i, n = tn + tx * 4 + j;
      if (m < g.M && n < g.N) g.C[(size_t)m * g.N + n] = acc[i][j];
    }
}

__global__ void k_ssd_identity(double* V, int n) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < (size_t)n * n) V[i] = (i / n == i % n) ? 1.0 : 0.0;
}

// Pair i of round t of the circle ordering over n (even) indices.
__device__ __forceinline__ void round_pair(int n, int t, int i, int& p, int& q) {
  const int m = n - 1;
  if (i == 0) {
    p = t;
    q = m;
  } else {
    p = (t + i) % m;
    q = (t - i + m) % m;
  }
  if (p > q) {
    const int x = p;
    p = q;
    q = x;
  }
}

// Rotation of each pair of the round: cs[4 i ..] = p, q, c, s (indices as
// doubles).  Indices >= n0 (the padding index of an odd size) do not rotate.
__global__ void k_jacobi_angles(const double* G, int n, int n0, int t, double* cs) {
  const int i = (int)(blockIdx.x * blockDim.x + threadIdx.x);
  if (i >= n / 2) return;
  int p, q;
  round_pair(n, t, i, p, q);
  double c = 1.0, s = 0.0;
  if (q < n0) {
    const double gpq = G[(size_t)p * n0 + q];
    if (gpq != 0.0) {
      const double theta = (G[(size_t)q * n0 + q] - G[(size_t)p * n0 + p]) / (2.0 * gpq);
      const double tt = (theta >= 0.0 ? 1.0 : -1.0) / (fabs(theta) + sqrt(theta * theta + 1.0));
      c = 1.0 / sqrt(tt * tt + 1.0);
      s = tt * c;
    }
  }
  cs[4 * i] = p;
  cs[4 * i + 1] = q;
  cs[4 * i + 2] = c;
  cs[4 * i + 3] = s;
}

// One round's rotations in one pass (after k_jacobi_angles): thread
// (i, j) < npairs^2 maps the 2 x 2 block of G at rows {p_i, q_i} and columns
// {p_j, q_j} to J_i^T B J_j (the disjoint rotations of a round commute, so
// this equals all column rotations followed by all row rotations); the
// remaining n0 * npairs threads rotate columns p, q of one row of V.
__global__ void k_jacobi_round(double* G, double* V, int n0, int npairs, const double* cs) {
  const size_t id = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const size_t nb = (size_t)npairs * npairs;
  if (id < nb) {
    const int i = (int)(id / npairs), j = (int)(id % npairs);  // neighbours: consecutive j
    const int pi = (int)cs[4 * i], qi = (int)cs[4 * i + 1];
    const int pjx = (int)cs[4 * j], qjx = (int)cs[4 * j + 1];
    if (qi >= n0 || qjx >= n0) {
      // a padding index: rotate only the real side (its partner index has
      // c = 1, s = 0, so the block reduces to one row or column pair)
      if (qi < n0 && pjx < n0 && qjx >= n0) {
        const double ci = cs[4 * i + 2], si = cs[4 * i + 3];
        const double a = G[(size_t)pi * n0 + pjx], b = G[(size_t)qi * n0 + pjx];
        G[(size_t)pi * n0 + pjx] = ci * a - si * b;
        G[(size_t)qi * n0 + pjx] = si * a + ci * b;
      } else if (qjx < n0 && pi < n0 && qi >= n0) {
        const double cj = cs[4 * j + 2], sj = cs[4 * j + 3];
        const double a = G[(size_t)pi * n0 + pjx], b = G[(size_t)pi * n0 + qjx];
        G[(size_t)pi * n0 + pjx] = cj * a - sj * b;
        G[(size_t)pi * n0 + qjx] = sj * a + cj * b;
      }
      return;
    }
    const double ci = cs[4 * i + 2], si = cs[4 * i + 3];
    const double cj = cs[4 * j + 2], sj = cs[4 * j + 3];
    double* rp = G + (size_t)pi * n0;
    double* rq = G + (size_t)qi * n0;
    const double b00 = rp[pjx], b01 = rp[qjx], b10 = rq[pjx], b11 = rq[qjx];
    // columns: B J_j
    const double c00 = cj * b00 - sj * b01, c01 = sj * b00 + cj * b01;
    const double c10 = cj * b10 - sj * b11, c11 = sj * b10 + cj * b11;
    // rows: J_i^T (B J_j)
    rp[pjx] = ci * c00 - si * c10;
    rp[qjx] = ci * c01 - si * c11;
    rq[pjx] = si * c00 + ci * c10;
    rq[qjx] = si * c01 + ci * c11;
    return;
  }
  const size_t v = id - nb;
  if (v >= (size_t)n0 * npairs) return;
  const int row = (int)(v / npairs), i = (int)(v % npairs);
  const int p = (int)cs[4 * i], q = (int)cs[4 * i + 1];
  if (q >= n0) return;
  const double c = cs[4 * i + 2], s = cs[4 * i + 3];
  double* r = V + (size_t)row * n0;
  const double mp = r[p], mq = r[q];
  r[p] = c * mp - s * mq;
  r[q] = s * mp + c * mq;
}

// out[0] = off-diagonal sum of squares, out[1] = total sum of squares (one
// work-group).
__global__ __launch_bounds__(1024) void k_jacobi_norms(const double* G, int n, double* out) {
  __shared__ double so[1024], st[1024];
  double off = 0.0, tot = 0.0;
  for (size_t i = threadIdx.x; i < (size_t)n * n; i += 1024) {
    const double v = G[i] * G[i];
    tot += v;
    if (i / n != i % n) off += v;
  }
  so[threadIdx.x] = off;
  st[threadIdx.x] = tot;
  __syncthreads();
  for (int d = 512; d > 0; d >>= 1) {
    if ((int)threadIdx.x < d) {
      so[threadIdx.x] += so[threadIdx.x + d];
      st[threadIdx.x] += st[threadIdx.x + d];
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    out[0] = so[0];
    out[1] = st[0];
  }
}

// order[rank] = index, eigenvalues descending (ties by index); and the sign
// of each eigenvector column: +1 when its first largest-magnitude entry is
// positive.
__global__ void k_ssd_rank(const double* G, const double* V, int n, int* order, double* sgn) {
  const int i = (int)(blockIdx.x * blockDim.x + threadIdx.x);
  if (i >= n) return;
  const double li = G[(size_t)i * n + i];
  int rank = 0;
  for (int j = 0; j < n; ++j) {
    const double lj = G[(size_t)j * n + j];
    rank += (lj > li || (lj == li && j < i)) ? 1 : 0;
  }
  order[rank] = i;
  double best = -1.0, sv = 1.0;
  for (int j = 0; j < n; ++j) {
    const double v = V[(size_t)j * n + i];
    if (fabs(v) > best) {
      best = fabs(v);
      sv = v < 0.0 ? -1.0 : 1.0;
    }
  }
  sgn[i] = sv;
}

// phi[j][k] = sgn V[j][order[k]]; a, p from P (rows = E dout, r columns;
// P was formed from the unsigned eigenvectors).
__global__ void k_ssd_outputs(const double* V, const int* order, const double* sgn,
                              const double* P, int E, int dout, int din, int r, float* phi,
                              float* a, float* p) {
  const int k = (int)blockIdx.x;
  const int e = (int)blockIdx.y;
  const int col = order[k];
  const double sg = sgn[col];
  if (e == 0)
    for (int j = (int)threadIdx.x; j < din; j += (int)blockDim.x)
      phi[(size_t)j * r + k] = (float)(sg * V[(size_t)j * din + col]);
  __shared__ double red[256];
  double ss = 0.0;
  for (int i = (int)threadIdx.x; i < dout; i += (int)blockDim.x) {
    const double v = P[((size_t)e * dout + i) * r + k];
    ss += v * v;
  }
  red[threadIdx.x] = ss;
  __syncthreads();
  for (int d = 128; d > 0; d >>= 1) {
    if ((int)threadIdx.x < d) red[threadIdx.x] += red[threadIdx.x + d];
    __syncthreads();
  }
  const double nrm = sqrt(red[0]);
  if (threadIdx.x == 0) a[(size_t)e * r + k] = (float)nrm;
  for (int i = (int)threadIdx.x; i < dout; i += (int)blockDim.x) {
    const double v = P[((size_t)e * dout + i) * r + k];
    p[((size_t)e * r + k) * dout + i] =
        nrm > 0.0 ? (float)(sg * v / nrm) : (i == 0 ? 1.0f : 0.0f);
  }
}

// sigma^2 in rank order: out[k] = G[order[k]][order[k]], k < r.
__global__ void k_ssd_sigma(const double* G, const int* order, int n, int r, double* out) {
  const int k = (int)(blockIdx.x * blockDim.x + threadIdx.x);
  if (k < r) out[k] = G[(size_t)order[k] * n + order[k]];
}

struct SsdWs {
  size_t G, V, cs, nrm, order, sgn, P, total;
};
SsdWs ssd_ws(int E, int dout, int din, int r) {
  const uint64_t n = (uint64_t)din + (din & 1);
  auto al = [](uint64_t x) { return (x + 255) / 256 * 256; };
  SsdWs w;
  w.G = 0;
  w.V = al(8ull * din * din);
  w.cs = w.V + al(8ull * din * din);
  w.nrm = w.cs + al(8ull * 4 * (n / 2));
  w.order = w.nrm + 256;
  w.sgn = w.order + al(4ull * din);
  w.P = w.sgn + al(8ull * din);
  w.total = w.P + al(8ull * E * dout * r);
  return w;
}

int hip_ok(hipError_t err, const char* what) {
  if (err != hipSuccess) return fail(BITSMOE_EHIP, "%s: %s", what, hipGetErrorString(err));
  return BITSMOE_OK;
}

int ssd_dims(int E, int dout, int din, int r) {
  if (E <= 0 || dout <= 0 || din <= 0 || r <= 0)
    return fail(BITSMOE_ESHAPE, "E=%d dout=%d din=%d r=%d must be positive", E, dout, din, r);
  if (din > 8192) return fail(BITSMOE_ESHAPE, "din=%d exceeds 8192", din);
  if (r > din || (long long)r > (long long)E * dout)
    return fail(BITSMOE_ESHAPE, "r=%d exceeds min(din, E*dout)", r);
  if ((long long)E * dout > (1LL << 28) || E > 65535)
    return fail(BITSMOE_ESHAPE, "E*dout too large");
  return BITSMOE_OK;
}

}  // namespace
}  // namespace bitsmoe

using namespace bitsmoe;

extern "C" {

int bitsmoe_ssd_workspace_size(int E, int dout, int din, int r, size_t* bytes) {
  if (!bytes) return fail(BITSMOE_EINVAL, "bytes is null");
  const int st = ssd_dims(E, dout, din, r);
  if (st) return st;
  *bytes = ssd_ws(E, dout, din, r).total;
  return BITSMOE_OK;
}

int bitsmoe_ssd(const float* W, int E, int dout, int din, int r, float* phi, float* a, float* p,
                double* sigma2, int* sweeps, int max_sweeps, void* ws, size_t ws_bytes,
                bitsmoe_stream_t stream) {
  int st = ssd_dims(E, dout, din, r);
  if (st) return st;
  if (!W || !phi || !a || !p || !ws) return fail(BITSMOE_EINVAL, "null pointer argument");
  if (((uintptr_t)ws & 255u) || ((uintptr_t)W & 3u) || ((uintptr_t)phi & 3u) ||
      ((uintptr_t)a & 3u) || ((uintptr_t)p & 3u))
    return fail(BITSMOE_EINVAL, "misaligned pointer (ws: 256 bytes; others: 4)");
  if (max_sweeps < 1) return fail(BITSMOE_EINVAL, "max_sweeps=%d < 1", max_sweeps);
  const SsdWs w = ssd_ws(E, dout, din, r);
  if (ws_bytes < w.total) return fail(BITSMOE_ENOSPC, "ws_bytes=%zu < %zu", ws_bytes, w.total);
  const hipStream_t s = (hipStream_t)stream;
  uint8_t* w8 = (uint8_t*)ws;
  double* G = (double*)(w8 + w.G);
  double* V = (double*)(w8 + w.V);
  double* cs = (double*)(w8 + w.cs);
  double* nrm = (double*)(w8 + w.nrm);
  int* order = (int*)(w8 + w.order);
  double* sgn = (double*)(w8 + w.sgn);
  double* P = (double*)(w8 + w.P);
  const int rows = E * dout;
  // Gram matrix
  GemmArgs ga{W, nullptr, nullptr, G, din, din, rows, din, 0};
  hipLaunchKernelGGL(k_ssd_gemm, dim3((din + kTileN - 1) / kTileN, (din + kTileM - 1) / kTileM),
                     dim3(256), 0, s, ga);
  if ((st = hip_ok(hipGetLastError(), "Gram launch"))) return st;
  hipLaunchKernelGGL(k_ssd_identity, dim3((unsigned)(((size_t)din * din + 255) / 256)), dim3(256),
                     0, s, V, din);
  if ((st = hip_ok(hipGetLastError(), "identity launch"))) return st;
  // cyclic Jacobi, circle ordering over an even index count
  const int n = din + (din & 1), npairs = n / 2;
  const unsigned gp = (unsigned)((npairs + 255) / 256);
  const unsigned gr =
      (unsigned)((((size_t)npairs * npairs + (size_t)din * npairs) + 255) / 256);
  int sw = 0;
  for (; sw < max_sweeps; ++sw) {
    hipLaunchKernelGGL(k_jacobi_norms, dim3(1), dim3(1024), 0, s, G, din, nrm);
    double hn[2] = {0.0, 0.0};
    if ((st = hip_ok(hipGetLastError(), "norm launch")) ||
        (st = hip_ok(hipMemcpyAsync(hn, nrm, 16, hipMemcpyDeviceToHost, s), "norm copy")) ||
        (st = hip_ok(hipStreamSynchronize(s), "ssd")))
      return st;
    if (!(hn[0] > 1e-30 * hn[1])) break;  // off-diagonal below (1e-15 ||G||)^2
    for (int t = 0; t < n - 1; ++t) {
      hipLaunchKernelGGL(k_jacobi_angles, dim3(gp), dim3(256), 0, s, G, n, din, t, cs);
      hipLaunchKernelGGL(k_jacobi_round, dim3(gr), dim3(256), 0, s, G, V, din, npairs, cs);
    }
    if ((st = hip_ok(hipGetLastError(), "rotation launch"))) return st;
  }
  hipLaunchKernelGGL(k_ssd_rank, dim3((din + 255) / 256), dim3(256), 0, s, G, V, din, order, sgn);
  GemmArgs gb{W, V, order, P, rows, r, din, din, 1};
  hipLaunchKernelGGL(k_ssd_gemm, dim3((r + kTileN - 1) / kTileN, (rows + kTileM - 1) / kTileM),
                     dim3(256), 0, s, gb);
  hipLaunchKernelGGL(k_ssd_outputs, dim3((unsigned)r, (unsigned)E), dim3(256), 0, s, V, order, sgn,
                     P, E, dout, din, r, phi, a, p);
  if ((st = hip_ok(hipGetLastError(), "output launch"))) return st;
  if (sigma2) {
    // squared singular values, descending (the rotation buffer holds 2 n >= r
    // doubles and is free now)
    hipLaunchKernelGGL(k_ssd_sigma, dim3((r + 255) / 256), dim3(256), 0, s, G, order, din, r, cs);
    if ((st = hip_ok(hipGetLastError(), "sigma launch")) ||
        (st = hip_ok(hipMemcpyAsync(sigma2, cs, 8ull * r, hipMemcpyDeviceToHost, s),
                     "sigma copy")))
      return st;
  }
  if ((st = hip_ok(hipStreamSynchronize(s), "ssd"))) return st;
  if (sweeps) *sweeps = sw;
  return BITSMOE_OK;
}

}  // extern "C"
