// Down projection and routing-weighted combine.
//
// The down projection restated with the two splits of the BitsMoE blog
// note's Methodology ("first split": a shared basis of the input space;
// "second split": quantized unit directions with magnitudes).  Its input is
// the gate/up output h, different for every (token, slot), so z =
// Phi_down^T h is formed per pair; the pages name only gate and up, and this
// is the plain extension of the same machinery.
//
//  1. k_h_to_f16: h (float32) -> fp16, the activation precision the
//     projection reads;
//  2. z = Phi_down^T h16 for the T*k pairs (the spectral projection kernel);
//  3. y = P_e diag(a_e) z per pair: the pairs are grouped by expert and
//     each tile of up to 16 pairs of one expert goes through the grouped MFMA
//     kernel in its one-projection mode (each pair is one B column with its
//     own z; the two wave halves take two 32-row segments); beyond the
//     grouped kernel's limits the per-pair apply kernel;
//  4. k_combine: out[t] = sum over slots j, in order, of g[t, j] y[t, j]
//     (float32); a pair whose id is outside [0, E) contributes nothing.
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include "bitsmoe.h"
#include "common.h"
#include "format.h"
#include "kernels.h"
#include "route.h"

namespace bitsmoe {
namespace {

// With a route job, the last work-group groups the pairs by expert
// (route.h) instead of converting.
__global__ __launch_bounds__(256) void k_h_to_f16(const float* __restrict__ h,
                                                  __half* __restrict__ h16, size_t n,
                                                  RouteJob rj) {
  __shared__ uint32_t cnt[2 * kRouteFuseMaxE];
  __shared__ uint32_t buf[256];
  const unsigned nconv = gridDim.x - (rj.ids ? 1u : 0u);
  if (blockIdx.x >= nconv) {
    route_lists<256>(rj, cnt, buf);
    return;
  }
  const size_t stride = (size_t)nconv * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
    h16[i] = __float2half_rn(h[i]);
}

__global__ __launch_bounds__(256) void k_combine(const float* __restrict__ y,
                                                 const int32_t* __restrict__ ids,
                                                 const float* __restrict__ g, int k, int E,
                                                 int din, float* __restrict__ out) {
  const int t = (int)blockIdx.y;
  const int i = (int)blockIdx.x * 256 + (int)threadIdx.x;
  if (i >= din) return;
  // the slots' ids, weights and y values loaded kCombineBatch at a time,
  // all before any is used, then summed in slot order
  constexpr int kCombineBatch = 16;
  float acc = 0.f;
  for (int j0 = 0; j0 < k; j0 += kCombineBatch) {
    int ev[kCombineBatch];
    float gv[kCombineBatch], yv[kCombineBatch];
#pragma unroll
    for (int u = 0; u < kCombineBatch; ++u) {
      const int j = j0 + u;
      ev[u] = -1;
      gv[u] = yv[u] = 0.f;
      if (j < k) {
        ev[u] = ids[t * k + j];
        gv[u] = g[t * k + j];
        yv[u] = y[((size_t)t * k + j) * din + i];
      }
    }
#pragma unroll
    for (int u = 0; u < kCombineBatch; ++u)
      if (ev[u] >= 0 && ev[u] < E) acc += gv[u] * yv[u];
  }
  out[(size_t)t * din + i] = acc;
}

struct DownWs {
  size_t h16, z, y, zpart, route, coef, total;
};
DownWs down_ws(int T, int k, int E, int dout, int din, int rd) {
  const uint64_t n = (uint64_t)T * k;
  auto al = [](uint64_t x) { return (size_t)((x + 255) / 256 * 256); };
  const uint64_t nzp = ((uint64_t)rd + kProjRowsPerBlock - 1) / kProjRowsPerBlock;
  DownWs w;
  w.h16 = 0;
  w.z = al(n * dout * 2);
  w.y = w.z + al(n * rd * 4);
  w.zpart = w.y + al(n * din * 4);
  w.route = w.zpart + al(n * nzp * 4);
  w.coef = w.route + al(route_ints(tile_cap(T, k, E), (size_t)n) * 4);
  w.total = w.coef + group_coef_bytes(tile_cap(T, k, E), rd);
  return w;
}

int down_dims(int T, int k, int E, int dout, int din, int rd) {
  if (T < 1 || k < 1 || k > E) return fail(BITSMOE_EINVAL, "T=%d k=%d E=%d", T, k, E);
  if (E <= 0 || dout <= 0 || din <= 0 || rd <= 0)
    return fail(BITSMOE_ESHAPE, "E=%d dout=%d din=%d r_d=%d", E, dout, din, rd);
  if (dout % 8) return fail(BITSMOE_ESHAPE, "dout=%d is not a multiple of 8", dout);
  if ((long long)T * k > (1LL << 24) || T > 65535)
    return fail(BITSMOE_ESHAPE, "T=%d k=%d too large", T, k);
  return BITSMOE_OK;
}

}  // namespace
}  // namespace bitsmoe

using namespace bitsmoe;

extern "C" {

int bitsmoe_moe_down_workspace_size(int T, int k, int E, int dout, int din, int r_d,
                                    size_t* bytes) {
  if (!bytes) return fail(BITSMOE_EINVAL, "bytes is null");
  const int st = down_dims(T, k, E, dout, din, r_d);
  if (st) return st;
  *bytes = down_ws(T, k, E, dout, din, r_d).total;
  return BITSMOE_OK;
}

int bitsmoe_moe_down(const void* packed_down, size_t down_bytes, const void* phi_t_down_f16,
                     const float* h, const int32_t* ids, const float* g, int T, int k, int E,
                     int dout, int din, int r_d, float* out, void* ws, size_t ws_bytes,
                     bitsmoe_stream_t stream) {
  int st = down_dims(T, k, E, dout, din, r_d);
  if (st) return st;
  if (!packed_down || !phi_t_down_f16 || !h || !ids || !g || !out || !ws)
    return fail(BITSMOE_EINVAL, "null pointer argument");
  if (((uintptr_t)ws & 255u) || ((uintptr_t)h & 3u) || ((uintptr_t)g & 3u) ||
      ((uintptr_t)ids & 3u) || ((uintptr_t)out & 3u))
    return fail(BITSMOE_EINVAL, "misaligned pointer (ws: 256 bytes; h, g, ids, out: 4)");
  const DownWs w = down_ws(T, k, E, dout, din, r_d);
  if (ws_bytes < w.total) return fail(BITSMOE_ENOSPC, "ws_bytes=%zu < %zu", ws_bytes, w.total);
  const hipStream_t s = (hipStream_t)stream;
  uint8_t* w8 = (uint8_t*)ws;
  const size_t n = (size_t)T * k * dout;
  float* z = (float*)(w8 + w.z);
  float* y = (float*)(w8 + w.y);
  const bool grouped = r_d <= kGroupMaxR && E <= kGroupMaxE && dout <= kGroupMaxDin;
  if (grouped && (((uintptr_t)packed_down & 15u) || ((uintptr_t)phi_t_down_f16 & 15u)))
    return fail(BITSMOE_EINVAL, "packed_down and phi_t_down_f16 must be 16-byte aligned");
  if (grouped && down_bytes < kHeaderBytes + (size_t)kDirRecBytes * E)
    return fail(BITSMOE_ENOSPC, "packed_down: %zu bytes cannot hold header and directory",
                down_bytes);
  // the grouped path's pair lists: grouped in the cast launch when E is small
  GroupArgs gs;
  RouteJob rj{};
  float* const zpart = (float*)(w8 + w.zpart);
  if (grouped) {
    gs.g.blob_g = gs.g.blob_u = (const uint8_t*)packed_down;
    gs.g.bytes_g = gs.g.bytes_u = (uint64_t)down_bytes;
    gs.g.E = E;
    gs.g.dout = din;
    gs.g.r = r_d;
    gs.g.ids = ids;
    gs.g.ktop = k;
    gs.g.npairs = T * k;
    gs.g.h = y;
    gs.g.n_seg = (din + kSegRows - 1) / kSegRows;
    gs.z = z;
    gs.zpart = zpart;
    gs.nzp = (r_d + kProjRowsPerBlock - 1) / kProjRowsPerBlock;
    gs.tcap = tile_cap(T, k, E);
    gs.single = 1;
    route_lists_at(gs.rl, (int*)(w8 + w.route), gs.tcap, (size_t)T * k);
    group_coef_tables(gs, w8 + w.coef, r_d);
    if (E <= kRouteFuseMaxE) rj = RouteJob{ids, T * k, E, din, y, gs.rl, gs.tbad, gs.tcap * 2};
  }
  // few pairs: the row projection reads float32 h itself (rounding to fp16
  // as it stages), so no cast launch
  const bool direct = grouped && !((long long)T * k >= 16 && dout % 32 == 0) && dout <= 4096 &&
                      ((uintptr_t)h & 15u) == 0;
  hipError_t err = hipSuccess;
  if (!direct) {
    size_t blocks = (n + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL(k_h_to_f16, dim3((unsigned)blocks + (rj.ids ? 1u : 0u)), dim3(256), 0, s,
                       h, (__half*)(w8 + w.h16), n, rj);
    err = hipGetLastError();
    if (err != hipSuccess)
      return fail(BITSMOE_EHIP, "fp16 cast launch: %s", hipGetErrorString(err));
  }
  if (!grouped) {
    if ((st = bitsmoe_spectral_proj(phi_t_down_f16, w8 + w.h16, z, T * k, dout, r_d, stream)))
      return st;
    if ((st = bitsmoe_expert_apply(packed_down, down_bytes, E, din, r_d, z, r_d, ids, T * k, 1,
                                   y, nullptr, 0, stream)))
      return st;
  } else {
    // z and, per 16-row block of the projection, the largest |z| the grouped
    // kernel scales its coefficients by
    bool routed = rj.ids != nullptr;  // done by the cast launch
    if (direct) {
      const RouteJob rjd{ids, T * k, E, din, y, gs.rl, gs.tbad, gs.tcap * 2};
      if ((st = launch_proj_maxima(phi_t_down_f16, h, z, zpart, T * k, dout, r_d, s, &rjd,
                                   &routed, true)))
        return st;
    } else if ((st = launch_proj_maxima(phi_t_down_f16, w8 + w.h16, z, zpart, T * k, dout, r_d,
                                        s))) {
      return st;
    }
    if (!routed) {
      launch_route_group(ids, T * k, E, din, y, gs.rl, s, gs.tbad, gs.tcap * 2);
      err = hipGetLastError();
      if (err != hipSuccess)
        return fail(BITSMOE_EHIP, "route grouping launch: %s", hipGetErrorString(err));
    }
    launch_group_coef(gs, s);
    err = hipGetLastError();
    if (err != hipSuccess)
      return fail(BITSMOE_EHIP, "tile coefficient launch: %s", hipGetErrorString(err));
    launch_gateup_grouped(gs, s);
    err = hipGetLastError();
    if (err != hipSuccess)
      return fail(BITSMOE_EHIP, "grouped apply launch: %s", hipGetErrorString(err));
  }
  hipLaunchKernelGGL(k_combine, dim3((unsigned)((din + 255) / 256), (unsigned)T), dim3(256), 0, s,
                     y, ids, g, k, E, din, out);
  err = hipGetLastError();
  if (err != hipSuccess) return fail(BITSMOE_EHIP, "combine launch: %s", hipGetErrorString(err));
  return BITSMOE_OK;
}

}  // extern "C"
