// Route grouping of the (token, slot) pairs by expert, as the body of one
// work-group of NT lanes.  It runs as a launch of its own (any E) or as one
// extra work-group of the launch before the coefficient pass (E up to
// kRouteFuseMaxE, counters in static LDS), which saves a dependent launch.
//
// BitsMoE blog note, Methodology, "first split": z is formed once per token
// and shared by every expert the token is routed to.  Grouping the pairs by
// expert extends that reuse across tokens: an expert's planes are read once
// per tile of up to kTile pairs.
//
// Counting sort: an LDS histogram of the ids, a block scan of per-thread
// runs of experts, then a scatter into per-expert pair lists (experts
// ascending; the order inside a list does not affect any result), cut into
// tiles, and the tiles of each expert into groups of up to kSuperTiles.
// Pairs whose id lies outside [0, E) get NaN rows in h.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

namespace bitsmoe {

constexpr int kRouteFuseMaxE = 1024;  // experts a fused route work-group handles
constexpr int kRouteBatch = 16;       // ids a lane loads at once

struct RouteJob {
  const int32_t* ids;  // null: no route work in this launch
  int P, E, dout;
  float* h;            // rows of pairs with an invalid id become NaN
  RouteLists rl;
  uint32_t* zero;      // zero[0, nzero) is cleared (the coefficient tables' flags)
  int nzero;
};

// Exclusive block scans of three values per thread over NT threads (NT a
// multiple of 64, at most 1024); total gets each sum.  Each wave scans its
// lanes with shuffles, publishes its totals in buf (3 NT / 64 words), and
// every wave adds the totals of the waves before it: two barriers for all
// three scans.
template <int NT>
__device__ __forceinline__ void route_scan3(const uint32_t (&v)[3], uint32_t* buf,
                                            uint32_t (&excl)[3], uint32_t (&total)[3]) {
  constexpr int kW = 64, NW = NT / kW;
  static_assert(NT % kW == 0 && NW <= 16, "route scan");
  const int lane = threadIdx.x & (kW - 1), wv = threadIdx.x / kW;
  uint32_t inc[3];
#pragma unroll
  for (int q = 0; q < 3; ++q) {
    inc[q] = v[q];
#pragma unroll
    for (int d = 1; d < kW; d <<= 1) {
      const uint32_t t = __shfl_up(inc[q], d, kW);
      if (lane >= d) inc[q] += t;
    }
    if (lane == kW - 1) buf[q * NW + wv] = inc[q];
  }
  __syncthreads();
#pragma unroll
  for (int q = 0; q < 3; ++q) {
    uint32_t off = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const uint32_t t = buf[q * NW + w];
      off += w < wv ? t : 0u;
      tot += t;
    }
    excl[q] = off + inc[q] - v[q];
    total[q] = tot;
  }
  __syncthreads();  // (buf is free again)
}

// cnt: 2 E words of LDS (counters, then cursors); buf: NT words of LDS.
template <int NT>
__device__ void route_lists(const RouteJob& j, uint32_t* cnt, uint32_t* buf) {
  uint32_t* cur = cnt + j.E;
  const int tid = threadIdx.x;
  for (int i = tid; i < j.nzero; i += NT) j.zero[i] = 0u;
  for (int i = tid; i < j.E; i += NT) cnt[i] = 0;
  __syncthreads();
  // (with more pairs than lanes, the ids of a batch are all loaded before
  // any is used: one round trip per kRouteBatch ids of a lane, not one each)
  if (j.P <= NT) {
    const int e = tid < j.P ? j.ids[tid] : -1;
    if (e >= 0 && e < j.E) atomicAdd(&cnt[e], 1u);
  } else for (int p0 = 0; p0 < j.P; p0 += NT * kRouteBatch) {
    int ev[kRouteBatch];
#pragma unroll
    for (int u = 0; u < kRouteBatch; ++u) {
      const int p = p0 + tid + u * NT;
      ev[u] = p < j.P ? j.ids[p] : -1;
    }
#pragma unroll
    for (int u = 0; u < kRouteBatch; ++u)
      if (ev[u] >= 0 && ev[u] < j.E) atomicAdd(&cnt[ev[u]], 1u);
  }
  __syncthreads();
  // each thread owns a contiguous run of experts
  const int per = (j.E + NT - 1) / NT;
  const int e0 = min(j.E, tid * per), e1 = min(j.E, e0 + per);
  uint32_t sum = 0, nt = 0, ns = 0;
  for (int e = e0; e < e1; ++e) {
    const uint32_t te = (cnt[e] + kTile - 1) / kTile;
    sum += cnt[e];
    nt += te;
    ns += (te + kSuperTiles - 1) / kSuperTiles;
  }
  const uint32_t sv[3] = {sum, nt, ns};
  uint32_t ex[3], tot[3];
  route_scan3<NT>(sv, buf, ex, tot);
  uint32_t off = ex[0], ti = ex[1], si = ex[2];
  const uint32_t total_tiles = tot[1], total_st = tot[2];
  for (int e = e0; e < e1; ++e) {
    const uint32_t c = cnt[e], t0 = ti;
    cur[e] = off;
    for (uint32_t i = 0; i < c; i += kTile, ++ti) {
      j.rl.tile[3 * ti] = e;
      j.rl.tile[3 * ti + 1] = (int)(off + i);
      j.rl.tile[3 * ti + 2] = (int)min((uint32_t)kTile, c - i);
    }
    // groups of up to kSuperTiles consecutive tiles of this expert
    for (uint32_t q = t0; q < ti; q += kSuperTiles, ++si) {
      const uint32_t nq = min((uint32_t)kSuperTiles, ti - q);
      int* g = j.rl.stile + (size_t)kGroupRec * si;
      g[0] = (int)q;
      g[1] = (int)nq;
      g[2] = e;
      for (uint32_t u = 0; u < (uint32_t)kSuperTiles; ++u) {
        const uint32_t i = (q - t0 + u) * kTile;  // the tile's first pair of this expert
        g[3 + 2 * u] = u < nq ? (int)(off + i) : 0;
        g[4 + 2 * u] = u < nq ? (int)min((uint32_t)kTile, c - i) : 0;
      }
      for (int u = 3 + 2 * kSuperTiles; u < kGroupRec; ++u) g[u] = 0;
    }
    off += c;
  }
  if (tid == 0) {
    j.rl.ntiles[0] = (int)total_tiles;
    j.rl.nstiles[0] = (int)total_st;
  }
  __syncthreads();
  if (j.P <= NT) {
    const int e = tid < j.P ? j.ids[tid] : 0;
    if (tid < j.P) {
      if (e >= 0 && e < j.E) {
        j.rl.pairs[atomicAdd(&cur[e], 1u)] = tid;
      } else {
        for (int i = 0; i < j.dout; ++i) j.h[(size_t)tid * j.dout + i] = __builtin_nanf("");
      }
    }
  } else for (int p0 = 0; p0 < j.P; p0 += NT * kRouteBatch) {
    int ev[kRouteBatch];
#pragma unroll
    for (int u = 0; u < kRouteBatch; ++u) {
      const int p = p0 + tid + u * NT;
      ev[u] = p < j.P ? j.ids[p] : 0;
    }
#pragma unroll
    for (int u = 0; u < kRouteBatch; ++u) {
      const int p = p0 + tid + u * NT, e = ev[u];
      if (p >= j.P) continue;
      if (e >= 0 && e < j.E) {
        j.rl.pairs[atomicAdd(&cur[e], 1u)] = p;
      } else {
        for (int i = 0; i < j.dout; ++i) j.h[(size_t)p * j.dout + i] = __builtin_nanf("");
      }
    }
  }
}

}  // namespace bitsmoe
