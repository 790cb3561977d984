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
// tiles.  Pairs whose id lies outside [0, E) get NaN rows in h.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

namespace bitsmoe {

constexpr int kRouteFuseMaxE = 1024;  // experts a fused route work-group handles

struct RouteJob {
  const int32_t* ids;  // null: no route work in this launch
  int P, E, dout;
  float* h;            // rows of pairs with an invalid id become NaN
  RouteLists rl;
  uint32_t* zero;      // zero[0, nzero) is cleared (the coefficient tables' flags)
  int nzero;
};

// Exclusive block scan of one value per thread over NT threads; total gets
// the sum.
template <int NT>
__device__ __forceinline__ uint32_t route_scan(uint32_t v, uint32_t* buf, uint32_t& total) {
  const int tid = threadIdx.x;
  buf[tid] = v;
  __syncthreads();
  for (int d = 1; d < NT; d <<= 1) {
    const uint32_t a = tid >= d ? buf[tid - d] : 0u;
    __syncthreads();
    buf[tid] += a;
    __syncthreads();
  }
  total = buf[NT - 1];
  const uint32_t incl = buf[tid];
  __syncthreads();
  return incl - v;
}

// cnt: 2 E words of LDS (counters, then cursors); buf: NT words of LDS.
template <int NT>
__device__ void route_lists(const RouteJob& j, uint32_t* cnt, uint32_t* buf) {
  uint32_t* cur = cnt + j.E;
  const int tid = threadIdx.x;
  for (int i = tid; i < j.nzero; i += NT) j.zero[i] = 0u;
  for (int i = tid; i < j.E; i += NT) cnt[i] = 0;
  __syncthreads();
  for (int p = tid; p < j.P; p += NT) {
    const int e = j.ids[p];
    if (e >= 0 && e < j.E) atomicAdd(&cnt[e], 1u);
  }
  __syncthreads();
  // each thread owns a contiguous run of experts
  const int per = (j.E + NT - 1) / NT;
  const int e0 = min(j.E, tid * per), e1 = min(j.E, e0 + per);
  uint32_t sum = 0, nt = 0;
  for (int e = e0; e < e1; ++e) {
    sum += cnt[e];
    nt += (cnt[e] + kTile - 1) / kTile;
  }
  uint32_t total_pairs, total_tiles;
  uint32_t off = route_scan<NT>(sum, buf, total_pairs);
  uint32_t ti = route_scan<NT>(nt, buf, total_tiles);
  for (int e = e0; e < e1; ++e) {
    const uint32_t c = cnt[e];
    cur[e] = off;
    for (uint32_t i = 0; i < c; i += kTile, ++ti) {
      j.rl.tile[3 * ti] = e;
      j.rl.tile[3 * ti + 1] = (int)(off + i);
      j.rl.tile[3 * ti + 2] = (int)min((uint32_t)kTile, c - i);
    }
    off += c;
  }
  if (tid == 0) j.rl.ntiles[0] = (int)total_tiles;
  __syncthreads();
  for (int p = tid; p < j.P; p += NT) {
    const int e = j.ids[p];
    if (e >= 0 && e < j.E) {
      j.rl.pairs[atomicAdd(&cur[e], 1u)] = p;
    } else {
      for (int i = 0; i < j.dout; ++i) j.h[(size_t)p * j.dout + i] = __builtin_nanf("");
    }
  }
}

}  // namespace bitsmoe
