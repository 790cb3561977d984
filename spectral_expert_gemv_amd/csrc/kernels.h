// Internal launchers shared by the C-ABI translation unit.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace bitsmoe {

constexpr int kHalfMaxTokens = 4;   // one-launch path: T <= this
constexpr int kHalfMaxR = 4096;      //   and r <= this (z of a token fits LDS)
constexpr int kGroupMaxR = 4096;     // grouped path: r <= this
constexpr int kGroupMaxE = 16384;    //   and E <= this (route histogram in LDS)

// Workspace layout of one gate/up call (offsets in bytes from ws).
struct GateUpPlan {
  size_t z_off;       // T x 2r float32 (projection launch of the batched paths)
  size_t zt_off;      // T x 2r uint64 tagged z (one-launch path)
  size_t sync_off;    // uint32 epoch, uint32 grid arrival counter (left at 0)
  size_t route_off;   // route lists: ngroups, gexp[gmax], goff[gmax + 1], pairs[T k]
  size_t total;
};
GateUpPlan gateup_plan(int T, int k, int E, int r);

struct GateUpArgs {
  const uint8_t* blob_g;
  const uint8_t* blob_u;
  uint64_t bytes_g, bytes_u;
  int E, dout, r;
  const int32_t* ids;
  int ktop, npairs;
  float* h;           // npairs x dout
  int n_slabs;
};

struct StagedArgs {
  GateUpArgs g;
  int T;
  const float* z;      // T x 2r z computed by the projection launch
};
// Staged gate/up kernel (second launch of the two-launch path): one
// work-group per (token, slot, 32-row half-slab).
size_t staged_lds_bytes();
long long staged_blocks(int T, int k, int dout);
int launch_gateup_staged(const StagedArgs& s, hipStream_t st);

// One-launch gate/up kernel, one work-group per (pair, half-slab) unit.
struct HalfArgs {
  GateUpArgs g;
  const uint4* phi_t;  // 2r x din fp16
  const uint4* x;      // T x din fp16
  int din8, T;
  uint64_t* zt;        // T x 2r tagged z
  uint32_t* epoch;
  uint32_t* arrive;
  int grid;            // multiple of 8
};
size_t half_lds_bytes();
int half_grid();  // work-groups of the half-slab kernel on this device (0: unavailable)
void launch_gateup_half(const HalfArgs& s, hipStream_t st);

// Pairs grouped by expert (written by the route-grouping launch).
struct RouteLists {
  int* ngroups;  // [1]
  int* gexp;     // expert of group g, ascending
  int* goff;     // pairs of group g: pairs[goff[g] .. goff[g + 1])
  int* pairs;    // pair indices t * k + slot
};
struct GroupArgs {
  GateUpArgs g;
  const float* z;  // T x 2r
  RouteLists rl;
  int gmax;        // min(E, T * k): groups the grid is sized for
};
size_t grouped_lds_bytes();
int grouped_tokens_per_batch(int r);  // 0: r too large for the grouped kernel
int launch_route_group(const int32_t* ids, int P, int E, int dout, float* h,
                       const RouteLists& rl, hipStream_t st);
int launch_gateup_grouped(const GroupArgs& s, hipStream_t st);

}  // namespace bitsmoe
