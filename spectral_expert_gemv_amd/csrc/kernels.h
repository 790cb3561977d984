// Internal launchers shared by the C-ABI translation unit.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace bitsmoe {

// Workspace layout of one gate/up call (offsets in bytes from ws).
struct GateUpPlan {
  int parts;          // most column parts per (pair, slab, projection)
  int n_slabs;
  size_t z_off;       // T x 2r float32 (two-launch path)
  size_t zt_off;      // T x 2r uint64 tagged z (one-launch path)
  size_t sync_off;    // uint32 epoch, uint32 grid arrival counter
  size_t part_off;    // pairs x n_slabs x 2 x parts x 64 float32
  size_t cnt_off;     // pairs x n_slabs uint32 arrival counters (left at 0)
  size_t total;
};
GateUpPlan gateup_plan(int T, int k, int dout, int r);

struct GateUpArgs {
  const uint8_t* blob_g;
  const uint8_t* blob_u;
  uint64_t bytes_g, bytes_u;
  int E, dout, r;
  const float* z;     // T x 2r: gate z at [t*2r + k], up z at [t*2r + r + k]
  const int32_t* ids;
  int ktop, npairs;
  float* h;           // npairs x dout
  float* part;
  uint32_t* cnt;
  int parts, n_slabs;
};
// Column-parallel expert kernel with the SiLU * mul epilogue (any T).
void launch_gateup_swar(const GateUpArgs& a, hipStream_t s);

struct FusedArgs {
  GateUpArgs g;
  const uint4* phi_t;  // 2r x din fp16
  const uint4* x;      // T x din fp16
  int din8, T;
  uint64_t* zt;        // T x 2r tagged z
  uint32_t* epoch;
  uint32_t* arrive;
};
// One-launch path (small T): z production and expert work in one grid.
// fused_capacity(): resident work-groups on the current device (0: unknown).
int fused_capacity();
void launch_gateup_fused(const FusedArgs& f, hipStream_t s);

}  // namespace bitsmoe
