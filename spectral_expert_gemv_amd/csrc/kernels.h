// Internal launchers shared by the C-ABI translation unit.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace bitsmoe {

// Workspace layout of one gate/up call (offsets in bytes from ws).
struct GateUpPlan {
  int parts;          // column parts per (pair, slab, projection)
  int n_slabs;
  size_t z_off;       // T x 2r float32
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
// Lane-mask expert kernel with the SiLU * mul epilogue (any T).
void launch_gateup_exec(const GateUpArgs& a, hipStream_t s);

}  // namespace bitsmoe
