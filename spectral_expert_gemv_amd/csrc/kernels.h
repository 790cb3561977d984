// Internal launchers shared by the C-ABI translation unit.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace bitsmoe {

// Workspace layout of one gate/up call (offsets in bytes from ws).
struct GateUpPlan {
  size_t z_off;       // T x 2r float32 (two-launch path)
  size_t zt_off;      // T x 2r uint64 tagged z (one-launch path)
  size_t sync_off;    // uint32 epoch, uint32 grid arrival counter (left at 0)
  size_t total;
};
GateUpPlan gateup_plan(int T, int r);

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
  const uint4* phi_t;  // 2r x din fp16 (one-launch path)
  const uint4* x;      // T x din fp16 (one-launch path)
  int din8, T;
  uint64_t* zt;        // T x 2r tagged z (one-launch path)
  const float* z;      // T x 2r z (two-launch path)
  uint32_t* epoch;
  uint32_t* arrive;
};
// Staged gate/up kernel: one work-group per (token, slot, 32-row half-slab).
// staged_capacity(): work-groups resident at once on the current device
// (0: unknown); the one-launch variant needs staged_blocks() <= capacity.
size_t staged_lds_bytes();
int staged_capacity();
long long staged_blocks(int T, int k, int dout);
void launch_gateup_staged(const StagedArgs& s, bool fused, hipStream_t st);

}  // namespace bitsmoe
