// Internal launchers shared by the C-ABI translation unit.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace bitsmoe {

constexpr int kFusedMaxTokens = 4;   // one-launch path: T <= this
constexpr int kFusedMaxR = 4096;     //   and r <= this
constexpr int kZRing = 8;            // tagged z buffers of the one-launch path (by launch)
constexpr size_t kSyncBytes = 128 + 64 * 128;  // epoch line + 64 hint counter lines
constexpr uint32_t kSpinDefault = 1u << 20;    // bound on the one-launch kernels' waits
constexpr int kGroupMaxR = 4096;     // grouped path: r <= this
constexpr int kGroupMaxE = 16384;    //   and E <= this (route histogram in LDS)
constexpr int kGroupMaxDin = 4096;   //   and din <= this (row-blocked projection)
constexpr int kProjRowsPerBlock = 16;  // Phi^T rows per work-group of the projection
constexpr int kTile = 16;            // tokens per grouped work unit (MFMA N)

// Workspace layout of one gate/up call (offsets in bytes from ws).  The sync
// words come first, at an offset that depends on nothing, so one workspace
// can serve calls of different shapes in turn: no other part of a call's
// layout ever overlaps them.
struct GateUpPlan {
  size_t sync_off;    // = 0: uint32 epoch (the last one-launch call's tag), then
                      // from byte 128 the 64 cumulative hint counters, 128 bytes
                      // apart (kSyncBytes in all)
  size_t z_off;       // T x 2r float32 (projection launch of the batched path)
  size_t zpart_off;   // T x ceil(2r / 16) float32: max |z| per projection work-group
  size_t zt_off;      // ring of kZRing x T x 2r uint64 tagged z (one-launch path)
  size_t cw_off;      // one-token kernel (T = 1): the rings of FusedArgs::cw and bw
  size_t route_off;   // route lists (see RouteLists)
  size_t coef_off;    // per-tile coefficient tables (batched path, see GroupArgs)
  size_t total;
};
GateUpPlan gateup_plan(int T, int k, int E, int r);
int tile_cap(int T, int k, int E);  // tiles the grouped grid is sized for

struct GateUpArgs {
  const uint8_t* blob_g;
  const uint8_t* blob_u;
  uint64_t bytes_g, bytes_u;
  int E, dout, r;
  const int32_t* ids;
  int ktop, npairs;
  float* h;           // npairs x dout
  int n_seg;          // ceil(dout / 32)
};

// One-launch gate/up kernel (T <= kFusedMaxTokens): z = Phi^T x produced by
// every work-group and exchanged through tagged words, then one work-group
// per (pair, 32-row segment) unit.
struct FusedArgs {
  GateUpArgs g;
  const uint4* phi_t;  // 2r x din fp16
  const uint4* x;      // T x din fp16
  int din8, T;
  uint64_t* zt;        // kZRing x T x 2r tagged z (launch with tag g uses buffer g % kZRing)
  uint32_t* epoch;     // tag of the previous launch
  uint32_t* hint;      // 64 counters, 32 words apart: producing waves done, cumulative over launches
  int grid;            // multiple of 8, all work-groups resident
  uint32_t spin;       // bound on the z exchange waits (0: give up at once, rows NaN)
  uint32_t* timeouts;  // waits that gave up, cumulative over launches (word 1 of the sync line)
  // one-token kernel: kZRing launch buffers (the tag picks one) of tagged
  // coefficient words, pairs x 2 x kOneSlots (slot order), and of tagged
  // row-independent partial sums, pairs x 2 x r
  uint64_t* cw;
  uint64_t* bw;
};
size_t fused_lds_bytes();
int fused_grid();  // work-groups of the fused kernel on this device (0: unavailable)
void launch_gateup_fused(const FusedArgs& s, hipStream_t st);

// One-token kernel (T = 1, r <= kOneMaxR, din <= kOneMaxDin, 2r <= 32 grid,
// pairs * segments <= grid): one
// unit per work-group, codes decoded before z arrives; same arguments, tags,
// ring and hint counters as the fused kernel (so one workspace serves both).
constexpr int kOneMaxR = 2048;
constexpr int kOneMaxDin = 2048;
constexpr int kOneMaxK = 16;        // routed slots (4 lanes of a producing wave each)
constexpr int kOneSlots = 2304;     // slots of one projection (r + 7 * 31, rounded up)
int one_grid();  // work-groups of the one-token kernel (0: unavailable)
void launch_gateup_one(const FusedArgs& s, hipStream_t st);

// Pairs grouped by expert and cut into tiles of <= kTile pairs (written by
// the route-grouping launch).
struct RouteLists {
  int* ntiles;   // [1]
  int* tile;     // per tile: expert id, first pair index into pairs, pair count (3 ints)
  int* pairs;    // pair indices t * k + slot, grouped by expert
  int* nstiles;  // [1]
  int* stile;    // per group of up to kSuperTiles consecutive tiles of one expert, one
                 // 8-int record: first tile, tile count, expert id, then first pair
                 // and pair count of each tile (0 past the count), 0
};
constexpr int kSuperTiles = 2;  // tiles of one expert a grouped work-group applies together
constexpr int kGroupRec = 8;    // ints of a group record
static_assert(3 + 2 * kSuperTiles <= kGroupRec, "group record");
// ints of the route lists for tcap tiles and P pairs, and their places
inline size_t route_ints(int tcap, size_t P) {
  return 2 + (3 + (size_t)kGroupRec) * (size_t)tcap + P;
}
inline void route_lists_at(RouteLists& rl, int* rb, int tcap, size_t P) {
  rl.ntiles = rb;
  rl.tile = rb + 1;
  rl.pairs = rb + 1 + 3 * (size_t)tcap;
  rl.nstiles = rl.pairs + P;
  rl.stile = rl.nstiles + 1;
}
struct GroupArgs {
  GateUpArgs g;
  const float* z;      // T x 2r
  const float* zpart;  // T x nzp: max |z| per projection work-group
  int nzp;             // projection work-groups (ceil(2r / 16))
  RouteLists rl;
  int tcap;            // tiles the grid is sized for
  // 0: gate and up (waves 0-3 / 4-7), SiLU * mul into h.  1: one projection
  // (blob_g == blob_u) with z per pair (row p of z, nzp maxima per pair):
  // the two wave halves take segments 2 s and 2 s + 1, y goes to h.
  int single;
  // per-tile coefficient tables (k_group_coef): fp16 hi and lo parts of
  // c 2^S of token column n and slot s at [((tile * 2 + proj) * kTile + n) *
  // rpad + s]; the row-independent sums per 256-slot chunk at
  // [((tile * 2 + proj) * nck + chunk) * kTile + n]; a flag per (tile, proj)
  // set when a column index is out of range; the scale S of token column n at
  // [(tile * 2 + proj) * kTile + n]
  _Float16* thi;
  _Float16* tlo;
  float* tbias;
  uint32_t* tbad;
  int* tsh;
  int rpad, nck;
};
// slots of a tile's coefficient rows: the largest slot count an expert can
// have (r plus group padding), rounded up to whole 256-slot chunks
inline int group_rpad(int r) { return (r + 7 * 31 + 255) / 256 * 256; }
int launch_group_coef(const GroupArgs& s, hipStream_t st);
size_t group_coef_bytes(int tcap, int r);                // workspace of the tables
void group_coef_tables(GroupArgs& gs, uint8_t* base, int r);  // sets thi .. nck (needs tcap)
size_t grouped_lds_bytes();
// z = Phi^T x and, when zpart is not null (din <= kGroupMaxDin), the largest
// |z| of every 16-row block of the projection per token.  A route job (may
// be null) runs inside the launch when the kernel taken can host it (E <=
// kRouteFuseMaxE); *routed tells whether it did.  x_f32: x is float32,
// rounded to fp16 as it is staged (T < 16 or din % 32 != 0, din <= 4096,
// x 16-byte aligned; otherwise an error).
struct RouteJob;
int launch_proj_maxima(const void* phi, const void* x, float* z, float* zpart, int T, int din,
                       int R, hipStream_t st, const RouteJob* route = nullptr,
                       bool* routed = nullptr, bool x_f32 = false);
// also zero-fills zero[0, nzero) (the coefficient tables' flags)
int launch_route_group(const int32_t* ids, int P, int E, int dout, float* h,
                       const RouteLists& rl, hipStream_t st, uint32_t* zero = nullptr,
                       int nzero = 0);
int launch_gateup_grouped(const GroupArgs& s, hipStream_t st);

}  // namespace bitsmoe
