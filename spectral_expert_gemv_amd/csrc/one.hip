// One-token gate/up kernel: z = Phi^T x, every routed expert's coefficients,
// both expert projections and SiLU(gate) * up in one launch, with one
// (slot, 32-row segment) unit per work-group.
//
// BitsMoE blog note, Methodology: "first split" (z = Phi^T x formed once per
// token and reused by every routed expert), "second split" (an expert's
// output is the sum over components of magnitude * z_k * quantized unit
// direction) and "execution" (components of one width stored together, plane
// by plane).
//
// gfx950 mapping.
//  * One 1024-lane work-group (16 waves) per compute unit, all resident: a
//    wave issues at most one instruction every four cycles, so the work of a
//    unit is spread over as many waves as one group can hold.  Work-group b
//    owns unit b = segment * pairs + pair when b < units and runs on XCD
//    b % 8, so with 8 routed slots all segments of one slot share one L2.
//  * Waves 0-7 of every work-group produce z for up to four rows of Phi^T
//    each and, with it, the coefficients of those components for every
//    routed slot: the blob's component table (slot, a, s, m of component k
//    in k order) is read right after the routed ids, before the Phi^T data
//    is back.  Lane (slot j, row i) forms c = a s z (a z for a 16-bit
//    component), the balanced base-256 digit bytes of rint(c 2^S) (fp16 hi
//    and lo parts of c 2^(S - 16) for 16-bit components) and publishes them
//    as one tagged word at the component's slot; the row-independent part
//    a m z is summed over the wave's rows and published per wave.  The
//    scale S comes from the expert's bound cmax and |z_k| <= ||x||_2 (rows
//    of Phi^T have unit norm), so every producer and consumer finds the
//    same S on its own; a component whose scaled value does not fit four
//    digits turns its rows into NaN.
//  * Waves 8-15 read the routed id (a scalar load issued before any Phi^T
//    load); waves 8-11 read the gate directory record and copy the unit's
//    gate segment record into LDS (global_load_lds), waves 12-15 the same
//    for up.
//  * After one barrier, waves 8-15 take the gate projection and waves 0-7
//    the up projection; wave w of a projection owns its K steps w, w + 8, ...
//    (1..8-bit groups in 64-slot steps for v_mfma_i32_16x16x64_i8, the
//    16-bit group in 32-slot steps for v_mfma_f32_16x16x32_f16).  It loads
//    its steps' coefficient words and its share of the partial sums, checks
//    the tags (stale words are re-read device-coherently, bounded), writes
//    the digit bytes into LDS rows and applies its steps: decode of the
//    staged planes into A operands, one MFMA per step and 16-row tile,
//    exact in int32.
//  * Epilogue: the eight waves of a projection fold their columns with
//    2^(8 n - S) and meet in LDS; wave 0 writes SiLU(gate) * up.
// Steps whose planes lie past the LDS arena are decoded from global memory.
// All waits are bounded: a time-out gives NaN rows and the kernel still
// exits.  Every work-group counts itself on the hint counters once all of
// its waves have read the launch tag; work-group 0 advances the epoch once
// every group has counted itself.
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include "device_common.h"
#include "format.h"
#include "kernels.h"
#include "seg_common.h"
#include "zx.h"

namespace bitsmoe {
namespace {

using namespace seg;
using namespace zx;

constexpr int kOWaves = 16;
constexpr int kOThreads = kOWaves * kWave;  // 1024
constexpr int kOPW = 8;                     // waves per projection
constexpr int kOHint = 4;                   // hint increments per work-group (as the fused kernel)
constexpr int kOArena = 8192;               // staged plane words per projection
constexpr int kONSMax = 9;                  // K steps per wave at most (r <= kOneMaxR: <= 70 steps)
constexpr int kOQ = 2240;                   // 1..8-bit slots per projection at most
constexpr int kO16 = 2080;                  // 16-bit slots per projection at most
constexpr int kOPart = 4;                   // partial sums per lane of a consumer wave
static_assert(kOneMaxR <= 2048, "arenas and the step bound assume r <= 2048");
static_assert(kOQ >= kOneMaxR + 6 * 31 && kO16 >= kOneMaxR + 31, "digit rows cover every slot");
static_assert(kOneSlots >= kOneMaxR + 7 * 31, "coefficient rows cover every slot");
static_assert(kOPart * kWave * kOPW >= kOneMaxR, "partial sums of one projection");
constexpr float kVMax = 2.0e9f;  // |rint(c 2^S)| below this has four balanced base-256 digits

struct __align__(16) OneLds {
  uint32_t W[2][kOArena + 16];    // planes of the unit's segment, gate and up
  int8_t Dg[2][kDigits][kOQ];     // digit rows of the 1..8-bit slots (by slot)
  _Float16 H[2][2][kO16];         // hi, lo rows of the 16-bit slots (by slot - n_qslot)
  int32_t acc[2][kSegRows][kDigits];  // digit columns of each projection, summed over waves
  float acc16[2][kSegRows];         // fp16 columns (hi + lo), summed over waves
  float bias[2][kOPW];
  uint32_t ok[kOWaves];
  uint32_t nst[2];                  // K steps of each projection (0: bad record)
  uint32_t wst[2][kOPW][kONSMax];   // entries (slot0 | nslot << 16) of the steps wave w of a
                                    // projection applies, in order
  uint32_t wsb[2][kOPW];            // the first of those steps
  float xb;                         // ||x||_2 (the bound of every |z_k|)
  SegProj desc[2];
};

// K step i of a projection (uniform): its group g, first slot, slots (64 or
// 32, fewer for a group's last half step) and first plane word.
struct StepInfo {
  int g;
  uint32_t slot0, nslot, word0;
};

struct StepTab {
  uint32_t gb[kNumGroups + 1];   // first block of group g (gb[7] = n_blk)
  uint32_t gw[kNumGroups];       // first plane word of group g
  uint32_t off[kNumGroups + 1];  // first step of group g (off[7] = steps)
};

__device__ __forceinline__ StepTab step_tab(const SegProj& p) {
  StepTab t;
  const uint32_t gb[kNumGroups + 1] = {0u, p.b1, p.b2, p.b3, p.b4, p.b5, p.b6, p.n_blk};
  const uint32_t gw[kNumGroups] = {0u, p.w1, p.w2, p.w3, p.w4, p.w5, p.w6};
  uint32_t o = 0;
#pragma unroll
  for (int g = 0; g < kNumGroups; ++g) {
    t.gb[g] = gb[g];
    t.gw[g] = gw[g];
    t.off[g] = o;
    const uint32_t n32 = (gb[g + 1] - gb[g]) / kBlkPerK;
    o += g < kNumQGroups ? (n32 + 1) / 2 : n32;
  }
  t.gb[kNumGroups] = gb[kNumGroups];
  t.off[kNumGroups] = o;
  return t;
}

__device__ __forceinline__ StepInfo step_info(const StepTab& t, uint32_t i) {
  // (selects with compile-time indices only: an indexed read of the table
  // would place it in scratch memory)
  int g = kNumGroups - 1;
  uint32_t gbs = t.gb[kNumGroups - 1], gbe = t.gb[kNumGroups], gws = t.gw[kNumGroups - 1],
           off = t.off[kNumGroups - 1];
#pragma unroll
  for (int k = 0; k < kNumGroups - 1; ++k) {
    const bool in = i >= t.off[k] && i < t.off[k + 1];
    g = in ? k : g;
    gbs = in ? t.gb[k] : gbs;
    gbe = in ? t.gb[k + 1] : gbe;
    gws = in ? t.gw[k] : gws;
    off = in ? t.off[k] : off;
  }
  StepInfo s;
  s.g = g;
  const bool q = g < kNumQGroups;
  const uint32_t bw = 4u * (uint32_t)group_width(g);  // words per block
  const uint32_t b0 = gbs + (i - off) * (q ? 2u * kBlkPerK : (uint32_t)kBlkPerK);
  const uint32_t nb = min(gbe - b0, q ? 2u * kBlkPerK : (uint32_t)kBlkPerK);
  s.slot0 = 4u * b0;
  s.nslot = 4u * nb;
  s.word0 = gws + (b0 - gbs) * bw;
  return s;
}

// A operands (two 16-row tiles) of one step of width W <= 8 (run-time value,
// uniform) whose plane words start at rec: lane (m, q) holds row m of each
// tile and slots 16 q .. + 15; width 8 as code - 128.  Word j of the lane's
// octet in block d of tile t is rec[16 W q + 4 W d + (2 t + m / 8) W + j];
// the plane loop is unrolled with a uniform test per plane, so every read
// has an immediate offset.  The upper half of a 32-slot step is zero.
template <typename P>
__device__ __forceinline__ void decode_i8(const P* rec, uint32_t W, bool half, int lane,
                                          u32x4& a0, u32x4& a1) {
  const int m = lane & 15, q = lane >> 4, rho = m & 7;
  uint32_t c[2][4] = {{0u, 0u, 0u, 0u}, {0u, 0u, 0u, 0u}};
  const bool live = !(half && q >= 2);
  if (live) {
    const P* r = rec + (16u * q + (uint32_t)(m >> 3)) * W;
    // planes in two halves of four: every read of a half is issued before
    // any of its words is used (reads past the W planes stay inside the
    // step's words plus 3, which the arena's and the block's padding cover;
    // only planes j < W are used), so a half costs one LDS round trip
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      if ((uint32_t)(4 * h) < W) {
        uint32_t w[4][2][4];
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
#pragma unroll
          for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int d = 0; d < 4; ++d) w[jj][t][d] = r[(4u * d + 2u * t) * W + 4 * h + jj];
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int j = 4 * h + jj;
          if ((uint32_t)j < W) {
            const uint32_t sh = (uint32_t)(rho - j) & 31u, mask = 0x01010101u << j;
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
              for (int d = 0; d < 4; ++d)
                c[t][d] |= __builtin_amdgcn_alignbit(w[jj][t][d], w[jj][t][d], sh) & mask;
          }
        }
      }
    }
  }
  // (the zero half stays zero: its B rows hold other slots' digits)
  const uint32_t x = W == 8 && live ? 0x80808080u : 0u;
  a0 = u32x4{c[0][0] ^ x, c[0][1] ^ x, c[0][2] ^ x, c[0][3] ^ x};
  a1 = u32x4{c[1][0] ^ x, c[1][1] ^ x, c[1][2] ^ x, c[1][3] ^ x};
}

// A operands of a 16-bit step: the stored fp16 values (lane q: slots 8 q ..).
template <typename P>
__device__ __forceinline__ void decode_f16(const P* rec, int lane, u32x4& a0, u32x4& a1) {
  h8 h0, h1;
  a_tiles_f16((const uint32_t*)(rec + 2 * (lane >> 4) * 64), lane & 15, h0, h1);
  a0 = __builtin_bit_cast(u32x4, h0);
  a1 = __builtin_bit_cast(u32x4, h1);
}

template <typename P>
__device__ __forceinline__ void decode_step(const P* rec, int g, uint32_t nslot, int lane,
                                            u32x4& a0, u32x4& a1) {
  if (g == kNumGroups - 1)
    decode_f16(rec, lane, a0, a1);
  else
    decode_i8(rec, (uint32_t)group_width(g), nslot < 64, lane, a0, a1);
}

// The same from the LDS arena with the width known at compile time: a
// lane's W words of one octet come with the widest LDS reads their
// alignment allows (a_i8).
template <int W>
__device__ __forceinline__ void decode_w(const uint32_t* rec, bool half, int lane, u32x4& a0,
                                         u32x4& a1) {
  const int m = lane & 15, q = lane >> 4;
  const u32x4 zero = {0u, 0u, 0u, 0u};
  a0 = a1 = zero;
  if (half && q >= 2) return;
  const uint32_t* r = rec + 16 * W * q;
  a0 = __builtin_bit_cast(u32x4, a_i8<W>(r, m, 0));
  a1 = __builtin_bit_cast(u32x4, a_i8<W>(r, m, 1));
}

__device__ __forceinline__ void decode_step_lds(const uint32_t* rec, int g, uint32_t nslot,
                                                int lane, u32x4& a0, u32x4& a1) {
  const bool half = nslot < 64;
  switch (g) {
    case 0: decode_w<1>(rec, half, lane, a0, a1); break;
    case 1: decode_w<2>(rec, half, lane, a0, a1); break;
    case 2: decode_w<3>(rec, half, lane, a0, a1); break;
    case 3: decode_w<4>(rec, half, lane, a0, a1); break;
    case 4: decode_w<6>(rec, half, lane, a0, a1); break;
    case 5: decode_w<8>(rec, half, lane, a0, a1); break;
    default: decode_f16(rec, lane, a0, a1); break;
  }
}

// B operand of a step that starts at slot0: lane (n, q) takes digit row n,
// slots slot0 + 16 q .. + 15 (i8, n < 4), or hi / lo row n of 16-bit slots
// slot0 - n_qslot + 8 q .. + 7 (n < 2).
__device__ __forceinline__ u32x4 b_rows(const OneLds& L, int pj, bool f16, uint32_t slot0,
                                        uint32_t nq, int lane) {
  const int n = lane & 15, q = lane >> 4;
  u32x4 b = {0u, 0u, 0u, 0u};
  if (f16) {
    if (n < 2) b = *reinterpret_cast<const u32x4*>(&L.H[pj][n][slot0 - nq + 8u * q]);
  } else if (n < kDigits) {
    b = *reinterpret_cast<const u32x4*>(&L.Dg[pj][n][slot0 + 16u * q]);
  }
  return b;
}

__device__ __forceinline__ void apply_step(bool f16, const u32x4& a0, const u32x4& a1,
                                           const u32x4& b, i32x4& ai0, i32x4& ai1, f4& af0,
                                           f4& af1) {
  if (f16) {
    const h8 bh = __builtin_bit_cast(h8, b);
    af0 = mfma(__builtin_bit_cast(h8, a0), bh, af0);
    af1 = mfma(__builtin_bit_cast(h8, a1), bh, af1);
  } else {
    const i32x4 bi = __builtin_bit_cast(i32x4, b);
    ai0 = mfma_i8(__builtin_bit_cast(i32x4, a0), bi, ai0);
    ai1 = mfma_i8(__builtin_bit_cast(i32x4, a1), bi, ai1);
  }
}

// This wave's K steps of width group G (steps [lo, hi) that lie in the
// group): decode of the step's planes (from the LDS arena when staged, else
// from global memory), B rows from the digit rows, one MFMA per tile.
template <int G>
__device__ __forceinline__ void apply_group(const OneLds& L, int pj, const StepTab& tb,
                                            uint32_t lo, uint32_t hi, uint32_t staged,
                                            const gu32* gpl, uint32_t nq, int lane,
                                            i32x4& ai0, i32x4& ai1, f4& af0, f4& af1) {
  constexpr bool kQ = G < kNumQGroups;
  constexpr uint32_t kW = G == 0 ? 1 : G == 1 ? 2 : G == 2 ? 3 : G == 3 ? 4 : G == 4 ? 6 : G == 5 ? 8 : 16;
  constexpr uint32_t kBps = kQ ? 2u * kBlkPerK : (uint32_t)kBlkPerK;  // blocks per step
  constexpr uint32_t kWps = kBps * 4u * kW;                            // plane words per whole step
  const uint32_t o0 = tb.off[G], o1 = min(tb.off[G + 1], hi);
  const uint32_t gb0 = tb.gb[G], gb1 = tb.gb[G + 1], gw0 = tb.gw[G];
  uint32_t i0 = max(o0, lo);
  if constexpr (kQ) {
    // Whole 64-slot steps whose planes are in the arena (a prefix of the
    // group's steps): no half-step test and no global-memory path; the B
    // rows are read by every lane and zeroed past the four digit rows.
    const uint32_t ifull = o0 + (gb1 - gb0) / kBps;
    const uint32_t istg = staged >= gw0 ? o0 + (staged - gw0) / kWps : o0;
    const uint32_t ie = min(o1, min(ifull, istg));
    const int n = lane & 15, q = lane >> 4;
    const int8_t* brow = &L.Dg[pj][n & (kDigits - 1)][16 * q];
    const uint32_t* rec = &L.W[pj][gw0 + (i0 - o0) * kWps];
#pragma unroll 1
    for (uint32_t i = i0; i < ie; ++i, rec += kWps) {
      u32x4 x0, x1;
      decode_w<(int)kW>(rec, false, lane, x0, x1);
      const uint32_t b0 = gb0 + (i - o0) * kBps;
      u32x4 b = *reinterpret_cast<const u32x4*>(brow + 4u * b0);
      if (n >= kDigits) b = u32x4{0u, 0u, 0u, 0u};
      apply_step(false, x0, x1, b, ai0, ai1, af0, af1);
    }
    i0 = max(i0, ie);
  }
  // the rest: half steps, and steps decoded from global memory
#pragma unroll 1
  for (uint32_t i = i0; i < o1; ++i) {
    const uint32_t b0 = gb0 + (i - o0) * kBps;
    const uint32_t nb = min(gb1 - b0, kBps);
    const uint32_t w0 = gw0 + (b0 - gb0) * 4u * kW, nw = nb * 4u * kW;
    u32x4 x0, x1;
    if (w0 + nw <= staged) {
      if constexpr (kQ)
        decode_w<(int)kW>(&L.W[pj][w0], nb < kBps, lane, x0, x1);
      else
        decode_f16(&L.W[pj][w0], lane, x0, x1);
    } else {
      decode_step(gpl + w0, G, 4u * nb, lane, x0, x1);
    }
    apply_step(!kQ, x0, x1, b_rows(L, pj, !kQ, 4u * b0, nq, lane), ai0, ai1, af0, af1);
  }
}

// One transposing exchange of an N-value reduction: lanes with bit O set
// keep the upper half of the values (O .. 2 O - 1), the others the lower half.
template <int O, int N>
__device__ __forceinline__ void tstep_n(float (&v)[N], bool up) {
#pragma unroll
  for (int i = 0; i < O; ++i) {
    const float send = up ? v[i] : v[i + O];
    const float keep = up ? v[i + O] : v[i];
    v[i] = keep + __shfl_xor(send, O, kWave);
  }
}

// ||x||_2 of the token (lane l holds 16-byte units l, l + 64, l + 128, l +
// 192 of x, zero past din): the bound on every |z_k| that fixes the
// coefficient scale.  Producers and consumers both call it; it is not
// inlined, so that both run the very same instructions and get the same
// value bit for bit (a butterfly sum is the same in every lane).
__device__ __noinline__ float x_bound(uint4 x0, uint4 x1, uint4 x2, uint4 x3) {
  float acc = 0.f;
  acc = fdot8(x0, x0, acc);
  acc = fdot8(x1, x1, acc);
  acc = fdot8(x2, x2, acc);
  acc = fdot8(x3, x3, acc);
  return sqrtf(wave_sum(acc));
}

// 2^S with |c| 2^S < 2^30 for |c| <= cmax ||x||_2 (0 when that is 0).
__device__ __forceinline__ int coef_scale(float cmax, float xb) { return digit_shift(cmax * xb); }

// Work-group barrier that waits for this wave's LDS accesses only (not for
// its outstanding global stores, which a fence-based barrier would wait
// for); the compiler moves no memory access across it.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

typedef __attribute__((address_space(1))) uint64_t gu64;
typedef __attribute__((address_space(1))) const uint16_t cg16;
typedef __attribute__((address_space(1))) const uint32_t cg32;

__global__ __launch_bounds__(kOThreads) void k_gateup_one(FusedArgs s) {
  extern __shared__ __align__(16) uint8_t lds_raw[];
  OneLds& L = *reinterpret_cast<OneLds*>(lds_raw);
  const GateUpArgs& a = s.g;
  const int lane = threadIdx.x & (kWave - 1);
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  typedef __attribute__((address_space(4))) const uint32_t CU32;
  const int np = a.npairs;  // (one token: the routed slots)
  const int U = np * a.n_seg;
  const bool have = (int)blockIdx.x < U;  // uniform
  const int pair = (int)blockIdx.x % np, sg = (int)blockIdx.x / np;
  const int wp = wv & (kOPW - 1);
  const int R = 2 * a.r;
  const int nzw = s.grid * kOPW;          // producing waves
  const int nrw = (R + nzw - 1) / nzw;    // rows per producing wave (1, 2 or 4; r % 4 == 0)
  const int n0 = ((int)blockIdx.x * kOPW + wp) * nrw;
  const int npp = a.r / nrw;              // producing waves per projection

  // ---- start: the routed ids go out before any Phi^T load ----
  // (a producing lane (slot j, row i) loads id j with a vector load: the
  // Phi^T loads issued after it need not be waited for to use it)
  int e = 0, ep = -1;
  if (wv < kOPW) {
    if ((lane >> 2) < np) ep = *(cg32*)(a.ids + (lane >> 2));
  } else if (have) {
    e = (int)*(CU32*)(a.ids + pair);
  }
  // (no wait for the loads: this barrier only orders the issue)
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");

  // The launch tag (the previous launch's epoch + 1) is read after the
  // first loads of each wave have been issued: its scalar load would
  // otherwise be waited for before them.
  uint32_t tag;
  if (wv < kOPW) {
    // ---- z for up to four rows and the coefficients of those components
    // (one body per rows-per-wave count NR, so no work is spent on rows the
    // wave does not own) ----
    float z = 0.f, xb = 0.f, cs = 0.f, cm = 0.f, ca = 0.f, cmax = 0.f;
    uint32_t cslot = kNoSlot;
    HdrF hd;
    const int pj = n0 >= a.r ? 1 : 0;     // this wave's projection
    const uint8_t* blob = pj ? a.blob_u : a.blob_g;
    const int p = lane >> 2, jr = lane & 3;
    const int k = n0 - pj * a.r + jr;     // this lane's component
    const bool live = p < np && jr < nrw && n0 < R;
    const bool eok = ep >= 0 && ep < a.E;
    auto produce = [&](auto nr_c) {
      constexpr int NR = decltype(nr_c)::value;
      // x first (its norm is formed while the Phi^T rows stream in), then
      // this wave's NR rows of Phi^T
      uint4 xv[4], pv[NR][4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int i = lane + u * kWave;
        xv[u] = i < s.din8 ? ld16(s.x + i) : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int j = 0; j < NR; ++j) {
        const bool own = n0 + j < R;  // uniform
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int i = lane + u * kWave;
          pv[j][u] = own && i < s.din8 ? ld16(s.phi_t + (size_t)(n0 + j) * s.din8 + i)
                                       : make_uint4(0, 0, 0, 0);
        }
      }
      asm volatile("" ::: "memory");
      tag = *(CU32*)s.epoch + 1u;
      hd = load_hdr(blob);
      const uint8_t* ct = blob + ctab_offset((uint64_t)a.E) +
                          (size_t)(eok ? ep : 0) * ctab_stride((uint64_t)a.r);
      // component table entries (global loads, issued behind the Phi^T loads)
      if (live) {
        const uint32_t kc = (uint32_t)k < (uint32_t)a.r ? (uint32_t)k : 0u;
        cslot = *(cg16*)(ct + 2u * kc);
        cs = __half2float(__ushort_as_half(*(cg16*)(ct + ctab_s_off(a.r) + 2u * kc)));
        cm = __half2float(__ushort_as_half(*(cg16*)(ct + ctab_m_off(a.r) + 2u * kc)));
        ca = __uint_as_float(*(cg32*)(ct + ctab_a_off(a.r) + 4u * kc));
        cmax = __uint_as_float(*(cg32*)(ct + ctab_cmax_off(a.r)));
      }
      xb = x_bound(xv[0], xv[1], xv[2], xv[3]);
      // z of row n0 + (lane & (NR - 1)): the NR partial dot products are
      // reduced together (log2 NR transposing exchanges leave row lane &
      // (NR - 1) in every lane, the remaining exchanges finish the sum)
      float v[NR];
#pragma unroll
      for (int j = 0; j < NR; ++j) {
        float acc = 0.f;
#pragma unroll
        for (int u = 0; u < 4; ++u) acc = fdot8(pv[j][u], xv[u], acc);
        v[j] = acc;
      }
      if constexpr (NR == 4) tstep_n<2, NR>(v, (lane & 2) != 0);
      if constexpr (NR >= 2) tstep_n<1, NR>(v, (lane & 1) != 0);
      z = v[0];
#pragma unroll
      for (int off = NR; off < kWave; off <<= 1) z += __shfl_xor(z, off, kWave);
    };
    if (nrw == 1)
      produce(std::integral_constant<int, 1>{});
    else if (nrw == 2)
      produce(std::integral_constant<int, 2>{});
    else
      produce(std::integral_constant<int, 4>{});
    if (wv == 0 && lane == 0) L.xb = xb;  // (every wave finds the same value)
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): every load of this wave is in
    const bool hok = hd.magic == kMagic && hd.version == kVersion && hd.E == (uint32_t)a.E &&
                     hd.dout == (uint32_t)a.dout && hd.r == (uint32_t)a.r;
    const int S = coef_scale(cmax, xb);
    const bool q16 = cs == 0.f;  // a 16-bit component (or none)
    const float c = q16 ? ca * z : (ca * cs) * z;
    const float vf = ldexpf(c, S);
    bool bad = live && (!eok || !hok || !(fabsf(vf) < kVMax) ||
                        (cslot != kNoSlot && cslot >= (uint32_t)kOneSlots));
    float part = q16 ? 0.f : (ca * cm) * z;
    uint64_t* const cwb = s.cw + (size_t)(tag % kZRing) * np * 2 * kOneSlots;
    uint64_t* const bwb = s.bw + (size_t)(tag % kZRing) * np * 2 * a.r;
    if (live && !bad && cslot != kNoSlot) {
      uint32_t w;
      if (q16) {
        const float f = ldexpf(c, S - 16);  // |f| < 2^15
        const _Float16 hi = (_Float16)f;
        const _Float16 lo = (_Float16)(f - (float)hi);
        w = (uint32_t)__builtin_bit_cast(uint16_t, hi) |
            ((uint32_t)__builtin_bit_cast(uint16_t, lo) << 16);
      } else {
        w = digit_bytes((int)rintf(vf));
      }
      __hip_atomic_store(cwb + ((size_t)p * 2 + pj) * kOneSlots + cslot,
                         ((uint64_t)tag << 32) | w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    // the wave's partial sum of a m z per routed slot (rows summed in
    // groups of four lanes); NaN marks a slot whose rows must be NaN
    part += dpp_move<0xB1>(part, 0.f);  // quad_perm [1,0,3,2]
    part += dpp_move<0x4E>(part, 0.f);  // quad_perm [2,3,0,1]
    bad |= __shfl_xor(bad ? 1 : 0, 1, kWave) != 0;
    bad |= __shfl_xor(bad ? 1 : 0, 2, kWave) != 0;
    if (jr == 0 && p < np && n0 < R) {
      const float pv = bad ? __builtin_nanf("") : part;
      __hip_atomic_store(bwb + ((size_t)p * 2 + pj) * a.r + (size_t)((n0 - pj * a.r) / nrw),
                         ((uint64_t)tag << 32) | __float_as_uint(pv), __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
    }
  } else if (have) {
    // ---- both directory records -> descriptors -> staging copies ----
    {
      // warm this XCD's L2 with both directories while the routed id is on
      // its way (one 4-byte copy per lane of a directory line, the first 512
      // lines of both blobs, into the digit rows, which nothing uses before
      // these copies have been waited for below)
      typedef __attribute__((address_space(1))) void gvoid;
      const uint32_t nl = ((uint32_t)a.E * kDirRecBytes + 127u) / 128u;
      uint32_t j = (uint32_t)threadIdx.x - kOPW * kWave;  // 0 .. 511
      j = j < 2u * nl ? j : 2u * nl - 1u;
      const uint8_t* line =
          (j < nl ? a.blob_g : a.blob_u) + kHeaderBytes + 128u * (j < nl ? j : j - nl);
      __builtin_amdgcn_global_load_lds((gvoid*)line,
                                       (lds_void*)(reinterpret_cast<uint8_t*>(&L.Dg[0][0][0]) +
                                                   256 * (wv - kOPW)),
                                       4, 0, 0);
    }
    // waves 8-11 take the gate projection, 12-15 the up projection: each
    // half reads its directory record and stages its segment record
    const int pj = (wv - kOPW) >> 2;
    const uint8_t* blob = pj ? a.blob_u : a.blob_g;
    const DirRec rd = load_rec_s(blob, e, a.E);
    const HdrF hd = load_hdr(blob);
    tag = *(CU32*)s.epoch + 1u;
    const SegProj SP =
        uniform_seg(make_seg(blob, pj ? a.bytes_u : a.bytes_g, e, rd, hd, a.E, a.dout, a.r));
    const int lq = (int)threadIdx.x & 255;
    if (SP.ok) {
      const uint32_t nw = min(SP.seg_words, (uint32_t)kOArena);
      stage16(&L.W[pj][0], SP.planes + (size_t)sg * SP.seg_words, nw / 4u, lq, lane, 256);
    }
    if ((wv & 3) == 0) {
      if (lane == 0) L.desc[pj] = SP;
      // (the column sums start at zero)
      for (int i = lane; i < kSegRows * (kDigits + 1); i += kWave) {
        if (i < kSegRows * kDigits)
          (&L.acc[pj][0][0])[i] = 0;
        else
          L.acc16[pj][i - kSegRows * kDigits] = 0.f;
      }
    } else if ((wv & 3) == 1) {
      // the projection's K steps, one entry per step (slot0 | nslot << 16),
      // and their split over the projection's eight waves: contiguous
      // ranges of about equal cost, a step of width w costing 4 + 4 w (its
      // plane decode is about 16 w + 16 vector instructions whether the
      // step is whole or half) and a 16-bit step 12; steps past
      // kOPW * kONSMax are left out (their records give NaN rows)
      const StepTab tb = step_tab(SP);
      const uint32_t nst = SP.ok ? tb.off[kNumGroups] : 0u;
      const uint32_t ns = min(nst, (uint32_t)(kOPW * kONSMax));
      uint32_t c[2] = {0u, 0u}, ent[2] = {0u, 0u};
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint32_t i = (uint32_t)lane + kWave * h;
        if (i < ns) {
          const StepInfo si = step_info(tb, i);
          ent[h] = si.slot0 | (si.nslot << 16);
          c[h] = si.g == kNumGroups - 1 ? 12u : 4u + 4u * (uint32_t)group_width(si.g);
        }
      }
      // inclusive prefix sums of the costs in step order
      uint32_t q0 = c[0], q1 = c[1];
#pragma unroll
      for (int d = 1; d < kWave; d <<= 1) {
        const uint32_t t0 = __shfl_up(q0, d, kWave), t1 = __shfl_up(q1, d, kWave);
        if (lane >= d) {
          q0 += t0;
          q1 += t1;
        }
      }
      q1 += (uint32_t)__shfl(q0, kWave - 1, kWave);
      const uint32_t tot = max((uint32_t)__shfl(q1, kWave - 1, kWave), 1u);
      // step i goes to wave floor(8 (cost before i + half its cost) / total)
      const uint32_t w0 = min((8u * (2u * (q0 - c[0]) + c[0])) / (2u * tot), (uint32_t)kOPW - 1);
      const uint32_t w1 = min((8u * (2u * (q1 - c[1]) + c[1])) / (2u * tot), (uint32_t)kOPW - 1);
      uint32_t bnd[kOPW + 1];
      bool fits = true;
      bnd[0] = 0u;
#pragma unroll
      for (int w = 1; w <= kOPW; ++w) {
        bnd[w] = w == kOPW ? ns
                           : (uint32_t)__popcll(__ballot((uint32_t)lane < ns && w0 < (uint32_t)w)) +
                                 (uint32_t)__popcll(__ballot((uint32_t)lane + kWave < ns &&
                                                             w1 < (uint32_t)w));
        fits = fits && bnd[w] - bnd[w - 1] <= (uint32_t)kONSMax;
      }
      // (equal counts where a range would be too long)
#pragma unroll
      for (int w = 0; w <= kOPW; ++w)
        bnd[w] = fits ? bnd[w] : ((uint32_t)w * ns + kOPW - 1) / kOPW;
      // each wave's own list: entry j of wave w is step bnd[w] + j (zero
      // past the wave's range, and for every wave of an over-long record)
      for (int i = lane; i < kOPW * kONSMax; i += kWave) (&L.wst[pj][0][0])[i] = 0u;
      const bool over = nst > (uint32_t)(kOPW * kONSMax);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint32_t i = (uint32_t)lane + kWave * h;
        uint32_t w = 0, b = 0;
#pragma unroll
        for (int v = 1; v < kOPW; ++v)
          if (i >= bnd[v]) {
            w = (uint32_t)v;
            b = bnd[v];
          }
        if (i < ns && !over) L.wst[pj][w][i - b] = ent[h];
      }
      uint32_t bl = 0;
#pragma unroll
      for (int v = 1; v < kOPW; ++v) bl = lane == v ? bnd[v] : bl;
      if (lane < kOPW) L.wsb[pj][lane] = bl;
      if (lane == 0) L.nst[pj] = nst;
    } else if ((wv & 3) == 2 && sg == 0 && SP.ok) {
      // the group padding slots of this pair's projection (each group's
      // slots past its stored columns) get tagged zero words, so that every
      // slot of a step has a word of this launch: the pair's segment-0
      // work-group writes them
      uint64_t* const cwb =
          s.cw + ((size_t)(tag % kZRing) * np * 2 + (size_t)pair * 2 + pj) * kOneSlots;
      const uint32_t gb[kNumGroups + 1] = {0u, SP.b1, SP.b2, SP.b3, SP.b4, SP.b5, SP.b6, SP.n_blk};
#pragma unroll
      for (int g = 0; g < kNumGroups; ++g) {
        const uint32_t q1 = min(4u * gb[g + 1], (uint32_t)kOneSlots);
        for (uint32_t q = 4u * gb[g] + rd.count[g] + (uint32_t)lane; q < q1; q += kWave)
          __hip_atomic_store(cwb + q, (uint64_t)tag << 32, __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    __builtin_amdgcn_s_waitcnt(0);  // this wave's copies have landed
  } else {
    // (nothing is outstanding here; the wait tells the compiler so, which
    // keeps it from waiting for the producers' stores at the barrier)
    __builtin_amdgcn_s_waitcnt(0);
    tag = *(CU32*)s.epoch + 1u;
  }
  lds_barrier();  // staged data and descriptors visible

  if (have) {
    const int pj = wv >= kOPW ? 0 : 1;  // waves 8-15 gate, 0-7 up
    // this wave's steps (a contiguous range of at most kONSMax; nst <= 70
    // for r <= 2048, a longer record gives NaN rows): lane j holds the entry
    // of step j (slot0 | nslot << 16), read back as uniform values with
    // v_readlane; the coefficient loads go out first
    const uint32_t e_x = lane < kONSMax ? L.wst[pj][wp][lane] : 0u;
    const uint32_t nmine = (uint32_t)__popcll(__ballot(e_x != 0u));
    gu64* const cwp =
        (gu64*)(s.cw + ((size_t)(tag % kZRing) * np * 2 + (size_t)pair * 2 + pj) * kOneSlots);
    gu64* const bwp = (gu64*)(s.bw + ((size_t)(tag % kZRing) * np * 2 + (size_t)pair * 2 + pj) *
                                         a.r);

#define ST_X(j) ((uint32_t)__builtin_amdgcn_readlane((int)e_x, (j)))
    // lane l's slot in step j: slot0 + l (lanes past a 32-slot step repeat
    // its slots; every slot, group padding included, has a word)
#define SLOT(j) ((ST_X(j) & 0xFFFFu) + ((uint32_t)lane & ((ST_X(j) >> 16) - 1u)))

    // ---- loads of this wave's coefficient words and partial sums ----
    uint64_t cw[kONSMax];
#pragma unroll
    for (int j = 0; j < kONSMax; ++j) {
      cw[j] = (uint64_t)tag << 32;
      if ((uint32_t)j < nmine) cw[j] = cwp[SLOT(j)];
    }
    const int nw4 = (npp + kOPW - 1) / kOPW;  // partial sums this wave adds
    uint64_t pw[kOPart];
#pragma unroll
    for (int i = 0; i < kOPart; ++i) {
      const int q = wp * nw4 + lane + kWave * i;
      pw[i] = (uint64_t)tag << 32;
      if (lane + kWave * i < nw4 && q < npp) pw[i] = bwp[q];
    }
    // every wave of the group has read the epoch: count the group on the
    // hint counters (kOHint waves, as the fused kernel does), after which
    // work-group 0 may advance the epoch
    if (wv < kOHint) hint_add(s, (int)blockIdx.x * kOHint + wv, lane);
    const SegProj P = uniform_seg(L.desc[pj]);
    const uint32_t staged = P.ok ? min(P.seg_words, (uint32_t)kOArena) : 0u;
    const uint32_t nq = P.n_qslot, s8a = 4u * P.b5, s8b = 4u * P.b6;  // width-8 slots
    const uint32_t nst = __builtin_amdgcn_readfirstlane(L.nst[pj]);
    const uint32_t sb0 = __builtin_amdgcn_readfirstlane(L.wsb[pj][wp]);
    const int S = coef_scale(P.cmax, L.xb);

    // ---- the tags: stale words re-read device-coherently, bounded ----
    uint32_t spins = 0;
    while (true) {
      bool ready = true;
#pragma unroll
      for (int j = 0; j < kONSMax; ++j) ready &= (uint32_t)(cw[j] >> 32) == tag;
#pragma unroll
      for (int i = 0; i < kOPart; ++i) ready &= (uint32_t)(pw[i] >> 32) == tag;
      if (__all(ready) || spins >= s.spin) break;
      __builtin_amdgcn_s_sleep(2);
#pragma unroll
      for (int j = 0; j < kONSMax; ++j)
        if ((uint32_t)(cw[j] >> 32) != tag)
          cw[j] = __hip_atomic_load(cwp + SLOT(j), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
      for (int i = 0; i < kOPart; ++i)
        if ((uint32_t)(pw[i] >> 32) != tag)
          pw[i] = __hip_atomic_load(bwp + (wp * nw4 + lane + kWave * i), __ATOMIC_RELAXED,
                                    __HIP_MEMORY_SCOPE_AGENT);
      ++spins;
    }
    const bool zok = spins < s.spin;
    count_timeout(s, !zok, lane);

    // ---- digit rows; the width-8 correction and the partial sums ----
    float corr = 0.f;  // sum of rint(c 2^S) over width-8 slots (those enter as code - 128)
#pragma unroll
    for (int j = 0; j < kONSMax; ++j) {
      if ((uint32_t)j < nmine) {
        const uint32_t ex = ST_X(j), s0 = ex & 0xFFFFu;  // (uniform)
        const uint32_t q0 = s0 + (uint32_t)lane;
        const uint32_t w = (uint32_t)cw[j];
        if ((uint32_t)lane < (ex >> 16)) {
          if (s0 < nq) {
            L.Dg[pj][0][q0] = (int8_t)w;
            L.Dg[pj][1][q0] = (int8_t)(w >> 8);
            L.Dg[pj][2][q0] = (int8_t)(w >> 16);
            L.Dg[pj][3][q0] = (int8_t)(w >> 24);
            if (s0 >= s8a && s0 < s8b) corr += (float)(int)((w ^ 0x80808080u) - 0x80808080u);
          } else {
            reinterpret_cast<uint16_t*>(&L.H[pj][0][0])[q0 - nq] = (uint16_t)w;
            reinterpret_cast<uint16_t*>(&L.H[pj][1][0])[q0 - nq] = (uint16_t)(w >> 16);
          }
        }
      }
    }
    float bias = 0.f;
#pragma unroll
    for (int i = 0; i < kOPart; ++i) bias += __uint_as_float((uint32_t)pw[i]) *
                                             ((lane + kWave * i < nw4) ? 1.f : 0.f);
    // (a NaN partial marks a bad slot: NaN * 0 is NaN too, so lanes past the
    // wave's share load nothing and keep the tag-only word, whose float is 0)
    bias += ldexpf(128.f * corr, -S);
    // (a step's B operand is read by the wave that wrote its digits: LDS
    // accesses of one wave complete in order)

    // ---- apply: decode each step's A operands and multiply, one loop per
    // width group (the width a compile-time value) ----
    i32x4 ai0 = {0, 0, 0, 0}, ai1 = {0, 0, 0, 0};  // column n: digit n
    f4 af0 = {0.f, 0.f, 0.f, 0.f}, af1 = {0.f, 0.f, 0.f, 0.f};  // fp16 columns: hi, lo
    {
      const StepTab tb = step_tab(P);
      const auto gpl = P.planes + (size_t)sg * P.seg_words;
      apply_group<0>(L, pj, tb, sb0, sb0 + nmine, staged, gpl, nq, lane, ai0, ai1, af0, af1);
      apply_group<1>(L, pj, tb, sb0, sb0 + nmine, staged, gpl, nq, lane, ai0, ai1, af0, af1);
      apply_group<2>(L, pj, tb, sb0, sb0 + nmine, staged, gpl, nq, lane, ai0, ai1, af0, af1);
      apply_group<3>(L, pj, tb, sb0, sb0 + nmine, staged, gpl, nq, lane, ai0, ai1, af0, af1);
      apply_group<4>(L, pj, tb, sb0, sb0 + nmine, staged, gpl, nq, lane, ai0, ai1, af0, af1);
      apply_group<5>(L, pj, tb, sb0, sb0 + nmine, staged, gpl, nq, lane, ai0, ai1, af0, af1);
      apply_group<6>(L, pj, tb, sb0, sb0 + nmine, staged, gpl, nq, lane, ai0, ai1, af0, af1);
    }

#undef ST_X
#undef SLOT
    // ---- the eight waves of a projection sum their columns in LDS (exact
    // for the integer columns: one scale serves the whole projection) ----
    {
      const int n = lane & 15, q = lane >> 4;
      if (nmine > 0) {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const i32x4& ai = t ? ai1 : ai0;
          const f4& a16 = t ? af1 : af0;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int row = 16 * t + 4 * q + i;
            if (n < kDigits) atomicAdd(&L.acc[pj][row][n], ai[i]);
            if (n < 2) atomicAdd(&L.acc16[pj][row], a16[i]);
          }
        }
      }
      const float bw = wave_sum_dpp(bias);
      const bool wok = zok && P.ok && nst <= (uint32_t)(kOPW * kONSMax);
      if (lane == 0) {
        L.bias[pj][wp] = bw;
        L.ok[wv] = wok ? 1u : 0u;
      }
    }
    lds_sync();
    if (wv == 0 && lane < kSegRows) {
      // y = sum over digits n of column n 2^(8 n - S) + fp16 columns
      // 2^(16 - S) + the row-independent part, per projection
      float ys[2];
      uint32_t okw = 1u;
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int Sq = q == pj ? S : coef_scale(L.desc[q].cmax, L.xb);
        float sum = ldexpf(L.acc16[q][lane], 16 - Sq), bsum = 0.f;
#pragma unroll
        for (int n = 0; n < kDigits; ++n) sum += ldexpf((float)L.acc[q][lane][n], 8 * n - Sq);
#pragma unroll
        for (int w = 0; w < kOPW; ++w) bsum += L.bias[q][w];
        ys[q] = sum + bsum;
      }
#pragma unroll
      for (int w = 0; w < kOWaves; ++w) okw &= L.ok[w];
      const int row = sg * kSegRows + lane;
      if (row < a.dout)
        a.h[(size_t)pair * a.dout + row] = okw ? silu_mul(ys[0], ys[1]) : __builtin_nanf("");
    }
  } else if (wv < kOHint) {
    hint_add(s, (int)blockIdx.x * kOHint + wv, lane);
  }

  // Work-group 0 advances the epoch once every producing wave has counted
  // itself (waited for with the default bound also when a test lowered the
  // launch's bound).
  if (blockIdx.x == 0 && wv == 0) {
    count_timeout(s, !wait_hint(s.hint, tag * (uint32_t)(s.grid * kOHint), max(s.spin, kSpinDefault)),
                  lane);
    if (lane == 0) __hip_atomic_store(s.epoch, tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

}  // namespace

int one_grid() {
  static int grid[64];
  static bool done[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  if (!done[dev]) {
    int cus = 0, nb = 0;
    (void)hipFuncSetAttribute((const void*)k_gateup_one,
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)sizeof(OneLds));
    (void)hipGetLastError();
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, k_gateup_one, kOThreads,
                                                     sizeof(OneLds)) != hipSuccess)
      return 0;
    grid[dev] = (nb >= 1 && cus >= 8) ? (cus & ~7) : 0;
    done[dev] = true;
  }
  return grid[dev];
}

void launch_gateup_one(const FusedArgs& s, hipStream_t st) {
  hipLaunchKernelGGL(k_gateup_one, dim3((unsigned)s.grid), dim3(kOThreads), sizeof(OneLds), st,
                     s);
}

}  // namespace bitsmoe
