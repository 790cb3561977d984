// One-launch gate/up kernel with one (pair, 32-row segment) unit per
// work-group (r <= 2048, units <= work-groups): the unit's codes are decoded
// into matrix-core operands held in registers while z is still being
// produced, so that once z has been exchanged only the coefficients, one
// pass of MFMAs and the epilogue remain on the critical path.
//
// BitsMoE blog note, Methodology: "first split" (z = Phi^T x once per token,
// reused by every routed expert), "second split" (an expert's output is the
// sum over components of magnitude * z_k * quantized unit direction) and
// "execution" (components of one width stored together, plane by plane).
//
// gfx950 mapping.
//  * Work-group u owns unit u = segment * pairs + pair and runs on XCD u % 8,
//    so with 8 pairs every segment of one pair shares one L2 (the pair's slot
//    metadata is fetched once per XCD).  Work-groups without a unit only
//    produce z.
//  * Waves 0-3 (gate) issue their Phi^T rows first, then read the routed id,
//    the gate directory record and the gate slot metadata; they produce and
//    publish z (zx.h).  Waves 4-7 (up) prefetch both directories into L2,
//    read the routed id and both records, copy the unit's gate and up
//    segment records into LDS with 16-byte global_load_lds and load the up
//    slot metadata.  None of the expert loads depends on z, so they queue
//    right behind the Phi^T stream.
//  * Decode before z: a projection's work is a list of K steps -- the 1..8-bit
//    width groups in 64-slot steps for v_mfma_i32_16x16x64_i8 (a group's
//    last step may be half), the 16-bit group in 32-slot steps for
//    v_mfma_f32_16x16x32_f16 -- and wave w of a projection takes steps w,
//    w + 4, ...: it decodes their A operands (the code bytes as the plane
//    decode produces them, width 8 as code - 128; fp16 values for 16-bit
//    slots) into up to 10 register slots of 8 VGPRs each.  The slot
//    metadata is folded into w = a s (a for 16-bit slots) and a m per slot.
//  * After z: one wave polls the hint counters, all lanes copy the token's
//    z into LDS and reduce max |z|; the coefficient scale S follows from the
//    expert's bound cmax (directory) and max |z| (|a s z| 2^S < 2^30).  Each
//    lane forms c = w z for its 9 slots: the 1..8-bit slots as the four
//    balanced base-256 digit bytes of v = rint(c 2^S) in four digit rows,
//    the 16-bit slots as the fp16 hi and lo parts of c 2^(S - 16).
//  * Apply: one MFMA per register slot and 16-row tile with the digit rows
//    as B columns 0-3 (exact int32 sums) or hi and lo as columns 0 and 1;
//    the columns are folded with 2^(8 n - S) and 2^(16 - S); the four waves'
//    row sums meet in LDS and wave 0 adds the width-8 correction and the
//    row-independent sum a m z and writes SiLU(gate) * up.
// Records larger than the LDS arena, or with more steps than the register
// slots hold, are decoded and applied in further batches after z (staged,
// decoded and applied one batch at a time).  Work-groups wait for other
// groups' z, so the host launches at most as many groups as can be resident
// at once; all waits are bounded (a time-out gives NaN rows and the kernel
// still exits).  Work-group 0 advances the epoch once every producer of the
// launch has counted itself.
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include "device_common.h"
#include "format.h"
#include "kernels.h"
#include "seg_common.h"
#include "slotmeta.h"
#include "zx.h"

namespace bitsmoe {
namespace {

using namespace seg;
using namespace zx;

constexpr int kUWaves = 8;
constexpr int kUThreads = kUWaves * kWave;  // 512
constexpr int kUProj = 256;                 // lanes per projection (waves 0-3 gate, 4-7 up)
constexpr int kUPW = kUWaves / 2;           // waves per projection
constexpr int kUSlot = 10;                  // register slots of A operands per wave
constexpr int kUBatch = kUPW * kUSlot;      // K steps of a projection per register batch
constexpr int kUArena = 10240;              // staged plane words per projection
constexpr int kUSper = 9;                   // slots per lane of the coefficient pass
constexpr int kUSlots = 9 * kUProj;         // slot space the lanes own: 8 lp + i, 2048 + lp
constexpr int kU16 = kUnitMaxR + 32;        // 16-bit slots of one projection (<= r + 31)
constexpr int kUZ = 2 * kUnitMaxR;          // z values of one token (gate, up)
constexpr int kUZPer = kUZ / kUThreads;     // tagged z words per lane
static_assert(kUSlots >= kUnitMaxR + 7 * 31, "every slot has an owner lane");
#define UNIT_SLOTS(X) X(0) X(1) X(2) X(3) X(4) X(5) X(6) X(7) X(8) X(9)
static_assert(kUSlot == 10, "UNIT_SLOTS lists the register slots");

struct __align__(16) UnitLds {
  uint32_t W[2][kUArena];            // staged plane words of the current batch
  float Z[kUZ];                      // the unit's token's z (gate, then up)
  int8_t Lb[2][kDigits][kUSlots];    // digit rows of v = rint(c 2^S), 1..8-bit slots
  _Float16 H[2][2][kU16];            // hi, lo of c 2^(S - 16), 16-bit slots
  float red[2][kUPW][kSegRows];
  float wmax[kUWaves];               // max |z| per wave
  float pbias[2][kUPW];              // row-independent sum a m z per wave
  float pcorr[2][kUPW];              // 128 sum v 2^-S over width-8 slots per wave
  uint32_t pok[2][kUPW];
  uint32_t zok[kUWaves];
};

// K step list of one projection (uniform): the 1..8-bit groups in 64-slot
// steps, then the 16-bit group in 32-slot steps.
struct Steps {
  uint32_t gb[kNumGroups + 1];   // first block of each group; gb[7] = n_blk
  uint32_t off[kNumGroups + 1];  // first step of each group; off[7] = all steps
};

__device__ __forceinline__ Steps make_steps(const SegProj& p) {
  Steps st;
  const uint32_t gb[kNumGroups + 1] = {0u, p.b1, p.b2, p.b3, p.b4, p.b5, p.b6, p.n_blk};
  uint32_t o = 0;
#pragma unroll
  for (int g = 0; g < kNumGroups; ++g) {
    st.gb[g] = gb[g];
    st.off[g] = o;
    const uint32_t n32 = (gb[g + 1] - gb[g]) / kBlkPerK;
    o += g < kNumQGroups ? (n32 + 1) / 2 : n32;
  }
  st.gb[kNumGroups] = gb[kNumGroups];
  st.off[kNumGroups] = o;
  return st;
}

// Blocks per step of group g: 16 (64 slots) for 1..8 bits, 8 for 16 bits.
__host__ __device__ constexpr uint32_t step_blocks(int g) {
  return g < kNumQGroups ? 2u * kBlkPerK : (uint32_t)kBlkPerK;
}

// First word of step i inside a segment record (the record's end for i at
// or beyond the step count); consecutive steps are contiguous in words.
// (Every per-group value is read with a compile-time index: a run-time
// index would place the arrays in scratch memory.)
__device__ __forceinline__ uint32_t step_word(const SegProj& p, const Steps& st, uint32_t i) {
  uint32_t b = p.n_blk;
#pragma unroll
  for (int g = 0; g < kNumGroups; ++g)
    if (i >= st.off[g] && i < st.off[g + 1]) b = st.gb[g] + (i - st.off[g]) * step_blocks(g);
  return block_word(p, b);
}

// End of the batch of steps that starts at step i0: at most kUBatch steps
// whose words fit the arena (one step is at most 512 words).
__device__ __forceinline__ uint32_t batch_end(const SegProj& p, const Steps& st, uint32_t i0) {
  const uint32_t n = st.off[kNumGroups];
  if (i0 >= n) return n;
  uint32_t i1 = min(n, i0 + (uint32_t)kUBatch);
  const uint32_t w0 = step_word(p, st, i0);
  while (i1 > i0 + 1 && step_word(p, st, i1) - w0 > (uint32_t)kUArena) --i1;
  return i1;
}

__device__ __forceinline__ uint32_t batch_count(const SegProj& p, const Steps& st) {
  uint32_t nb = 0;
  for (uint32_t i = 0; i < st.off[kNumGroups]; i = batch_end(p, st, i)) ++nb;
  return nb;
}

// Copy the words of steps [i0, i1) of segment sg into the arena (nl lanes).
__device__ __forceinline__ void stage_steps(uint32_t* arena, const SegProj& p, const Steps& st,
                                            int sg, uint32_t i0, uint32_t i1, int lp, int lane,
                                            int nl) {
  if (i1 <= i0) return;
  const uint32_t w0 = step_word(p, st, i0), w1 = step_word(p, st, i1);
  stage16(arena, p.planes + (size_t)sg * p.seg_words + w0, (w1 - w0) / 4u, lp, lane, nl);
}

// A operands of step i (of group G) for this lane (tile 0: rows 0-15,
// tile 1: rows 16-31), decoded from the staged words (base: word 0 of the
// segment record relative to the arena).  1..8-bit groups: the int8 code
// bytes of the lane's 4 blocks (a_i8, width 8 as code - 128), zero in the
// absent half of a half step; 16-bit group: the fp16 values of the lane's 2
// blocks.  bs, ws: the group's first block and first word.
template <int G>
__device__ __forceinline__ void decode_group_step(const Steps& st, uint32_t i, uint32_t bs,
                                                  uint32_t ws, const uint32_t* base, int lane,
                                                  i32x4& a0, i32x4& a1) {
  const uint32_t b = st.gb[G] + (i - st.off[G]) * step_blocks(G);
  const int m = lane & 15, q = lane >> 4;
  if constexpr (G == kNumGroups - 1) {
    h8 h0, h1;
    a_tiles_f16(base + ws + (b + 2u * (uint32_t)q - bs) * 64u, m, h0, h1);
    a0 = __builtin_bit_cast(i32x4, h0);
    a1 = __builtin_bit_cast(i32x4, h1);
  } else {
    constexpr int W = G < 4 ? G + 1 : (G == 4 ? 6 : 8);
    const i32x4 zero = {0, 0, 0, 0};
    a0 = zero;
    a1 = zero;
    const uint32_t lb = b + 4u * (uint32_t)q;  // the lane's first block
    if (lb < st.gb[G + 1]) {                   // (absent half of a half step)
      const uint32_t* rec = base + ws + (lb - bs) * 4u * W;
      a0 = a_i8<W>(rec, m, 0);
      a1 = a_i8<W>(rec, m, 1);
    }
  }
}

__device__ __forceinline__ void decode_step(const SegProj& p, const Steps& st, uint32_t i,
                                            const uint32_t* base, int lane, i32x4& a0,
                                            i32x4& a1) {
  if (i < st.off[1]) decode_group_step<0>(st, i, 0u, 0u, base, lane, a0, a1);
  else if (i < st.off[2]) decode_group_step<1>(st, i, p.b1, p.w1, base, lane, a0, a1);
  else if (i < st.off[3]) decode_group_step<2>(st, i, p.b2, p.w2, base, lane, a0, a1);
  else if (i < st.off[4]) decode_group_step<3>(st, i, p.b3, p.w3, base, lane, a0, a1);
  else if (i < st.off[5]) decode_group_step<4>(st, i, p.b4, p.w4, base, lane, a0, a1);
  else if (i < st.off[6]) decode_group_step<5>(st, i, p.b5, p.w5, base, lane, a0, a1);
  else decode_group_step<6>(st, i, p.b6, p.w6, base, lane, a0, a1);
}

// The MFMAs of step i with the A operands of its register slot: B is the
// digit rows (1..8-bit steps; lanes of columns >= 4 and of an absent half
// use zeros) or the hi and lo rows (16-bit steps, columns 0 and 1).
__device__ __forceinline__ void apply_step(const Steps& st, uint32_t i, const int8_t* lb,
                                           const _Float16* hh, const _Float16* hl, int lane,
                                           const i32x4& a0, const i32x4& a1, i32x4& acc_0,
                                           i32x4& acc_1, f4& acc16_0, f4& acc16_1) {
  const int m = lane & 15, q = lane >> 4;
  if (i >= st.off[kNumGroups - 1]) {
    const uint32_t so = 32u * (i - st.off[kNumGroups - 1]) + 8u * (uint32_t)q;
    uint4 bv = make_uint4(0, 0, 0, 0);
    if (m == 0) bv = *reinterpret_cast<const uint4*>(hh + so);
    if (m == 1) bv = *reinterpret_cast<const uint4*>(hl + so);
    const h8 bb = h8_of(bv);
    acc16_0 = mfma(__builtin_bit_cast(h8, a0), bb, acc16_0);
    acc16_1 = mfma(__builtin_bit_cast(h8, a1), bb, acc16_1);
    return;
  }
  // the step's first block and its group's end block
  uint32_t b = 0, be = 0;
#pragma unroll
  for (int g = 0; g < kNumQGroups; ++g)
    if (i >= st.off[g] && i < st.off[g + 1]) {
      b = st.gb[g] + (i - st.off[g]) * step_blocks(g);
      be = st.gb[g + 1];
    }
  const uint32_t lbk = b + 4u * (uint32_t)q;
  i32x4 bv = {0, 0, 0, 0};
  if (m < kDigits && lbk < be)
    bv = *reinterpret_cast<const i32x4*>(lb + (m & 3) * kUSlots + 4u * lbk);
  acc_0 = mfma_i8(a0, bv, acc_0);
  acc_1 = mfma_i8(a1, bv, acc_1);
}

__device__ __forceinline__ SegProj unit_seg(const uint8_t* blob, uint64_t bytes, int e,
                                            const GateUpArgs& a) {
  return uniform_seg(
      make_seg(blob, bytes, e, load_rec_s(blob, e, a.E), load_hdr(blob), a.E, a.dout, a.r));
}

// v = rint(c 2^S), kept within |v| < 2^30 (the scale bound guarantees it for
// a well-formed blob; the clamp keeps a malformed bound from overflowing).
__device__ __forceinline__ int coef_int(float c, int S) {
  const float f = ldexpf(c, S);
  return (int)rintf(fminf(fmaxf(f, -1073741760.f), 1073741760.f));
}

__global__ __launch_bounds__(kUThreads) void k_gateup_unit(FusedArgs s) {
  extern __shared__ __align__(16) uint8_t lds_raw[];
  UnitLds& L = *reinterpret_cast<UnitLds*>(lds_raw);
  const GateUpArgs& a = s.g;
  const int lane = threadIdx.x & (kWave - 1);
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int pj = wv >= kUPW ? 1 : 0;  // waves 0-3 gate, 4-7 up
  const int wp = wv & (kUPW - 1);
  const int lp = (int)threadIdx.x & (kUProj - 1);
  const int R = 2 * a.r;
  const int np = a.npairs;
  const int u = (int)blockIdx.x;
  const bool have = u < np * a.n_seg;  // uniform
  const int pair = u % np, sg = u / np, t = pair / a.ktop;
  typedef __attribute__((address_space(4))) const uint32_t CU32;
  // The routed id and the epoch are read first (scalar loads, ahead of the
  // Phi^T stream); the epoch changes only between launches.
  const int e = have ? (int)*(CU32*)(a.ids + pair) : 0;
  const uint32_t tag = *(CU32*)s.epoch + 1u;
  uint64_t* const zt = s.zt + (size_t)(tag % kZRing) * s.T * 2 * a.r;
  const int nzw = s.grid * kUPW;        // producing waves
  const int nrw = (R + nzw - 1) / nzw;  // rows per producing wave
  const int n0 = (u * kUPW + wp) * nrw;

  // ---- before z: loads, z production (waves 0-3), staging (waves 4-7) ----
  // (structures are built per branch, never picked from two by a run-time
  // condition: that would place them in scratch memory)
  SlotMeta<kUSper> md;  // this wave's projection
  SegProj P;            // this wave's projection (uniform)
  uint32_t nb_other;    // register batches of the other projection
  if (pj == 0) {
    PhiRegs phr;
    phi_issue(s, n0, nrw, lane, phr);
    if (have) {
      P = unit_seg(a.blob_g, a.bytes_g, e, a);
      load_meta<kUSper>(P, lp, md);  // straight-line: z below waits for Phi^T only
    }
    z_finish(s, zt, n0, nrw, lane, tag, phr);
    hint_add(s, u * kUPW + wp, lane);
    if (!have) return;
    const SegProj PO = unit_seg(a.blob_u, a.bytes_u, e, a);
    nb_other = batch_count(PO, make_steps(PO));
  } else {
    if (!have) return;
    // warm this XCD's L2 with both directories (the first 256 lines): the
    // record loads after the routed id then hit L2.  One 4-byte copy per
    // lane into the digit rows, which nothing uses before these copies have
    // been waited for (below).
    typedef __attribute__((address_space(1))) void gvoid;
    const uint32_t nl = ((uint32_t)a.E * kDirRecBytes + 127u) / 128u;
    uint32_t j = (uint32_t)threadIdx.x - kUProj;
    j = j < 2u * nl ? j : 2u * nl - 1u;
    const uint8_t* line =
        (j < nl ? a.blob_g : a.blob_u) + kHeaderBytes + 128u * (j < nl ? j : j - nl);
    __builtin_amdgcn_global_load_lds(
        (gvoid*)line,
        (lds_void*)(reinterpret_cast<uint8_t*>(&L.Lb[0][0][0]) + 256 * (wv - kUPW)), 4, 0, 0);
    P = unit_seg(a.blob_u, a.bytes_u, e, a);
    {
      // waves 4-5 copy the gate record's first batch, waves 6-7 the up one's
      const bool up = (wv & 2) != 0;
      const SegProj SP = unit_seg(up ? a.blob_u : a.blob_g, up ? a.bytes_u : a.bytes_g, e, a);
      const Steps SS = make_steps(SP);
      stage_steps(&L.W[up ? 1 : 0][0], SP, SS, sg, 0u, batch_end(SP, SS, 0u),
                  (int)threadIdx.x & 127, lane, 128);
    }
    load_meta<kUSper>(P, lp, md);
    const SegProj PO = unit_seg(a.blob_g, a.bytes_g, e, a);
    nb_other = batch_count(PO, make_steps(PO));
    __builtin_amdgcn_s_waitcnt(0);  // staged words (and the prefetch) landed
  }
  lds_sync();  // #1: batch 0 of both records is in LDS

  const Steps st = make_steps(P);
  const uint32_t nb = max(batch_count(P, st), nb_other);
  uint32_t i1 = batch_end(P, st, 0u);

  // ---- decode batch 0 into registers (z not needed) ----
  // (the register slots are written out one by one: a loop over them, which
  // the compiler may keep rolled, would place the operands in scratch memory)
  i32x4 A0[kUSlot], A1[kUSlot];
#define UNIT_DECODE(q)                                                     \
  if (4u * (q) + (uint32_t)wp < i1)                                        \
    decode_step(P, st, 4u * (q) + (uint32_t)wp, &L.W[pj][0], lane, A0[q], A1[q]);
  UNIT_SLOTS(UNIT_DECODE)
#undef UNIT_DECODE
  // coefficient inputs: k, w = a s (a for 16-bit slots), a m
  uint32_t kk[kUSper];
  float cw[kUSper], cam[kUSper];
  bool good = P.ok;
#pragma unroll
  for (int i = 0; i < kUSper; ++i) {
    uint32_t k;
    float av, sv, mv;
    meta_get<kUSper>(md, lp, i, P.n_slot, P.n_qslot, k, av, sv, mv);
    good &= k < (uint32_t)a.r;
    kk[i] = k < (uint32_t)a.r ? k : 0u;
    cw[i] = av * sv;
    cam[i] = av * mv;
  }

  // ---- z of the unit's token ----
  if (wv == 0) wait_hint(s.hint, tag * (uint32_t)nzw, s.spin);
  lds_sync();  // #2
  {
    float zmx;
    const bool zok = __all(stage_z<kUThreads, kUZPer>(zt + (size_t)t * R, R, tag, &L.Z[0], s.spin,
                                                      zmx));
    zmx = wave_max_dpp(zmx);
    if (lane == 0) {
      L.zok[wv] = zok;
      L.wmax[wv] = zmx;
    }
  }
  lds_sync();  // #3: L.Z and the maxima complete

  // ---- coefficients ----
  float zm = L.wmax[0];
#pragma unroll
  for (int w = 1; w < kUWaves; ++w) zm = fmaxf(zm, L.wmax[w]);
  const int S = digit_shift(P.cmax * zm);  // |a s z| 2^S < 2^30
  {
    const float* zrow = &L.Z[pj ? a.r : 0];
    float zv[kUSper];
#pragma unroll
    for (int i = 0; i < kUSper; ++i) zv[i] = zrow[kk[i]];
    const uint32_t e8a = 4u * P.b5, s16 = 4u * P.b6, ns = P.n_slot;
    float bias = 0.f, corr = 0.f;
    uint32_t wd[8];
#pragma unroll
    for (int i = 0; i < kUSper; ++i) {
      const uint32_t sl = meta_slot<kUSper>(lp, i);
      const float c = cw[i] * zv[i];
      bias += cam[i] * zv[i];  // m = 0 for 16-bit and padding slots
      const int vi = coef_int(c, S);
      corr += (sl >= e8a && sl < s16) ? (float)vi : 0.f;
      if (sl >= s16 && sl < ns) {
        const float hv = ldexpf(c, S - 16);
        const _Float16 hi = (_Float16)hv;
        L.H[pj][0][sl - s16] = hi;
        L.H[pj][1][sl - s16] = (_Float16)(hv - (float)hi);
      }
      if (i < 8) {
        wd[i] = digit_bytes(vi);
      } else {
        const uint32_t wt = digit_bytes(vi);
#pragma unroll
        for (int l = 0; l < kDigits; ++l) L.Lb[pj][l][sl] = (int8_t)(wt >> (8 * l));
      }
    }
    uint32_t r0[4], r1[4];
    transpose4(wd[0], wd[1], wd[2], wd[3], r0);
    transpose4(wd[4], wd[5], wd[6], wd[7], r1);
#pragma unroll
    for (int l = 0; l < kDigits; ++l)
      *reinterpret_cast<uint2*>(&L.Lb[pj][l][8 * lp]) = make_uint2(r0[l], r1[l]);
    bias = wave_sum_dpp(bias);
    corr = wave_sum_dpp(corr);
    const bool wok = __all(good);
    if (lane == 0) {
      L.pbias[pj][wp] = bias;
      L.pcorr[pj][wp] = ldexpf(128.f * corr, -S);
      L.pok[pj][wp] = wok ? 1u : 0u;
    }
  }
  lds_sync();  // #4: digit rows and hi/lo rows complete

  // ---- apply ----
  i32x4 acc_0 = {0, 0, 0, 0}, acc_1 = {0, 0, 0, 0};  // column n: digit n
  f4 acc16_0 = {0.f, 0.f, 0.f, 0.f}, acc16_1 = {0.f, 0.f, 0.f, 0.f};  // columns: hi, lo
  const int8_t* lbp = &L.Lb[pj][0][0];
  const _Float16* hh = &L.H[pj][0][0];
  const _Float16* hl = &L.H[pj][1][0];
#define UNIT_APPLY(q)                                                                  \
  if (4u * (q) + (uint32_t)wp < i1)                                                    \
    apply_step(st, 4u * (q) + (uint32_t)wp, lbp, hh, hl, lane, A0[q], A1[q], acc_0, acc_1, \
               acc16_0, acc16_1);
  UNIT_SLOTS(UNIT_APPLY)
#undef UNIT_APPLY
  // records beyond one batch: staged, decoded and applied a batch at a time
  for (uint32_t bt = 1; bt < nb; ++bt) {
    const uint32_t i0 = i1;
    i1 = batch_end(P, st, i0);
    lds_sync();  // every wave is done with the arena
    stage_steps(&L.W[pj][0], P, st, sg, i0, i1, lp, lane, kUProj);
    __builtin_amdgcn_s_waitcnt(0);
    lds_sync();
    const uint32_t* base = &L.W[pj][0] - (i0 < i1 ? step_word(P, st, i0) : 0u);
#pragma unroll
    for (int q = 0; q < kUSlot; ++q) {
      const uint32_t i = i0 + 4u * q + (uint32_t)wp;
      if (i < i1) {
        i32x4 t0, t1;
        decode_step(P, st, i, base, lane, t0, t1);
        apply_step(st, i, lbp, hh, hl, lane, t0, t1, acc_0, acc_1, acc16_0, acc16_1);
      }
    }
  }

  // ---- row sums of the 4 waves, SiLU * mul ----
  {
    // lane (n, quarter) holds column n of rows 4 quarter .. + 3; integer
    // column n is worth 2^(8 n - S), fp16 columns 0, 1 2^(16 - S); a quad
    // sum leaves each row's total in column 0
    const int n = lane & 15, kg = lane >> 4;
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2) {
      const i32x4& ai = t2 ? acc_1 : acc_0;
      const f4& a16 = t2 ? acc16_1 : acc16_0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float v = (n < kDigits ? ldexpf((float)ai[i], 8 * n - S) : 0.f) +
                  (n < 2 ? ldexpf(a16[i], 16 - S) : 0.f);
        v += dpp_move<0xB1>(v, 0.f);  // quad_perm [1,0,3,2]
        v += dpp_move<0x4E>(v, 0.f);  // quad_perm [2,3,0,1]
        if (n == 0) L.red[pj][wp][16 * t2 + 4 * kg + i] = v;
      }
    }
  }
  lds_sync();  // #5
  if (wv == 0 && lane < kSegRows) {
    // every flag read first and combined without branches
    float ys[2];
    uint32_t okw = 1u;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      float sum = 0.f, bsum = 0.f;
#pragma unroll
      for (int w = 0; w < kUPW; ++w) {
        sum += L.red[q][w][lane] + L.pcorr[q][w];
        bsum += L.pbias[q][w];
        okw &= L.pok[q][w];
      }
      ys[q] = sum + bsum;
    }
#pragma unroll
    for (int w = 0; w < kUWaves; ++w) okw &= L.zok[w];
    const int row = sg * kSegRows + lane;
    if (row < a.dout)
      a.h[(size_t)pair * a.dout + row] = okw ? silu_mul(ys[0], ys[1]) : __builtin_nanf("");
  }

  // Work-group 0 advances the epoch once every producing wave has counted
  // itself: by then every work-group has read the old epoch (its tag is in
  // its registers), and the next launch reads the new one.  (Waited for
  // with the default bound also when a test lowered the launch's bound.)
  if (blockIdx.x == 0 && wv == 0) {
    wait_hint(s.hint, tag * (uint32_t)nzw, max(s.spin, kSpinDefault));
    if (lane == 0) __hip_atomic_store(s.epoch, tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

}  // namespace

size_t unit_lds_bytes() { return sizeof(UnitLds); }

int unit_grid() {
  static int grid[64];
  static bool done[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  if (!done[dev]) {
    int cus = 0, nb = 0;
    (void)hipFuncSetAttribute((const void*)k_gateup_unit,
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)sizeof(UnitLds));
    (void)hipGetLastError();
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, k_gateup_unit, kUThreads,
                                                     sizeof(UnitLds)) != hipSuccess)
      return 0;
    // one group per compute unit, all resident at once, a multiple of 8
    grid[dev] = (nb >= 1 && cus >= 8) ? (cus & ~7) : 0;
    done[dev] = true;
  }
  return grid[dev];
}

void launch_gateup_unit(const FusedArgs& s, hipStream_t st) {
  hipLaunchKernelGGL(k_gateup_unit, dim3((unsigned)s.grid), dim3(kUThreads), sizeof(UnitLds), st,
                     s);
}

}  // namespace bitsmoe
