// One-launch gate/up kernel for a few tokens: z = Phi^T x is produced inside
// the launch, then one 512-lane work-group per (token, slot, 32-row segment)
// unit applies both projections with MFMA and writes SiLU(gate) * up.
//
// BitsMoE blog note, Methodology: "first split" (z = Phi^T x once per token,
// reused by every routed expert), "second split" (an expert's output is the
// sum over components of magnitude * z_k * quantized unit direction) and
// "execution" (components of one width stored together, plane by plane).
//
// gfx950 mapping.
//  * Units u = segment * pairs + pair go to XCD u % 8 (work-group b runs on
//    XCD b % 8 and takes units b, b + G, ...); with 8 or more pairs every
//    segment of a pair sits on one XCD, whose L2 then serves the pair's
//    column metadata to all of them.
//  * Waves 0-3 of every work-group issue the loads of their run of Phi^T
//    rows first (nothing they depend on), compute z for them
//    (v_dot2_f32_f16, a transposing 4-row reduction) and publish each value
//    as one 64-bit word (float bits | launch tag << 32) into a ring of 8
//    buffers (the tag picks one), then add one to a hint counter without
//    waiting for the stores.  The counters are cumulative over launches: after
//    the launch with tag g their sum is g times the number of producing waves.
//  * Waves 4-7 meanwhile read the routed id and the two directory records
//    (scalar loads), issue the raw slot metadata of both projections (16-byte
//    loads kept in registers) and copy the unit's gate and up segment records
//    into LDS with 16-byte global_load_lds; wave 4 publishes the descriptors.
//  * One wave polls the hint counters; then the token's 2r tagged words are
//    copied into LDS (an L2-shared read; a word whose tag is stale is re-read
//    device-coherently, bounded).
//  * Coefficients: waves 4-7 form c = a s z (a z for 16-bit slots) and a m z
//    for both projections and write c into LDS; then all eight waves split
//    their projection's c into v = rint(c 2^S) (S from the largest |c| of the
//    1..8-bit slots, S16 for the 16-bit ones) and store its four balanced
//    base-256 digit bytes as digit rows.
//  * Apply: per 64-slot step one v_mfma_i32_16x16x64_i8 per 16-row tile, the
//    decoded code bytes as A (width 8 as code - 128) and the digit rows as B
//    columns 0-3, so every product and sum is exact in int32; the 16-bit
//    group uses v_mfma_f32_16x16x32_f16 with the fp16 hi and lo parts of
//    v 2^-16 in columns 0 and 1.  Each wave of a projection takes every 4th
//    step.
//  * Epilogue: the columns are folded with 2^(8n - S) (2^(16 - S16)), the
//    four waves' row sums meet in LDS, and wave 0 adds the width-8 offset
//    correction and the row-independent sum a m z and writes SiLU(gate) * up.
// Segments whose record exceeds the LDS arena are applied in chunks of K
// steps.  Work-groups wait for other groups' z, so the host launches at most
// as many groups as can be resident at once; all waits are bounded (a
// time-out gives NaN rows, the kernel still exits).  Work-group 0 advances
// the epoch once every producer of the launch has counted itself.  Barriers
// order LDS only (lds_sync): the staging copies are waited for explicitly
// where their data is needed.
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

constexpr int kFWaves = 8;
constexpr int kFThreads = kFWaves * kWave;  // 512
constexpr int kFProj = 256;                 // lanes per projection (waves 0-3 gate, 4-7 up)
constexpr int kFPW = kFWaves / 2;           // waves per projection
constexpr int kFMaxW = 10240;               // plane words per projection per chunk
constexpr int kFMaxS = 4320;                // slots per projection (r <= 4096, padded)
// slots per lane of the coefficient pass: 9 covers r <= 2048, 17 r <= 4096

constexpr int kFZ = 2 * kFusedMaxR;         // z values of one token (gate, up)
constexpr int kFZPer = kFZ / kFThreads;     // tagged z words per lane

struct __align__(16) FusedLds {
  uint32_t W[2][kFMaxW + 64];
  float Z[kFZ];
  int8_t Lb[2][kDigits][kFMaxS];  // coefficient digits per projection (v = sum 2^(8 l) d_l)
  float red[2][kFPW][kSegRows];
  float pmax[2][kFPW];    // largest |c| of 1..8-bit slots
  float pmax16[2][kFPW];  // largest |c| of 16-bit slots
  float pbias[2][kFPW];
  float pcorr[2][kFPW];  // 128 * sum of v 2^-S over width-8 slots (those enter as code - 128)
  uint32_t pok[2][kFPW];
  int nch[2];
  uint32_t zok[kFWaves];  // each wave's staged z words arrived
  SegProj desc[2];  // the unit's gate and up descriptors (written by wave 4)
};

// Stage chunk [b0, b1) of segment sg of projection p into arena (nl lanes).
__device__ __forceinline__ void stage_chunk(uint32_t* arena, const SegProj& p, int sg,
                                            uint32_t b0, uint32_t b1, int lp, int lane, int nl) {
  if (b1 <= b0) return;
  const uint32_t w0 = block_word(p, b0), w1 = block_word(p, b1);
  stage16(arena, p.planes + (size_t)sg * p.seg_words + w0, (w1 - w0) / 4u, lp, lane, nl);
}

template <int kFSper>
__global__ __launch_bounds__(kFThreads) void k_gateup_fused(FusedArgs s) {
  extern __shared__ __align__(16) uint8_t lds_raw[];
  FusedLds& L = *reinterpret_cast<FusedLds*>(lds_raw);
  const GateUpArgs& a = s.g;
  const int lane = threadIdx.x & (kWave - 1);
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // The epoch changes only between launches (the previous launch's last
  // group wrote it), so a scalar load sees it; unlike a vector load it does
  // not hold up the Phi^T loads behind it.
  typedef __attribute__((address_space(4))) const uint32_t CU32;
  const uint32_t tag = *(CU32*)s.epoch + 1u;
  // this launch's tagged z buffer: a line that an XCD's L2 still holds from
  // the launch kZRing launches back carries an old tag and is re-read
  uint64_t* const zt = s.zt + (size_t)(tag % kZRing) * s.T * 2 * a.r;
  const int pj = wv >= kFPW ? 1 : 0;           // waves 0-3 gate, 4-7 up
  const int wp = wv & (kFPW - 1);
  const int lp = (int)threadIdx.x & (kFProj - 1);
  const int R = 2 * a.r;
  const int G = s.grid;
  const int np = a.npairs;
  const int U = np * a.n_seg;

  const int nzw = G * kFPW;              // producing waves
  const int nrw = (R + nzw - 1) / nzw;   // rows per producing wave
  const int n0 = ((int)blockIdx.x * kFPW + wp) * nrw;

  // ---- prologue ----
  // Waves 0-3 issue their Phi^T rows at once and produce z, touching nothing
  // else until it is published; the unit's loads are all made by waves 4-7
  // (below), which need them only once z has been exchanged.
  int u = (int)blockIdx.x;
  bool have = u < U;
  if (pj == 0) {
    // (the r > 2048 instantiation keeps whole rows of up to 4096 inputs in
    // registers; the other keeps its first 2048)
    constexpr int kNU = kFSper > 9 ? 8 : 4;
    PhiRegs<kNU> phr;
    phi_issue<kNU>(s, n0, nrw, lane, phr);
    z_finish<kNU>(s, zt, n0, nrw, lane, tag, phr);
    // (the hint may run ahead of the z stores: a reader that comes too early
    // finds old tags and re-reads those words)
    hint_add(s, (int)blockIdx.x * kFPW + wp, lane);
  }

  if (pj == 1) {
    // Warm this XCD's L2 with both directories (128-byte lines; the first
    // 256 of them): the record loads that follow the routed id then hit L2
    // instead of queueing behind the Phi^T loads.  One unconditional 4-byte
    // copy per lane into the digit-table area, which nothing reads before
    // these copies have been waited for (the coefficient pass waits for all
    // of the wave's loads first).
    typedef __attribute__((address_space(1))) void gvoid;
    const uint32_t nl = ((uint32_t)a.E * kDirRecBytes + 127u) / 128u;  // lines per projection
    uint32_t j = (uint32_t)threadIdx.x - kFProj;
    j = j < 2u * nl ? j : 2u * nl - 1u;
    const uint8_t* line = (j < nl ? a.blob_g : a.blob_u) + kHeaderBytes + 128u * (j < nl ? j : j - nl);
    __builtin_amdgcn_global_load_lds((gvoid*)line,
                                     (lds_void*)(reinterpret_cast<uint8_t*>(&L.Lb[0][0][0]) +
                                                 256 * (wv - kFPW)),
                                     4, 0, 0);
  }
  int zt_cached = -1;  // token whose z is in L.Z
  // pair whose digit tables, scales and offset sums are in LDS: the units
  // of a work-group (b, b + G, ...) share one pair whenever the grid is a
  // multiple of the pair count, and then the coefficient pass runs once
  // (long slot lists, where a work-group has many units)
  int coef_pair = -1;
  bool zok = true;     // this wave's words of L.Z arrived
  for (; have; u += G, have = u < U) {
    const int pair = u % np;
    // (the r <= 2048 instantiation keeps its one-unit code unchanged: there
    // the extra branches cost more than they save)
    const bool reuse = kFSper > 9 && pair == coef_pair;  // uniform
    const int sg = u / np;
    const int t = pair / a.ktop;
    // kBoth: waves 4-7 form the coefficients of both projections; otherwise
    // (long slot lists: too many registers) each half forms its own, waves
    // 0-3 loading the gate metadata after the descriptors are published.
    constexpr bool kBoth = kFSper <= 9;
    constexpr int V = SlotMeta<kFSper>::V;
    SlotMeta<kFSper> md0, md1;  // kBoth: gate, up; otherwise md0 is this wave's projection
    bool ok0 = true, ok1 = true;
    uint32_t ns0 = 0, nq0 = 0, ns1 = 0, nq1 = 0;  // n_slot, n_qslot of md0, md1
    if (pj == 1) {
      // routed id -> both directory records (scalar loads) -> slot metadata,
      // staging copies (waves 4-5 gate, 6-7 up) and the descriptors in LDS
      const int e = (int)*(CU32*)(a.ids + pair);
      const DirRec rg = load_rec_s(a.blob_g, e, a.E);
      const DirRec ru = load_rec_s(a.blob_u, e, a.E);
      const HdrF hg = load_hdr(a.blob_g), hu = load_hdr(a.blob_u);
      const SegProj PG = uniform_seg(make_seg(a.blob_g, a.bytes_g, e, rg, hg, a.E, a.dout, a.r));
      const SegProj PU = uniform_seg(make_seg(a.blob_u, a.bytes_u, e, ru, hu, a.E, a.dout, a.r));
      if (kBoth) {
        ok0 = PG.ok;
        ok1 = PU.ok;
        ns0 = PG.n_slot; nq0 = PG.n_qslot;
        ns1 = PU.n_slot; nq1 = PU.n_qslot;
        if (!reuse) {
          load_meta<kFSper>(PG, lp, md0);
          load_meta<kFSper>(PU, lp, md1);
        }
      } else {
        ok0 = PU.ok;
        ns0 = PU.n_slot; nq0 = PU.n_qslot;
        if (!reuse) load_meta<kFSper>(PU, lp, md0);
      }
      const SegProj& SP = (wv & 2) ? PU : PG;
      stage_chunk(&L.W[(wv >> 1) & 1][0], SP, sg, 0, chunk_end(SP, 0, kFMaxW),
                  (int)threadIdx.x & 127, lane, 128);
      if (wv == kFPW && lane == 0) {
        L.desc[0] = PG;
        L.desc[1] = PU;
        int nc = 0;
        for (uint32_t b = 0; b < PG.n_blk; b = chunk_end(PG, b, kFMaxW)) ++nc;
        L.nch[0] = nc;
        nc = 0;
        for (uint32_t b = 0; b < PU.n_blk; b = chunk_end(PU, b, kFMaxW)) ++nc;
        L.nch[1] = nc;
      }
    }
    if (!kBoth) {
      // waves 0-3 load the gate metadata themselves: descriptors first
      lds_sync();
      if (pj == 0) {
        const SegProj PG = uniform_seg(L.desc[0]);
        ok0 = PG.ok;
        ns0 = PG.n_slot; nq0 = PG.n_qslot;
        if (!reuse) load_meta<kFSper>(PG, lp, md0);
      }
    }
    if (t != zt_cached) {
      // one wave polls the hint counters (the first time only), the rest wait
      if (zt_cached < 0 && wv == 0) (void)wait_hint(s.hint, tag * (uint32_t)nzw, s.spin);
      lds_sync();
      float zmx;
      zok = stage_z<kFThreads, kFZPer>(zt + (size_t)t * R, R, tag, &L.Z[0], s.spin, zmx);
      zok = __all(zok);
      count_timeout(s, !zok, lane);
      if (lane == 0) L.zok[wv] = zok;  // every wave's words: combined in the epilogue
      lds_sync();                  // L.Z complete
      zt_cached = t;
    }
    SegProj P;  // this wave's projection
    if (!reuse) {
    // ---- coefficients ----
    // (kBoth: waves 4-7 do projection 0 = gate from md0 and 1 = up from md1;
    // otherwise every wave does its own projection pj from md0).  All the
    // z gathers from LDS are issued before any is used.
    constexpr int kNQ = kBoth ? 2 : 1;
    float cv[kNQ][kFSper];
    if (!kBoth || pj == 1) {
      uint32_t kk[kNQ][kFSper];
      float av[kNQ][kFSper], sv[kNQ][kFSper], mv[kNQ][kFSper], zv[kNQ][kFSper];
      bool good[kNQ];
#pragma unroll
      for (int j = 0; j < kNQ; ++j) {
        const SlotMeta<kFSper>& md = j ? md1 : md0;
        const uint32_t ns = j ? ns1 : ns0, nq = j ? nq1 : nq0;
        good[j] = (j ? ok1 : ok0) && zok;
#pragma unroll
        for (int i = 0; i < kFSper; ++i) {
          meta_get<kFSper>(md, lp, i, ns, nq, kk[j][i], av[j][i], sv[j][i], mv[j][i]);
          good[j] &= kk[j][i] < (uint32_t)a.r;
          kk[j][i] = kk[j][i] < (uint32_t)a.r ? kk[j][i] : 0u;
        }
      }
#pragma unroll
      for (int j = 0; j < kNQ; ++j) {
        const int q = kBoth ? j : pj;
        const float* zrow = &L.Z[q ? a.r : 0];
#pragma unroll
        for (int i = 0; i < kFSper; ++i) zv[j][i] = zrow[kk[j][i]];
      }
#pragma unroll
      for (int j = 0; j < kNQ; ++j) {
        const int q = kBoth ? j : pj;
        const uint32_t nq = j ? nq1 : nq0;
        float bias = 0.f, cmx = 0.f, cmx16 = 0.f;
#pragma unroll
        for (int i = 0; i < kFSper; ++i) {
          const float az = av[j][i] * zv[j][i];
          bias += az * mv[j][i];          // m = 0 for 16-bit and padding slots
          const float c = az * sv[j][i];  // s = 1 for 16-bit slots
          cv[j][i] = c;
          if (meta_slot<kFSper>(lp, i) < nq)
            cmx = fmaxf(cmx, fabsf(c));
          else
            cmx16 = fmaxf(cmx16, fabsf(c));
        }
        cmx = wave_max_dpp(cmx);
        cmx16 = wave_max_dpp(cmx16);
        const float bw = wave_sum_dpp(bias);
        const bool wok = __all(good[j]);
        if (kBoth) {
          // the coefficients go through LDS (the digit table's space, as
          // floats) so that all eight waves split them, each its own
          // projection
          float* cz = reinterpret_cast<float*>(&L.Lb[q][0][0]);
#pragma unroll
          for (int v = 0; v < V; ++v) {
            const uint32_t sv = 8u * V * (uint32_t)lp + 8u * v;
            *reinterpret_cast<float4*>(cz + sv) =
                make_float4(cv[j][8 * v], cv[j][8 * v + 1], cv[j][8 * v + 2], cv[j][8 * v + 3]);
            *reinterpret_cast<float4*>(cz + sv + 4) =
                make_float4(cv[j][8 * v + 4], cv[j][8 * v + 5], cv[j][8 * v + 6], cv[j][8 * v + 7]);
          }
          cz[meta_slot<kFSper>(lp, 8 * V)] = cv[j][8 * V];
        }
        if (lane == 0) {
          L.pmax[q][wp] = cmx;
          L.pmax16[q][wp] = cmx16;
          L.pbias[q][wp] = bw;
          L.pok[q][wp] = wok;
        }
      }
    }
    lds_sync();
    // this wave's projection (wave 4 published the descriptors before any
    // barrier of this unit that came before this one)
    P = uniform_seg(L.desc[pj]);
    {
      float cq[kFSper];
      if (kBoth) {
        const float* cz = reinterpret_cast<const float*>(&L.Lb[pj][0][0]);
#pragma unroll
        for (int v = 0; v < V; ++v) {
          const uint32_t sv = 8u * V * (uint32_t)lp + 8u * v;
          const float4 c0 = *reinterpret_cast<const float4*>(cz + sv);
          const float4 c1 = *reinterpret_cast<const float4*>(cz + sv + 4);
          cq[8 * v] = c0.x; cq[8 * v + 1] = c0.y; cq[8 * v + 2] = c0.z; cq[8 * v + 3] = c0.w;
          cq[8 * v + 4] = c1.x; cq[8 * v + 5] = c1.y; cq[8 * v + 6] = c1.z; cq[8 * v + 7] = c1.w;
        }
        cq[8 * V] = cz[meta_slot<kFSper>(lp, 8 * V)];
        lds_sync();  // every wave has its coefficients before the digits overwrite them
      } else {
#pragma unroll
        for (int i = 0; i < kFSper; ++i) cq[i] = cv[0][i];
      }
      const float pmx =
          fmaxf(fmaxf(L.pmax[pj][0], L.pmax[pj][1]), fmaxf(L.pmax[pj][2], L.pmax[pj][3]));
      const float pmx16 =
          fmaxf(fmaxf(L.pmax16[pj][0], L.pmax16[pj][1]), fmaxf(L.pmax16[pj][2], L.pmax16[pj][3]));
      const int S = digit_shift(pmx), S16 = digit_shift(pmx16);
      const uint32_t nq = P.n_qslot, e8a = 4u * P.b5, e8b = 4u * P.b6;
      // digits of v = rint(c 2^S) (2^S16 for 16-bit slots; zeros past
      // n_slot; the tail slot can lie past the arrays), and the width-8
      // correction
      float corr = 0.f;
#pragma unroll
      for (int v = 0; v < V; ++v) {
        const uint32_t sv = 8u * V * (uint32_t)lp + 8u * v;
        uint32_t w[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int vi = (int)rintf(ldexpf(cq[8 * v + i], sv + i < nq ? S : S16));
          w[i] = digit_bytes(vi);
          corr += (sv + i >= e8a && sv + i < e8b) ? (float)vi : 0.f;
        }
        uint32_t r0[4], r1[4];
        transpose4(w[0], w[1], w[2], w[3], r0);
        transpose4(w[4], w[5], w[6], w[7], r1);
#pragma unroll
        for (int l = 0; l < kDigits; ++l)
          *reinterpret_cast<uint2*>(&L.Lb[pj][l][sv]) = make_uint2(r0[l], r1[l]);
      }
      const uint32_t sl = meta_slot<kFSper>(lp, 8 * V);
      if (sl < kFMaxS) {
        const int vi = (int)rintf(ldexpf(cq[8 * V], sl < nq ? S : S16));
        const uint32_t wt = digit_bytes(vi);
#pragma unroll
        for (int l = 0; l < kDigits; ++l) L.Lb[pj][l][sl] = (int8_t)(wt >> (8 * l));
        corr += (sl >= e8a && sl < e8b) ? (float)vi : 0.f;
      }
      corr = wave_sum_dpp(corr);
      if (lane == 0) L.pcorr[pj][wp] = ldexpf(128.f * corr, -S);
    }
    }  // !reuse
    coef_pair = pair;
    __builtin_amdgcn_s_waitcnt(0);
    lds_sync();
    if (reuse) P = uniform_seg(L.desc[pj]);  // published by wave 4 before this barrier
    const int nch = __builtin_amdgcn_readfirstlane(max(L.nch[0], L.nch[1]));  // uniform
    // ---- apply ----
    i32x4 acc_0 = {0, 0, 0, 0}, acc_1 = {0, 0, 0, 0};  // column n: digit n
    f4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};  // fp16 columns: hi, lo
    uint32_t b0 = 0;
    for (int ch = 0; ch < max(nch, 1); ++ch) {
      const uint32_t b1 = chunk_end(P, b0, kFMaxW);
      if (ch > 0) {
        lds_sync();  // every wave is done with the previous chunk
        stage_chunk(&L.W[pj][0], P, sg, b0, b1, lp, lane, kFProj);
        __builtin_amdgcn_s_waitcnt(0);
        lds_sync();
      }
      if (b1 > b0) {
        const uint32_t* base = &L.W[pj][0] - block_word(P, b0);
        i8_ksteps(P, base, &L.Lb[pj][0][0], kFMaxS, b0 / kBlkPerK,
                  (b1 + kBlkPerK - 1) / kBlkPerK, wp, lane, acc_0, acc_1, acc0, acc1);
      }
      b0 = b1;
    }
    // ---- row sums of the 4 waves, SiLU * mul ----
    {
      // fold the columns: lane (n, quarter) holds column n of rows 4 quarter
      // .. + 3; integer column n is worth 2^(8 n - S), fp16 columns 0, 1
      // 2^(16 - S16); a quad sum leaves each row's total in column 0
      const float mq = fmaxf(fmaxf(L.pmax[pj][0], L.pmax[pj][1]), fmaxf(L.pmax[pj][2], L.pmax[pj][3]));
      const float m16 =
          fmaxf(fmaxf(L.pmax16[pj][0], L.pmax16[pj][1]), fmaxf(L.pmax16[pj][2], L.pmax16[pj][3]));
      const int S = digit_shift(mq), S16 = digit_shift(m16);
      const int n = lane & 15, kg = lane >> 4;
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2) {
        const i32x4& ai = t2 ? acc_1 : acc_0;
        const f4& a16 = t2 ? acc1 : acc0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float v = (n < kDigits ? ldexpf((float)ai[i], 8 * n - S) : 0.f) +
                    (n < 2 ? ldexpf(a16[i], 16 - S16) : 0.f);
          v += dpp_move<0xB1>(v, 0.f);  // quad_perm [1,0,3,2]
          v += dpp_move<0x4E>(v, 0.f);  // quad_perm [2,3,0,1]
          if (n == 0) L.red[pj][wp][16 * t2 + 4 * kg + i] = v;
        }
      }
    }
    lds_sync();
    if (wv == 0 && lane < kSegRows) {
      // every flag read first and combined without branches (a short-circuit
      // && would wait for each LDS read in turn)
      float ys[2];
      uint32_t okw = 1u;
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        float sum = 0.f, bsum = 0.f;
#pragma unroll
        for (int w = 0; w < kFPW; ++w) {
          sum += L.red[q][w][lane] + L.pcorr[q][w];
          bsum += L.pbias[q][w];
          okw &= L.pok[q][w];
        }
        ys[q] = sum + bsum;
      }
#pragma unroll
      for (int w = 0; w < kFWaves; ++w) okw &= L.zok[w];
      const bool ok = okw != 0u;
      const int row = sg * kSegRows + lane;
      if (row < a.dout)
        a.h[(size_t)pair * a.dout + row] = ok ? silu_mul(ys[0], ys[1]) : __builtin_nanf("");
    }
    lds_sync();  // LDS is reused by the next unit
  }

  // Work-group 0 advances the epoch once every producing wave has counted
  // itself: by then every work-group has read the old epoch (its tag is in
  // its registers), and the next launch reads the new one.
  // (Waited for with the default bound also when a test lowered the
  // launch's bound.)
  if (blockIdx.x == 0 && wv == 0) {
    count_timeout(s, !wait_hint(s.hint, tag * (uint32_t)nzw, max(s.spin, kSpinDefault)), lane);
    if (lane == 0) __hip_atomic_store(s.epoch, tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

}  // namespace

size_t fused_lds_bytes() { return sizeof(FusedLds); }

int fused_grid() {
  static int grid[64];
  static bool done[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  if (!done[dev]) {
    int cus = 0, nb9 = 0, nb17 = 0;
    (void)hipFuncSetAttribute((const void*)k_gateup_fused<9>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)sizeof(FusedLds));
    (void)hipFuncSetAttribute((const void*)k_gateup_fused<17>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)sizeof(FusedLds));
    (void)hipGetLastError();
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb9, k_gateup_fused<9>, kFThreads,
                                                     sizeof(FusedLds)) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb17, k_gateup_fused<17>, kFThreads,
                                                     sizeof(FusedLds)) != hipSuccess)
      return 0;
    // one group per compute unit, all resident at once, a multiple of 8
    grid[dev] = (nb9 >= 1 && nb17 >= 1 && cus >= 8) ? (cus & ~7) : 0;
    done[dev] = true;
  }
  return grid[dev];
}

void launch_gateup_fused(const FusedArgs& s, hipStream_t st) {
  // slots per lane: n_slot <= r + 7 * 31 (each width group padded to 32 slots)
  if (s.g.r + 7 * 31 <= 9 * kFProj)
    hipLaunchKernelGGL(k_gateup_fused<9>, dim3((unsigned)s.grid), dim3(kFThreads),
                       sizeof(FusedLds), st, s);
  else
    hipLaunchKernelGGL(k_gateup_fused<17>, dim3((unsigned)s.grid), dim3(kFThreads),
                       sizeof(FusedLds), st, s);
}

}  // namespace bitsmoe
