// Route grouping and the grouped gate/up expert kernel (token batches).
//
// BitsMoE blog note, Methodology: "first split" (z = Phi^T x is computed once
// per token and reused by every expert the token is routed to), "second
// split" (expert output = sum over components of magnitude * z_k * quantized
// unit direction) and "execution" (components of one width stored together,
// plane by plane).  Grouping the batch's (token, slot) pairs by expert
// extends the first split's reuse across tokens: an expert's planes are read
// from HBM and unpacked once per tile of up to 16 routed tokens instead of
// once per token, and the tokens become the N columns of the MFMA.
//
// k_route_group (one work-group): the counting sort of the T*k pairs by
// expert id into tiles of at most 16 pairs (route.h), for expert counts
// beyond what the work-group added to the projection launch handles.
//
// k_group_coef: the coefficients of every tile, once per tile instead of
// once per row segment: c = a s z_t[k] (a z for 16-bit slots) of each of the
// tile's tokens as the fp16 hi + lo parts of c 2^S_t, S_t from the expert's
// bound max |a s| (directory) and the token's max |z| (partial maxima written
// by the projection launch), and the row-independent sums a m z per 256-slot
// chunk, into tables in the workspace.
//
// k_gateup_grouped: one 512-lane work-group per (group of up to kSuperTiles
// tiles of one expert, 32-row segment) unit, both projections (waves 0-3
// gate, 4-7 up): each K step's planes are decoded once and applied to every
// tile of the group (up to 16 kSuperTiles token columns).  Group x + 8 i runs on XCD x with its
// segment units one after another, so the segments of a group share one L2
// for its coefficient tables; blocks past the group count exit at once.  The segment records are staged in LDS in chunks of at most
// 7168 words per projection; each wave reads the B operands of its K steps
// (16 bytes a lane, two steps ahead) straight from the tile's coefficient
// tables, so a chunk's steps run without barriers.  The work-group's LDS
// stays under half of a CU's, so two units share a CU and each one's chain
// of dependent loads overlaps the other's products.  A one-projection mode
// (the down projection) gives each pair its own z and lets the two wave
// halves take two segments.
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include "device_common.h"
#include "format.h"
#include "kernels.h"
#include "route.h"
#include "seg_common.h"

namespace bitsmoe {
namespace {

using namespace seg;

// ------------------------------------------------------------ route groups
constexpr int kRThreads = 1024;

__global__ __launch_bounds__(kRThreads) void k_route_group(RouteJob j) {
  extern __shared__ uint32_t cnt[];  // E counters, then E cursors
  __shared__ uint32_t buf[kRThreads];
  route_lists<kRThreads>(j, cnt, buf);
}

// ------------------------------------------------------- grouped gate/up
constexpr int kGWaves = 8;
constexpr int kGThreads = kGWaves * kWave;  // 512
constexpr int kGProj = 256;                 // lanes per projection
constexpr int kGPW = kGWaves / 2;           // waves per projection
constexpr int kGMaxW = 7168;                // plane words per projection per chunk
constexpr int kGZP = 16;                    // lanes per token for the partial maxima
constexpr int kGZPer = 16;                  // partial maxima a lane loads at once (r <= 4096)
constexpr int kGBPer = 9;                   // chunk sums a lane loads up front (r <= 2048)

// Largest of zp[i], i = i0, i0 + kGZP, ... < i1 (all >= 0): the first kGZPer
// loads are all issued before any is used, so they cost one round trip, not
// one each.
__device__ __forceinline__ float strided_max(const float* zp, int i0, int i1) {
  float v[kGZPer];
#pragma unroll
  for (int u = 0; u < kGZPer; ++u) {
    const int i = i0 + u * kGZP;
    v[u] = i < i1 ? zp[i] : 0.f;
  }
  float m = 0.f;
#pragma unroll
  for (int u = 0; u < kGZPer; ++u) m = fmaxf(m, v[u]);
  for (int i = i0 + kGZPer * kGZP; i < i1; i += kGZP) m = fmaxf(m, zp[i]);
  return m;
}

struct __align__(16) GroupLds {
  uint32_t W[2][kGMaxW + 64];
  union {
    float red[2][kGPW][kTile][kSegRows];
  } u;
  float pbias[2][kGPW][kTile];
  int S[2][kSuperTiles * kTile];
  int pair[kSuperTiles * kTile];
  uint32_t pok[2][kGPW];
  int nch[2];
};
static_assert(sizeof(GroupLds) <= 80 * 1024, "two work-groups per CU (160 KB of LDS)");
static_assert(kSuperTiles == kMaxNB, "tiles per group");

__device__ __forceinline__ void stage_chunk(uint32_t* arena, const SegProj& p, int sg,
                                            uint32_t b0, uint32_t b1, int lp, int lane, int nl) {
  if (b1 <= b0) return;
  const uint32_t w0 = block_word(p, b0), w1 = block_word(p, b1);
  stage16(arena, p.planes + (size_t)sg * p.seg_words + w0, (w1 - w0) / 4u, lp, lane, nl);
}

// Coefficients of every tile, once (not once per row segment): one
// 256-lane work-group per (256-slot chunk, tile, projection).  Lane l takes
// slot 256 chunk + l of the tile's expert and forms, for each of the tile's
// tokens, c = a s z[k] (a z for 16-bit slots) and a m z[k], writes the fp16
// hi and lo parts of c 2^S_n and the chunk's row-independent sums.  The
// scale S_n follows from the expert's bound and the token's max |z| exactly
// as the apply kernel forms it.
__global__ __launch_bounds__(256) void k_group_coef(GroupArgs s) {
  const GateUpArgs& a = s.g;
  const int ck = (int)blockIdx.x, ti = (int)blockIdx.y, pj = (int)blockIdx.z;
  // the tile count and this tile's entry (ti < tcap: inside the lists) are
  // read together
  typedef __attribute__((address_space(4))) const int CI32;
  const int ntl = *(CI32*)s.rl.ntiles;
  const int e = ((CI32*)s.rl.tile)[3 * ti];
  const int p0 = ((CI32*)s.rl.tile)[3 * ti + 1];
  const int nt = ((CI32*)s.rl.tile)[3 * ti + 2];
  if ((ti >= ntl) | (nt <= 0)) return;
  const bool single = s.single != 0;
  const int lane = threadIdx.x & (kWave - 1);
  const int wv = threadIdx.x >> 6;
  const uint8_t* blob = pj ? a.blob_u : a.blob_g;
  const SegProj P = uniform_seg(make_seg(blob, pj ? a.bytes_u : a.bytes_g, e,
                                         load_rec_s(blob, e, a.E), load_hdr(blob), a.E, a.dout,
                                         a.r));
  // this thread's slot: its entries loaded first (they do not depend on the
  // tile's tokens), all four issued before any is used
  const uint32_t sl = 256u * (uint32_t)ck + threadIdx.x;
  const bool live = sl < P.n_slot;
  const bool isq = sl < P.n_qslot;
  uint32_t k = 0u;
  float av = 0.f;
  uint16_t sraw = 0x3C00u, mraw = 0u;  // fp16 1 and 0
  if (live) {
    k = P.kidx[sl];
    av = P.A[sl];
    if (isq) {
      sraw = P.S[sl];
      mraw = P.M[sl];
    }
  }
  __shared__ int S[kTile];
  __shared__ int zoff[kTile];
  __shared__ float bred[4][kTile];
  __shared__ uint32_t bad[4];
  {
    const int n = threadIdx.x / kGZP, j = threadIdx.x % kGZP;
    const int pz0 = (pj && !single) ? a.r / kProjRowsPerBlock : 0;
    const int pz1 = (pj || single) ? s.nzp : (a.r + kProjRowsPerBlock - 1) / kProjRowsPerBlock;
    float zm = 0.f;
    int pr = 0;
    if (n < nt) {
      pr = s.rl.pairs[p0 + n];
      const int t = single ? pr : pr / a.ktop;
      const float* zp = s.zpart + (size_t)t * s.nzp;
      zm = strided_max(zp, pz0 + j, pz1);
    }
#pragma unroll
    for (int off = kGZP / 2; off > 0; off >>= 1) zm = fmaxf(zm, __shfl_xor(zm, off, kWave));
    if (j == 0 && n < nt) {
      S[n] = coef_shift(P.cmax, zm);
      if (ck == 0) s.tsh[(ti * 2 + pj) * kTile + n] = S[n];  // for the grouped kernel
      zoff[n] = single ? pr * a.r : (pr / a.ktop) * (2 * a.r) + (pj ? a.r : 0);
    }
  }
  __syncthreads();
  bool good = k < (uint32_t)a.r;
  k = good ? k : 0u;
  const float sv = __half2float(__ushort_as_half(sraw));
  const float mv = __half2float(__ushort_as_half(mraw));
  const size_t row0 = (size_t)(ti * 2 + pj) * kTile;
  // the tile's z values of this slot, all loaded before any is used
  float zv[kTile];
#pragma unroll
  for (int n = 0; n < kTile; ++n) zv[n] = (live && n < nt) ? s.z[zoff[n] + k] : 0.f;
#pragma unroll
  for (int n = 0; n < kTile; ++n) {
    if (n < nt) {  // uniform
      const float az = av * zv[n];
      _Float16 hi, lo;
      split_coef(az * sv, S[n], hi, lo);
      s.thi[(row0 + n) * s.rpad + sl] = hi;
      s.tlo[(row0 + n) * s.rpad + sl] = lo;
      const float bw = wave_sum(az * mv);
      if (lane == 0) bred[wv][n] = bw;
    }
  }
  const bool wok = __all(good);
  if (lane == 0) bad[wv] = wok ? 0u : 1u;
  __syncthreads();
  if ((int)threadIdx.x < nt) {
    const int n = threadIdx.x;
    s.tbias[((size_t)(ti * 2 + pj) * s.nck + ck) * kTile + n] =
        (bred[0][n] + bred[1][n]) + (bred[2][n] + bred[3][n]);
  }
  if (threadIdx.x == 0 && (bad[0] | bad[1] | bad[2] | bad[3]))
    atomicOr(&s.tbad[ti * 2 + pj], 1u);
}

__global__ __launch_bounds__(kGThreads) void k_gateup_grouped(GroupArgs s) {
  extern __shared__ __align__(16) uint8_t lds_raw[];
  GroupLds& L = *reinterpret_cast<GroupLds*>(lds_raw);
  const GateUpArgs& a = s.g;
  const int lane = threadIdx.x & (kWave - 1);
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int pj = wv >= kGPW ? 1 : 0;  // waves 0-3 gate, 4-7 up
  const int wp = wv & (kGPW - 1);
  const int lp = (int)threadIdx.x & (kGProj - 1);

  // A unit is (group of up to kSuperTiles consecutive tiles of one expert,
  // segment): the group's planes are decoded once per K step and applied
  // to every tile of the group.  Block b runs on XCD b % 8; group x + 8 i
  // goes to XCD x, its segment units one after another, so the segments of
  // a group share one L2 for its coefficient tables; blocks past the group
  // count exit at once.
  typedef __attribute__((address_space(4))) const int CI32;
  const bool single = s.single != 0;
  const int nsu = single ? (a.n_seg + 1) / 2 : a.n_seg;  // segment units per group
  const int xcd = (int)blockIdx.x & 7, jx = (int)blockIdx.x >> 3;
  const int gi = xcd + 8 * (jx / nsu), su = jx % nsu;
  // the group count and this group's record (both written by the route step
  // before this launch) are read together; the record of a block past the
  // count is read from a group inside the lists and not used
  int grec[kGroupRec];
  {
    CI32* gr = (CI32*)(s.rl.stile + (size_t)kGroupRec * min(gi, s.tcap - 1));
#pragma unroll
    for (int u = 0; u < kGroupRec; ++u) grec[u] = gr[u];
  }
  const int ngr = *(CI32*)s.rl.nstiles;
  // (a record of a live group has a tile count of at least 1: testing it here
  // keeps its load ahead of this branch, beside the count's)
  if ((ngr <= 0) | (gi >= ngr) | (grec[1] <= 0)) return;
  // single: this half's segment (a half past the last segment repeats it
  // and writes nothing)
  const int sg0 = single ? 2 * su : su;
  const int sgh = single ? sg0 + pj : sg0;
  const int sg = sgh < a.n_seg ? sgh : a.n_seg - 1;
  const int ti0 = grec[0];
  const int nb = min(max(grec[1], 1), kSuperTiles);
  const int e = grec[2];
  int p0[kSuperTiles], ntb[kSuperTiles];  // each tile's first pair and pair count (uniform)
#pragma unroll
  for (int t = 0; t < kSuperTiles; ++t) {
    p0[t] = t < nb ? grec[3 + 2 * t] : 0;
    ntb[t] = t < nb ? grec[4 + 2 * t] : 0;
  }

  const uint8_t* blob = pj ? a.blob_u : a.blob_g;
  const SegProj P = uniform_seg(make_seg(blob, pj ? a.bytes_u : a.bytes_g, e,
                                         load_rec_s(blob, e, a.E), load_hdr(blob), a.E, a.dout,
                                         a.r));
  // the tiles' pairs (output rows), coefficient scales and row-independent
  // chunk sums (k_group_coef's) and column-index flags: every load issued
  // before the staging copies, the values used after them
  int prv[kSuperTiles], shv[kSuperTiles];
  uint32_t tbv[kSuperTiles];
  float bpv[kSuperTiles][kGBPer];
#pragma unroll
  for (int t = 0; t < kSuperTiles; ++t) {
    prv[t] = shv[t] = 0;
    tbv[t] = 0u;
    const int row = (ti0 + t) * 2 + (single ? 0 : pj);
    if (t < nb && threadIdx.x < (unsigned)ntb[t]) prv[t] = s.rl.pairs[p0[t] + threadIdx.x];
    if (t < nb && lp < ntb[t]) shv[t] = s.tsh[row * kTile + lp];
    if (t < nb) tbv[t] = s.tbad[row];
#pragma unroll
    for (int c = 0; c < kGBPer; ++c) {
      bpv[t][c] = 0.f;
      if (t < nb && wp == 0 && lane < ntb[t] && c < s.nck)
        bpv[t][c] = s.tbias[((size_t)row * s.nck + c) * kTile + lane];
    }
  }
  uint32_t b1 = chunk_end(P, 0, kGMaxW);
  stage_chunk(&L.W[pj][0], P, sg, 0, b1, lp, lane, kGProj);

  // The tiles' coefficients (k_group_coef) are read straight from the
  // tables: lane (m, kg) takes token row m of each tile (the tile's last
  // token's row past its tokens: same cache lines, columns never stored),
  // slots 8 kg ..
  uint32_t boff[kSuperTiles];
#pragma unroll
  for (int t = 0; t < kSuperTiles; ++t) {
    const int tt = t < nb ? t : 0;
    const size_t trow = (size_t)((ti0 + tt) * 2 + (single ? 0 : pj)) * kTile;
    boff[t] = (uint32_t)((trow + (size_t)min(lane & 15, max(ntb[tt], 1) - 1)) * s.rpad) +
              8u * (uint32_t)(lane >> 4);
  }

  // Plane chunks of at most kGMaxW words per projection: the two
  // projections' counts may differ, the barriers are shared, so the
  // work-group runs the larger count and a half past its own count only
  // takes part in the barriers.
  {
    int nc = 0;
    for (uint32_t b = 0; b < P.n_blk; b = chunk_end(P, b, kGMaxW)) ++nc;
    if (threadIdx.x == (unsigned)(pj * kGProj)) L.nch[pj] = nc;
  }
  float bsum[kSuperTiles];  // (wave 0 of each half, lanes of the tile's tokens)
#pragma unroll
  for (int t = 0; t < kSuperTiles; ++t) {
    if (t < nb && threadIdx.x < (unsigned)ntb[t]) L.pair[kTile * t + threadIdx.x] = prv[t];
    if (t < nb && lp < ntb[t]) L.S[pj][kTile * t + lp] = shv[t];
    // the chunks' row-independent sums in chunk order
    bsum[t] = 0.f;
#pragma unroll
    for (int c = 0; c < kGBPer; ++c) bsum[t] += bpv[t][c];
    if (t < nb && wp == 0 && lane < ntb[t])
      for (int c = kGBPer; c < s.nck; ++c)
        bsum[t] += s.tbias[((size_t)((ti0 + t) * 2 + (single ? 0 : pj)) * s.nck + c) * kTile + lane];
  }
  // the first plane chunk's staged words have landed
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  const int nch = __builtin_amdgcn_readfirstlane(max(L.nch[0], L.nch[1]));  // uniform
  const bool good = P.ok;
  f4 acc0[kSuperTiles], acc1[kSuperTiles];
#pragma unroll
  for (int t = 0; t < kSuperTiles; ++t) acc0[t] = acc1[t] = f4{0.f, 0.f, 0.f, 0.f};
  uint32_t b0 = 0;
  for (int ch = 0; ch < max(nch, 1); ++ch) {
    if (ch > 0) {
      const uint32_t b1n = chunk_end(P, b0, kGMaxW);
      lds_sync();  // every wave is done with the previous chunk
      b1 = b1n;
      stage_chunk(&L.W[pj][0], P, sg, b0, b1, lp, lane, kGProj);
      __builtin_amdgcn_s_waitcnt(0);  // this wave's staged words have landed
      lds_sync();
    }
    if (b1 > b0) {
      const uint32_t* base = &L.W[pj][0] - block_word(P, b0);
      const uint32_t kb0 = b0 / kBlkPerK, kb1 = (b1 + kBlkPerK - 1) / kBlkPerK;
      if (nb == 1)
        mfma_ksteps_gb(P, base, s.thi + boff[0], s.tlo + boff[0], kb0, kb1, wp, lane, acc0[0],
                       acc1[0]);
      else
        mfma_ksteps_gbn(P, base, s.thi, s.tlo, boff, nb, kb0, kb1, wp, lane, acc0, acc1);
    }
    b0 = b1;
  }
  // ---- per tile: row sums of the 4 waves per token, SiLU * mul ----
#pragma unroll
  for (int t = 0; t < kSuperTiles; ++t) {
    if (t >= nb) continue;  // (uniform)
    const int nt = ntb[t];
    __syncthreads();  // the previous tile's sums are read
    {
      const int n = lane & 15, kg = lane >> 4;
      if (n < nt) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          L.u.red[pj][wp][n][4 * kg + i] = acc0[t][i];
          L.u.red[pj][wp][n][16 + 4 * kg + i] = acc1[t][i];
        }
      }
      // the row-independent sums of the tile's chunks (wave 0 of each half),
      // the column-index check from the coefficient pass
      if (wp == 0 && lane < nt) {
        L.pbias[pj][0][lane] = bsum[t];
      } else if (lane < nt) {
        L.pbias[pj][wp][lane] = 0.f;
      }
      const bool wok = __all(good) && tbv[t] == 0u;
      if (lane == 0) L.pok[pj][wp] = wok;
    }
    __syncthreads();
    {
      const int n = threadIdx.x >> 5, row = threadIdx.x & 31;
      if (n < nt) {
        float ys[2];
        uint32_t okq[2];
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          float sum = 0.f, bsum = 0.f;
          uint32_t okw = 1u;
#pragma unroll
          for (int w = 0; w < kGPW; ++w) {
            sum += L.u.red[q][w][n][row];
            bsum += L.pbias[q][w][n];
            okw &= L.pok[q][w];
          }
          ys[q] = ldexpf(sum, -L.S[q][kTile * t + n]) + bsum;
          okq[q] = okw;
        }
        const int pr = L.pair[kTile * t + n];
        if (!single) {
          const int orow = sg * kSegRows + row;
          if (orow < a.dout)
            a.h[(size_t)pr * a.dout + orow] =
                (okq[0] & okq[1]) ? silu_mul(ys[0], ys[1]) : __builtin_nanf("");
        } else {
#pragma unroll
          for (int q = 0; q < 2; ++q) {
            const int orow = (sg0 + q) * kSegRows + row;
            if (sg0 + q < a.n_seg && orow < a.dout)
              a.h[(size_t)pr * a.dout + orow] = okq[q] ? ys[q] : __builtin_nanf("");
          }
        }
      }
    }
  }
}

}  // namespace

size_t grouped_lds_bytes() { return sizeof(GroupLds); }

int launch_route_group(const int32_t* ids, int P, int E, int dout, float* h,
                       const RouteLists& rl, hipStream_t st, uint32_t* zero, int nzero) {
  const RouteJob j{ids, P, E, dout, h, rl, zero, nzero};
  hipLaunchKernelGGL(k_route_group, dim3(1), dim3(kRThreads), (size_t)2 * E * sizeof(uint32_t),
                     st, j);
  return 0;
}

int launch_group_coef(const GroupArgs& s, hipStream_t st) {
  hipLaunchKernelGGL(k_group_coef, dim3((unsigned)s.nck, (unsigned)s.tcap, s.single ? 1u : 2u),
                     dim3(256), 0, st, s);
  return 0;
}

int launch_gateup_grouped(const GroupArgs& s, hipStream_t st) {
  static bool attr_done[64];
  int dev = 0;
  if (hipGetDevice(&dev) == hipSuccess && dev >= 0 && dev < 64 && !attr_done[dev]) {
    (void)hipFuncSetAttribute((const void*)k_gateup_grouped,
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)sizeof(GroupLds));
    (void)hipGetLastError();
    attr_done[dev] = true;
  }
  // (tile group x + 8 i on XCD x: 8 blocks per segment unit and group
  // octet; there are at most tcap groups)
  const long long blocks =
      8ll * ((s.tcap + 7) / 8) * (s.single ? (s.g.n_seg + 1) / 2 : s.g.n_seg);
  hipLaunchKernelGGL(k_gateup_grouped, dim3((unsigned)blocks), dim3(kGThreads), sizeof(GroupLds),
                     st, s);
  return 0;
}

}  // namespace bitsmoe
