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
// k_gateup_grouped: one 512-lane work-group per (tile, 32-row segment) unit,
// both projections (waves 0-3 gate, 4-7 up); unit u = segment * tcap + tile
// runs on XCD u % 8, so every segment of a tile shares one L2 (and reads the
// tile's coefficient tables from it).  The segment records are staged in
// LDS in chunks of at most 7168 words per projection; the tile's
// coefficients go through LDS in 128-slot chunks, each loaded into
// registers (16 bytes a lane) while the previous chunk's products run.  The
// work-group's LDS stays under half of a CU's, so two units share a CU and
// each one's chain of dependent loads overlaps the other's products.  The
// apply is the same MFMA K-step loop as the
// one-launch kernel with up to 16 token columns.  A one-projection mode
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
constexpr int kGCS = 128;                   // slots per coefficient chunk of the apply
constexpr int kGCStride = kGCS + 8;         // fp16 per token row (bank spread)
constexpr int kGZP = 16;                    // lanes per token for the partial maxima

struct __align__(16) GroupLds {
  uint32_t W[2][kGMaxW + 64];
  union {
    struct {
      _Float16 hi[2][kTile * kGCStride];
      _Float16 lo[2][kTile * kGCStride];
    } c;
    float red[2][kGPW][kTile][kSegRows];
  } u;
  float pbias[2][kGPW][kTile];
  int S[2][kTile];
  int pair[kTile];
  uint32_t pok[2][kGPW];
  int nch[2];
  int ncc[2][2];  // [plane chunk parity][projection]: coefficient chunks
};
static_assert(sizeof(GroupLds) <= 80 * 1024, "two work-groups per CU (160 KB of LDS)");

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
  if (ti >= s.rl.ntiles[0]) return;
  const bool single = s.single != 0;
  const int lane = threadIdx.x & (kWave - 1);
  const int wv = threadIdx.x >> 6;
  const int e = __builtin_amdgcn_readfirstlane(s.rl.tile[3 * ti]);
  const int p0 = __builtin_amdgcn_readfirstlane(s.rl.tile[3 * ti + 1]);
  const int nt = __builtin_amdgcn_readfirstlane(s.rl.tile[3 * ti + 2]);
  const uint8_t* blob = pj ? a.blob_u : a.blob_g;
  const SegProj P = uniform_seg(make_seg(blob, pj ? a.bytes_u : a.bytes_g, e,
                                         load_rec_s(blob, e, a.E), load_hdr(blob), a.E, a.dout,
                                         a.r));
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
      for (int i = pz0 + j; i < pz1; i += kGZP) zm = fmaxf(zm, zp[i]);
    }
#pragma unroll
    for (int off = kGZP / 2; off > 0; off >>= 1) zm = fmaxf(zm, __shfl_xor(zm, off, kWave));
    if (j == 0 && n < nt) {
      S[n] = coef_shift(P.cmax, zm);
      zoff[n] = single ? pr * a.r : (pr / a.ktop) * (2 * a.r) + (pj ? a.r : 0);
    }
  }
  __syncthreads();
  const uint32_t sl = 256u * (uint32_t)ck + threadIdx.x;
  const bool live = sl < P.n_slot;
  uint32_t k = live ? P.kidx[sl] : 0u;
  bool good = k < (uint32_t)a.r;
  k = good ? k : 0u;
  const float av = live ? P.A[sl] : 0.f;
  const bool isq = sl < P.n_qslot;
  const float sv = (live && isq) ? __half2float(__ushort_as_half(P.S[sl])) : 1.f;
  const float mv = (live && isq) ? __half2float(__ushort_as_half(P.M[sl])) : 0.f;
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

  const int u = blockIdx.x;
  const int ti = u % s.tcap;
  const bool single = s.single != 0;
  // single: this half's segment (a half past the last segment repeats it
  // and writes nothing)
  const int sg0 = single ? 2 * (u / s.tcap) : u / s.tcap;
  if (sg0 >= a.n_seg || ti >= s.rl.ntiles[0]) return;
  const int sgh = single ? sg0 + pj : sg0;
  const int sg = sgh < a.n_seg ? sgh : a.n_seg - 1;
  const int e = __builtin_amdgcn_readfirstlane(s.rl.tile[3 * ti]);
  const int p0 = __builtin_amdgcn_readfirstlane(s.rl.tile[3 * ti + 1]);
  const int nt = __builtin_amdgcn_readfirstlane(s.rl.tile[3 * ti + 2]);

  const uint8_t* blob = pj ? a.blob_u : a.blob_g;
  const SegProj P = uniform_seg(make_seg(blob, pj ? a.bytes_u : a.bytes_g, e,
                                         load_rec_s(blob, e, a.E), load_hdr(blob), a.E, a.dout,
                                         a.r));
  uint32_t b1 = chunk_end(P, 0, kGMaxW);
  stage_chunk(&L.W[pj][0], P, sg, 0, b1, lp, lane, kGProj);

  // The tile's coefficients (k_group_coef) pass through registers: lane lp
  // holds the 16-byte piece 8 (lp % 16) .. + 7 of row lp / 16 of the hi and
  // lo tables; the next 128-slot chunk is loaded while the products of the
  // current one run.  Rows past the tile's tokens load the last token's row
  // (same cache lines) and are not stored.
  const size_t trow = (size_t)(ti * 2 + (single ? 0 : pj)) * kTile;
  static_assert(kGProj == kTile * kGCS / 8, "one 16-byte piece per lane");
  const int cq = lp / (kGCS / 8), c8 = 8 * (lp % (kGCS / 8));
  const bool cA = cq < nt;
  const size_t oA = (trow + (size_t)min(cq, nt - 1)) * s.rpad + c8;
  _Float16* const dA = &L.u.c.hi[pj][0] + cq * kGCStride + c8;
  _Float16* const dAl = &L.u.c.lo[pj][0] + cq * kGCStride + c8;
  uint4 chA, clA;
#define GROUPED_COEF_FETCH(s0)                                             \
  do {                                                                     \
    chA = *reinterpret_cast<const uint4*>(s.thi + oA + (s0));             \
    clA = *reinterpret_cast<const uint4*>(s.tlo + oA + (s0));             \
  } while (0)
  GROUPED_COEF_FETCH(0u);

  // tokens of the tile and their coefficient scales: lanes (n, j) of the
  // projection take partial maxima j, j + 16, ... of token n
  if (threadIdx.x < (unsigned)nt) L.pair[threadIdx.x] = s.rl.pairs[p0 + threadIdx.x];
  {
    const int n = lp / kGZP, j = lp % kGZP;
    const int pz0 = (pj && !single) ? a.r / kProjRowsPerBlock : 0;
    const int pz1 = (pj || single) ? s.nzp : (a.r + kProjRowsPerBlock - 1) / kProjRowsPerBlock;
    float zm = 0.f;
    if (n < nt) {
      const int pr = s.rl.pairs[p0 + n];
      const int t = single ? pr : pr / a.ktop;  // z row: the pair's own (single) or its token's
      const float* zp = s.zpart + (size_t)t * s.nzp;
      for (int i = pz0 + j; i < pz1; i += kGZP) zm = fmaxf(zm, zp[i]);
    }
#pragma unroll
    for (int off = kGZP / 2; off > 0; off >>= 1) zm = fmaxf(zm, __shfl_xor(zm, off, kWave));
    if (j == 0 && n < nt) L.S[pj][n] = coef_shift(P.cmax, zm);
  }
  // Coefficient chunks of kGCS slots (kGCS / 4 blocks, kGCS / 32 K steps)
  // inside each plane chunk.  The two projections' plane chunks end at
  // different blocks, so their counts of coefficient chunks may differ; the
  // barriers are shared, so the work-group runs the larger count (published
  // through L.ncc, one slot per chunk parity) and a half past its own count
  // only takes part in the barriers.
  constexpr uint32_t kCB = kGCS / 4;
  auto n_coef_chunks = [](uint32_t c0, uint32_t c1) {
    return max((int)((c1 - c0 + kCB - 1) / kCB), 1);
  };
  {
    int nc = 0;
    for (uint32_t b = 0; b < P.n_blk; b = chunk_end(P, b, kGMaxW)) ++nc;
    if (threadIdx.x == (unsigned)(pj * kGProj)) {
      L.nch[pj] = nc;
      L.ncc[0][pj] = n_coef_chunks(0u, b1);
    }
  }
  // the first plane chunk's staged words have landed (waited for here, once,
  // so that no later LDS read is made to wait for the coefficient loads)
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  const int nch = __builtin_amdgcn_readfirstlane(max(L.nch[0], L.nch[1]));  // uniform
  bool good = P.ok;
  f4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
  uint32_t b0 = 0;
  for (int ch = 0; ch < max(nch, 1); ++ch) {
    if (ch > 0) {
      const uint32_t b1n = chunk_end(P, b0, kGMaxW);
      if (threadIdx.x == (unsigned)(pj * kGProj)) L.ncc[ch & 1][pj] = n_coef_chunks(b0, b1n);
      lds_sync();  // every wave is done with the previous chunk; L.ncc is set
      b1 = b1n;
      stage_chunk(&L.W[pj][0], P, sg, b0, b1, lp, lane, kGProj);
      __builtin_amdgcn_s_waitcnt(0);  // the staged words have landed
    }
    const uint32_t kbe = (b1 + kBlkPerK - 1) / kBlkPerK;
    const int ncc = n_coef_chunks(b0, b1);  // this half's
    const int nccw = __builtin_amdgcn_readfirstlane(max(L.ncc[ch & 1][0], L.ncc[ch & 1][1]));
    for (int cc = 0; cc < nccw; ++cc) {
      const uint32_t cb0 = b0 + kCB * cc;
      const uint32_t s0 = 4u * cb0;
      const bool mine = cc < ncc;
      if (cc > 0) lds_sync();  // the previous coefficient chunk is read
      if (mine) {
        if (cA) {
          *reinterpret_cast<uint4*>(dA) = chA;
          *reinterpret_cast<uint4*>(dAl) = clA;
        }
        if (cc + 1 < ncc)
          GROUPED_COEF_FETCH(s0 + (uint32_t)kGCS);
        else if (ch + 1 < nch)
          GROUPED_COEF_FETCH(4u * b1);
      }
      lds_sync();
      const uint32_t kb0 = cb0 / kBlkPerK;
      const uint32_t kb1 = min(kb0 + kCB / kBlkPerK, kbe);
      if (mine && b1 > cb0) {
        const uint32_t* base = &L.W[pj][0] - block_word(P, b0);
        mfma_ksteps(P, base, &L.u.c.hi[pj][0], &L.u.c.lo[pj][0], kGCStride, s0,
                    nt, kb0, kb1, wp, lane, acc0, acc1);
      }
    }
    b0 = b1;
  }
#undef GROUPED_COEF_FETCH
  __syncthreads();  // coefficient tables are reused as row-sum buffers
  // ---- row sums of the 4 waves per token, SiLU * mul ----
  {
    const int n = lane & 15, kg = lane >> 4;
    if (n < nt) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        L.u.red[pj][wp][n][4 * kg + i] = acc0[i];
        L.u.red[pj][wp][n][16 + 4 * kg + i] = acc1[i];
      }
    }
    // the row-independent sums of the tile's chunks (wave 0 of each half),
    // the column-index check from the coefficient pass
    if (wp == 0 && lane < nt) {
      const float* tb = s.tbias + (size_t)(ti * 2 + (single ? 0 : pj)) * s.nck * kTile + lane;
      float bsum = 0.f;
      for (int c = 0; c < s.nck; ++c) bsum += tb[(size_t)c * kTile];
      L.pbias[pj][0][lane] = bsum;
    } else if (lane < nt) {
      L.pbias[pj][wp][lane] = 0.f;
    }
    const bool wok = __all(good) && s.tbad[ti * 2 + (single ? 0 : pj)] == 0u;
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
        ys[q] = ldexpf(sum, -L.S[q][n]) + bsum;
        okq[q] = okw;
      }
      if (!single) {
        const int orow = sg * kSegRows + row;
        if (orow < a.dout)
          a.h[(size_t)L.pair[n] * a.dout + orow] =
              (okq[0] & okq[1]) ? silu_mul(ys[0], ys[1]) : __builtin_nanf("");
      } else {
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const int orow = (sg0 + q) * kSegRows + row;
          if (sg0 + q < a.n_seg && orow < a.dout)
            a.h[(size_t)L.pair[n] * a.dout + orow] = okq[q] ? ys[q] : __builtin_nanf("");
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
  const long long blocks = (long long)s.tcap * (s.single ? (s.g.n_seg + 1) / 2 : s.g.n_seg);
  hipLaunchKernelGGL(k_gateup_grouped, dim3((unsigned)blocks), dim3(kGThreads), sizeof(GroupLds),
                     st, s);
  return 0;
}

}  // namespace bitsmoe
