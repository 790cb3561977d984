// gfx950 kernels and the device entry points of the C ABI.
//
// Path (BitsMoE blog note, Methodology): z = Phi^T x once per token ("first
// split"), then for each routed expert y_e = sum_k a_{e,k} z_k p_hat_{e,k}
// over the width-grouped bit planes ("second split", "execution"), then
// h = SiLU(y_gate) * y_up.
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include <atomic>
#include <mutex>
#include <type_traits>

#include "bitsmoe.h"
#include "common.h"
#include "device_common.h"
#include "format.h"
#include "kernels.h"
#include "route.h"
#include "seg_common.h"

namespace bitsmoe {
namespace {

// Bound on the waits of the one-launch kernels (polls of the hint counters
// and re-reads of stale z words); a test hook can lower it.
std::atomic<uint32_t> g_wait_limit{kSpinDefault};

// ---------------------------------------------------------------------------
// Shared projection for din > 4096: one wave per basis vector n.  Lanes
// stride the din reduction with 16-byte loads; fp16 pairs are multiplied and
// accumulated in float32 by v_dot2_f32_f16; a wave reduction finishes it.
// Phi^T is read once per chunk of kTokChunk tokens.
// ---------------------------------------------------------------------------
constexpr int kProjWaves = 4;
constexpr int kTokChunk = 4;

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

__device__ inline float dot8(uint4 a, uint4 b, float acc) {
  const half2_t* ha = reinterpret_cast<const half2_t*>(&a);
  const half2_t* hb = reinterpret_cast<const half2_t*>(&b);
#pragma unroll
  for (int i = 0; i < 4; ++i) acc = __builtin_amdgcn_fdot2(ha[i], hb[i], acc, false);
  return acc;
}

__global__ __launch_bounds__(kProjWaves * kWave) void k_proj_gemv(
    const uint4* __restrict__ phi_t, const uint4* __restrict__ x, float* __restrict__ z,
    int T, int din8, int R) {
  constexpr int U = 4;  // 16-byte loads in flight per lane
  const int lane = threadIdx.x & (kWave - 1);
  const int n = blockIdx.x * kProjWaves + (threadIdx.x >> 6);
  if (n >= R) return;
  const uint4* prow = phi_t + (size_t)n * din8;
  for (int t0 = 0; t0 < T; t0 += kTokChunk) {
    float acc[kTokChunk] = {0.f, 0.f, 0.f, 0.f};
    for (int i0 = lane; i0 < din8; i0 += kWave * U) {
      uint4 pv[U];
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (i0 + u * kWave < din8) pv[u] = prow[i0 + u * kWave];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (i0 + u * kWave >= din8) break;
#pragma unroll
        for (int tt = 0; tt < kTokChunk; ++tt)
          if (t0 + tt < T)
            acc[tt] = dot8(pv[u], x[(size_t)(t0 + tt) * din8 + i0 + u * kWave], acc[tt]);
      }
    }
#pragma unroll
    for (int tt = 0; tt < kTokChunk; ++tt) {
      const float s = wave_sum(acc[tt]);
      if (lane == 0 && t0 + tt < T) z[(size_t)(t0 + tt) * R + n] = s;
    }
  }
}

// ---------------------------------------------------------------------------
// Shared projection, token batches: a work-group of 4 waves owns 16 Phi^T
// rows (4 per wave, held in registers, read once) and walks the tokens 4 at a
// time; each batch of x is copied into LDS once with 16-byte
// global_load_lds and read by all 16 rows.  A wave's 16 dot products (4
// rows x 4 tokens) are finished with a transpose reduction (17 lane
// exchanges) and lanes 0-15 store them.  When zpart is given, the
// work-group also writes max |z| over its 16 rows per token (zpart[t * nzp
// + group]), from which the grouped kernel sizes its fp16 coefficient
// scale.  U: 16-byte x units per lane (din <= 512 U).
// ---------------------------------------------------------------------------
constexpr int kPRW = 4;     // Phi^T rows per wave
constexpr int kPT = 4;      // tokens per batch
constexpr int kPMaxU = 8;   // din <= 4096

typedef __attribute__((address_space(3))) void lds_void_t;

template <int O>
__device__ __forceinline__ void pstep(float (&v)[kPRW * kPT], bool up) {
#pragma unroll
  for (int i = 0; i < O; ++i) {
    const float send = up ? v[i] : v[i + O];
    const float keep = up ? v[i + O] : v[i];
    v[i] = keep + __shfl_xor(send, O, kWave);
  }
}

// Batched projection on the matrix cores (T >= 16, din a multiple of 32):
// z^T = Phi^T x^T as a dense contraction over din.  Work-group (b, c): rows
// 16 b .. 16 b + 15 of Phi^T and tokens 64 c .. 64 c + 63 (four 16-token
// blocks).  Wave w takes the K steps (32 of din each) k = w, w + 8, ...: it
// loads the Phi^T piece of a step once and applies it to every token block
// present with v_mfma_f32_16x16x32_f16, four steps' loads in flight, so the
// work-group keeps 8 waves' worth of Phi^T reads outstanding.  Both operands
// are read from global memory in 16-byte pieces (Phi^T rows and x rows are
// contiguous along din).  The 8 partial sums are added through LDS in wave
// order.  fp16 products are exact in fp32; the sums are fp32.  zpart gets
// the largest |z| of the 16 rows per token.  With a route job, one more
// column of work-groups is launched and its first one groups the pairs by
// expert (route.h) while the others project.
typedef _Float16 h8v __attribute__((ext_vector_type(8)));
typedef float f4v __attribute__((ext_vector_type(4)));
constexpr int kPMWaves = 8;   // waves of a projection work-group (K split)
constexpr int kPMBlocks = 4;  // 16-token blocks of a work-group

__device__ __forceinline__ f4v mfma16(const uint4& a, const uint4& b, f4v c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(*reinterpret_cast<const h8v*>(&a),
                                                *reinterpret_cast<const h8v*>(&b), c, 0, 0, 0);
}

__global__ __launch_bounds__(kPMWaves * kWave) void k_proj_mfma(const uint4* __restrict__ phi_t,
                                                               const uint4* __restrict__ x,
                                                               float* __restrict__ z,
                                                               float* __restrict__ zpart, int T,
                                                               int din8, int R, int nzp,
                                                               RouteJob rj) {
  __shared__ union {
    f4v part[kPMWaves][kPMBlocks][kWave];
    struct {
      uint32_t cnt[2 * kRouteFuseMaxE];
      uint32_t buf[kPMWaves * kWave];
    } r;
  } L;
  if (rj.ids && (int)blockIdx.x == nzp) {
    if (blockIdx.y == 0) route_lists<kPMWaves * kWave>(rj, L.r.cnt, L.r.buf);
    return;
  }
  f4v(&part)[kPMWaves][kPMBlocks][kWave] = L.part;
  const int lane = threadIdx.x & (kWave - 1);
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int row0 = (int)blockIdx.x * 16;
  const int tok0 = (int)blockIdx.y * 16 * kPMBlocks;
  const int nb = min(kPMBlocks, (T - tok0 + 15) / 16);  // token blocks present (>= 1)
  const int m = lane & 15, kg = lane >> 4;
  const uint4* pa = phi_t + (size_t)min(row0 + m, R - 1) * din8 + kg;
  const uint4* pb[kPMBlocks];
#pragma unroll
  for (int b = 0; b < kPMBlocks; ++b)
    pb[b] = x + (size_t)min(tok0 + 16 * b + m, T - 1) * din8 + kg;
  f4v acc[kPMBlocks];
#pragma unroll
  for (int b = 0; b < kPMBlocks; ++b) acc[b] = f4v{0.f, 0.f, 0.f, 0.f};
  const int nk = din8 / 4;  // K steps of 32
  int k = wv;
  for (; k + 3 * kPMWaves < nk; k += 4 * kPMWaves) {
    uint4 av[4], bv[4][kPMBlocks];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      av[j] = pa[4 * (k + j * kPMWaves)];
#pragma unroll
      for (int b = 0; b < kPMBlocks; ++b)
        if (b < nb) bv[j][b] = pb[b][4 * (k + j * kPMWaves)];
    }
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int b = 0; b < kPMBlocks; ++b)
        if (b < nb) acc[b] = mfma16(av[j], bv[j][b], acc[b]);
  }
  for (; k < nk; k += kPMWaves) {
    const uint4 av = pa[4 * k];
#pragma unroll
    for (int b = 0; b < kPMBlocks; ++b)
      if (b < nb) acc[b] = mfma16(av, pb[b][4 * k], acc[b]);
  }
#pragma unroll
  for (int b = 0; b < kPMBlocks; ++b)
    if (b < nb) part[wv][b][lane] = acc[b];
  __syncthreads();
  // wave b < nb sums block b: s[i] = z of row row0 + 4 kg + i, token
  // tok0 + 16 b + m
  if (wv >= nb) return;
  f4v sum = part[0][wv][lane];
#pragma unroll
  for (int w = 1; w < kPMWaves; ++w) sum += part[w][wv][lane];
  const int tok = tok0 + 16 * wv + m;
  float mx = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = row0 + 4 * kg + i;
    if (tok < T && row < R) z[(size_t)tok * R + row] = sum[i];
    mx = fmaxf(mx, row < R ? fabsf(sum[i]) : 0.f);
  }
  mx = fmaxf(mx, __shfl_xor(mx, 16, kWave));
  mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
  if (zpart && kg == 0 && tok < T) zpart[(size_t)tok * nzp + blockIdx.x] = mx;
}

// Batched projection for token counts where z^T = Phi^T x^T is a real dense
// contraction (T >= 64, din a multiple of 128): work-group (b, c) computes
// rows 128 b .. + 127 of Phi^T against tokens 64 c .. + 63.  din runs in
// chunks of 128; each chunk's Phi^T rows (32 KB) and x rows (16 KB) are
// copied into LDS with 16-byte global_load_lds into one of three buffers,
// two chunks ahead of the one being multiplied.  The 16-byte pieces of a
// row are stored with their index xor the row's low four bits, so the
// sixteen rows one matrix-core read touches spread over the banks.  Wave w
// takes rows 32 w .. + 31 and all 64 tokens: per 32-wide K step two A
// pieces, four B pieces and eight v_mfma_f32_16x16x32_f16.  fp16 products
// are exact in fp32; the sums are fp32 in K order.  zpart gets the largest
// |z| of each 16 rows per token.  With a route job, one more column of
// work-groups is launched and its first one groups the pairs by expert.
constexpr int kQM = 128, kQN = 64, kQK = 128;  // rows, tokens, din per chunk
constexpr int kQWaves = 4;
constexpr int kQStages = 3;
constexpr int kQP = kQK / 8;  // 16-byte pieces per row and chunk
constexpr int kQCopies = (kQM + kQN) * kQP / kWave / kQWaves;  // copies per wave and chunk

__shared__ __align__(16) uint4 g_qa0[kQM * kQP], g_qa1[kQM * kQP], g_qa2[kQM * kQP];
__shared__ __align__(16) uint4 g_qb0[kQN * kQP], g_qb1[kQN * kQP], g_qb2[kQN * kQP];

// One 16-byte-per-lane copy from global memory into LDS (lane l writes
// lds + 16 l).  Issued as a one-instruction asm block: the compiler then
// does not treat the copy as a pending LDS write, so it inserts no wait for
// it before the reads of the other buffers; the kernel orders the copies
// with explicit vmcnt waits and barriers.  (The copy writes no VGPR.)
__device__ __forceinline__ void lds_copy16(const void* src, const void* lds) {
  const uint32_t m0 = (uint32_t)(uintptr_t)lds;  // the LDS offset (low half of the address)
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(src), "s"(m0)
               : "memory", "m0");
}

__device__ __forceinline__ void proj_stage(uint4* la, uint4* lb, const uint4* phi_t,
                                           const uint4* x, int row0, int tok0, int R, int T,
                                           int din8, int ck, int wv, int lane) {
  constexpr int kRowsPerCopy = kWave / kQP;  // 4
  const int j = lane % kQP;
#pragma unroll
  for (int q = 0; q < kQM / kRowsPerCopy / kQWaves; ++q) {
    const int g = wv * (kQM / kRowsPerCopy / kQWaves) + q, r = kRowsPerCopy * g + lane / kQP;
    lds_copy16(phi_t + (size_t)min(row0 + r, R - 1) * din8 + kQP * ck + (j ^ (r & 15)),
               la + kWave * g);
  }
#pragma unroll
  for (int q = 0; q < kQN / kRowsPerCopy / kQWaves; ++q) {
    const int g = wv * (kQN / kRowsPerCopy / kQWaves) + q, t = kRowsPerCopy * g + lane / kQP;
    lds_copy16(x + (size_t)min(tok0 + t, T - 1) * din8 + kQP * ck + (j ^ (t & 15)),
               lb + kWave * g);
  }
}

// The products of one chunk held in buffers (la, lb).
__device__ __forceinline__ void proj_chunk(const uint4* la, const uint4* lb, int wv, int m,
                                           int kg, f4v (&acc)[2][4]) {
#pragma unroll
  for (int kk = 0; kk < kQP / 4; ++kk) {
    const int c = 4 * kk + kg;
    uint4 av[2], bv[4];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int r = 32 * wv + 16 * t + m;
      av[t] = la[kQP * r + (c ^ (r & 15))];
    }
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int tt = 16 * b + m;
      bv[b] = lb[kQP * tt + (c ^ (tt & 15))];
    }
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int b = 0; b < 4; ++b) acc[t][b] = mfma16(av[t], bv[b], acc[t][b]);
  }
}

// Work-group barrier over LDS only (a fence-based barrier would wait for
// the copies in flight); the compiler moves no memory access across it.
__device__ __forceinline__ void proj_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__global__ __launch_bounds__(kQWaves * kWave) void k_proj_gemm(const uint4* __restrict__ phi_t,
                                                              const uint4* __restrict__ x,
                                                              float* __restrict__ z,
                                                              float* __restrict__ zpart, int T,
                                                              int din8, int R, int nzp,
                                                              RouteJob rj) {
  // Work-group b runs on XCD b % 8.  The work-groups of XCD x take the row
  // blocks x, x + 8, ..., each with all of its token tiles one after
  // another, so a row block's Phi^T rows come from HBM into one L2 and its
  // token tiles read them there (with the tiles on different XCDs every L2
  // fetched all of Phi^T).  The work-group after them groups the routed
  // pairs when a route job is given.
  const int nmb = (R + kQM - 1) / kQM, ntb = (T + kQN - 1) / kQN;
  const int nmain = 8 * ((nmb + 7) / 8) * ntb;
  if ((int)blockIdx.x >= nmain) {
    if (rj.ids) {
      uint32_t* cnt = reinterpret_cast<uint32_t*>(g_qa0);
      static_assert(sizeof(g_qa0) >= (2 * kRouteFuseMaxE + kQWaves * kWave) * 4, "route LDS");
      route_lists<kQWaves * kWave>(rj, cnt, cnt + 2 * kRouteFuseMaxE);
    }
    return;
  }
  const int jx = (int)blockIdx.x >> 3;
  const int mb = ((int)blockIdx.x & 7) + 8 * (jx / ntb), tb = jx % ntb;
  if (mb >= nmb) return;
  const int lane = threadIdx.x & (kWave - 1);
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int row0 = mb * kQM, tok0 = tb * kQN;
  const int m = lane & 15, kg = lane >> 4;
  const int nck = din8 / kQP;
  f4v acc[2][4];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[t][b] = f4v{0.f, 0.f, 0.f, 0.f};
  proj_stage(g_qa0, g_qb0, phi_t, x, row0, tok0, R, T, din8, 0, wv, lane);
  if (nck > 1) proj_stage(g_qa1, g_qb1, phi_t, x, row0, tok0, R, T, din8, 1, wv, lane);
  // chunk ck: this wave's copies of it are in (those of chunk ck + 1 may
  // still be on their way), then every wave's; the buffer of chunk ck + 2
  // was last read for chunk ck - 1, which every wave has finished
  static_assert(kQCopies < 16, "vmcnt field");
#define PROJ_STEP(CK, LA, LB, NA, NB)                                                do {                                                                                 if ((CK) + 1 < nck)                                                                  __builtin_amdgcn_s_waitcnt(0x0F70 | kQCopies);                                   else                                                                                 __builtin_amdgcn_s_waitcnt(0x0F70);                                              proj_barrier();                                                                    if ((CK) + 2 < nck)                                                                  proj_stage(NA, NB, phi_t, x, row0, tok0, R, T, din8, (CK) + 2, wv, lane);        proj_chunk(LA, LB, wv, m, kg, acc);                                              } while (0)
  for (int ck = 0; ck < nck; ck += kQStages) {
    PROJ_STEP(ck, g_qa0, g_qb0, g_qa2, g_qb2);
    if (ck + 1 < nck) PROJ_STEP(ck + 1, g_qa1, g_qb1, g_qa0, g_qb0);
    if (ck + 2 < nck) PROJ_STEP(ck + 2, g_qa2, g_qb2, g_qa1, g_qb1);
  }
#undef PROJ_STEP
  // lane (m, kg) of block (t, b) holds rows 4 kg .. + 3 of the 16-row block
  // for token 16 b + m
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int rb = row0 + 32 * wv + 16 * t;  // first row of the block
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int tok = tok0 + 16 * b + m;
      float mx = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = rb + 4 * kg + i;
        if (tok < T && row < R) z[(size_t)tok * R + row] = acc[t][b][i];
        mx = fmaxf(mx, row < R ? fabsf(acc[t][b][i]) : 0.f);
      }
      mx = fmaxf(mx, __shfl_xor(mx, 16, kWave));
      mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
      if (zpart && kg == 0 && tok < T && rb < R) zpart[(size_t)tok * nzp + rb / 16] = mx;
    }
  }
}

// F32: x holds float32 values, rounded to fp16 (to nearest even) while they
// are staged, so z is the projection of fp16(x) exactly as with an fp16 x.
// With a route job, the last work-group groups the pairs by expert
// (route.h) instead of projecting.
template <int U, bool F32>
__global__ __launch_bounds__(kProjWaves * kWave) void k_proj_rows(
    const uint4* __restrict__ phi_t, const void* __restrict__ xin, float* __restrict__ z,
    float* __restrict__ zpart, int T, int din8, int R, RouteJob rj) {
  __shared__ union {
    uint4 xs[kPT][kPMaxU * kWave];
    struct {
      uint32_t cnt[2 * kRouteFuseMaxE];
      uint32_t buf[kProjWaves * kWave];
    } r;
  } L;
  __shared__ float wmx[kProjWaves][kPT];
  // projection work-groups: the row stride of zpart (the route work-group,
  // if any, is the last one and writes no maxima)
  const unsigned nproj = gridDim.x - (rj.ids ? 1u : 0u);
  if (blockIdx.x >= nproj) {
    route_lists<kProjWaves * kWave>(rj, L.r.cnt, L.r.buf);
    return;
  }
  uint4(&xs)[kPT][kPMaxU * kWave] = L.xs;
  const uint4* __restrict__ x = static_cast<const uint4*>(xin);
  const float* __restrict__ xf = static_cast<const float*>(xin);
  const int lane = threadIdx.x & (kWave - 1);
  const int wv = threadIdx.x >> 6;
  const int n0 = (blockIdx.x * kProjWaves + wv) * kPRW;
  uint4 ph[kPRW][U];
#pragma unroll
  for (int i = 0; i < kPRW; ++i) {
    const int n = n0 + i;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int idx = lane + kWave * u;
      ph[i][u] = (n < R && idx < din8) ? phi_t[(size_t)n * din8 + idx] : make_uint4(0, 0, 0, 0);
    }
  }
  for (int t0 = 0; t0 < T; t0 += kPT) {
    __syncthreads();  // the previous batch has been read
    for (int tt = 0; tt < kPT && t0 + tt < T; ++tt) {
      if constexpr (F32) {
        const float4* src = reinterpret_cast<const float4*>(xf + (size_t)(t0 + tt) * din8 * 8);
        for (int i = threadIdx.x; i < din8; i += kProjWaves * kWave) {
          const float4 a = src[2 * i], b = src[2 * i + 1];
          union {
            _Float16 h[8];
            uint4 u;
          } c;
          c.h[0] = (_Float16)a.x;
          c.h[1] = (_Float16)a.y;
          c.h[2] = (_Float16)a.z;
          c.h[3] = (_Float16)a.w;
          c.h[4] = (_Float16)b.x;
          c.h[5] = (_Float16)b.y;
          c.h[6] = (_Float16)b.z;
          c.h[7] = (_Float16)b.w;
          xs[tt][i] = c.u;
        }
      } else {
        const uint4* src = x + (size_t)(t0 + tt) * din8;
        uint8_t* dst = reinterpret_cast<uint8_t*>(&xs[tt][0]);
        for (int i = threadIdx.x; i < din8; i += kProjWaves * kWave)
          __builtin_amdgcn_global_load_lds(static_cast<const void*>(src + i),
                                           (lds_void_t*)(dst + 16 * (size_t)(i - lane)), 16, 0,
                                           0);
      }
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    float v[kPRW * kPT];
#pragma unroll
    for (int i = 0; i < kPRW * kPT; ++i) v[i] = 0.f;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int idx = lane + kWave * u;
      if (idx < din8) {
#pragma unroll
        for (int tt = 0; tt < kPT; ++tt) {
          const uint4 xv = xs[tt][idx];
#pragma unroll
          for (int i = 0; i < kPRW; ++i) v[i * kPT + tt] = dot8(ph[i][u], xv, v[i * kPT + tt]);
        }
      }
    }
    pstep<8>(v, (lane & 8) != 0);
    pstep<4>(v, (lane & 4) != 0);
    pstep<2>(v, (lane & 2) != 0);
    pstep<1>(v, (lane & 1) != 0);
    float sum = v[0] + __shfl_xor(v[0], 16, kWave);
    sum += __shfl_xor(sum, 32, kWave);
    if (lane < kPRW * kPT) {
      const int i = lane / kPT, tt = lane % kPT;
      if (n0 + i < R && t0 + tt < T) z[(size_t)(t0 + tt) * R + n0 + i] = sum;
    }
    if (zpart) {
      float m = lane < kPRW * kPT ? fabsf(sum) : 0.f;
      m = fmaxf(m, __shfl_xor(m, 4, kWave));
      m = fmaxf(m, __shfl_xor(m, 8, kWave));
      if (lane < kPT) wmx[wv][lane] = m;
      __syncthreads();
      const int tt = threadIdx.x;
      if (tt < kPT && t0 + tt < T) {
        const float mm = fmaxf(fmaxf(wmx[0][tt], wmx[1][tt]), fmaxf(wmx[2][tt], wmx[3][tt]));
        zpart[(size_t)(t0 + tt) * nproj + blockIdx.x] = mm;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Expert apply over one 32-row segment, lane = row (a wave covers two
// segments).  For every slot (width groups 1..8 then 16, ascending k inside
// a group, zero padding slots contribute nothing):
//   y += (a z s) q + (a z m)     for 1..8-bit columns
//   y += (a z) p16               for 16-bit columns.
// Returns false when the blob or the expert id cannot be used.
// ---------------------------------------------------------------------------
__device__ float apply_seg(const uint8_t* __restrict__ blob, uint64_t blob_bytes, int e, int E,
                           int dout, int r, const float* __restrict__ zrow, int seg, int row,
                           bool& ok) {
  DirRec d;
  if (!load_dir(blob, blob_bytes, e, E, dout, r, d)) {
    ok = false;
    return 0.f;
  }
  const uint8_t* blk = blob + d.block_offset;
  const uint16_t* kidx = reinterpret_cast<const uint16_t*>(blk);
  const float* A = reinterpret_cast<const float*>(blk + d.a_off);
  const __half* S = reinterpret_cast<const __half*>(blk + d.s_off);
  const __half* M = reinterpret_cast<const __half*>(blk + d.m_off);
  const uint32_t* rec =
      reinterpret_cast<const uint32_t*>(blk + d.planes_off) + (size_t)seg * d.seg_words;
  const SlotGeo geo = slot_geo(d.count);
  float acc = 0.f, bias = 0.f;
  uint32_t slot = 0, word = 0;
  bool good = true;
  for (int g = 0; g < kNumGroups; ++g) {
    const int w = kGroupWidth[g];
    for (uint32_t b = 0; b < geo.nb[g]; ++b, slot += 4, word += 4u * w) {
      for (int u = 0; u < 4; ++u) {
        uint32_t k = kidx[slot + u];
        good &= k < (uint32_t)r;
        k = k < (uint32_t)r ? k : 0;
        const float az = A[slot + u] * zrow[k];
        if (w == 16) {
          acc += az * __half2float(__ushort_as_half((unsigned short)decode_f16(rec + word, row, u)));
        } else {
          bias += az * __half2float(M[slot + u]);
          acc += (az * __half2float(S[slot + u])) * (float)decode_code(rec + word, w, row, u);
        }
      }
    }
  }
  ok = good;
  return acc + bias;
}

// grid (T*k, ceil(n_seg / 2)); block 64 (apply) or 128 (gate wave + up wave).
template <bool kGateUp>
__global__ __launch_bounds__(kGateUp ? 128 : 64) void k_expert_seg(
    const uint8_t* __restrict__ blob_g, uint64_t bytes_g, const uint8_t* __restrict__ blob_u,
    uint64_t bytes_u, int E, int dout, int r, const float* __restrict__ z, int z_stride,
    int z_off_up, const int32_t* __restrict__ ids, int ktop, float* __restrict__ out) {
  const int pair = blockIdx.x;
  const int lane = threadIdx.x & (kWave - 1);
  const int wv = threadIdx.x >> 6;
  const int seg = 2 * (int)blockIdx.y + (lane >> 5);
  const int row = lane & 31;
  const int orow = seg * kSegRows + row;
  const int t = pair / ktop;
  const int e = ids[pair];
  bool ok = true;
  const uint8_t* blob = wv ? blob_u : blob_g;
  const uint64_t bytes = wv ? bytes_u : bytes_g;
  const float* zrow = z + (size_t)t * z_stride + (wv ? z_off_up : 0);
  const bool live = orow < dout;
  const float y = live ? apply_seg(blob, bytes, e, E, dout, r, zrow, seg, row, ok) : 0.f;
  if (!kGateUp) {
    if (live) out[(size_t)pair * dout + orow] = ok ? y : __builtin_nanf("");
    return;
  }
  __shared__ float s_y[kWave];
  __shared__ int s_ok[kWave];
  if (wv == 1) {
    s_y[lane] = y;
    s_ok[lane] = ok;
  }
  __syncthreads();
  if (wv == 0 && live)
    out[(size_t)pair * dout + orow] =
        (ok && s_ok[lane]) ? silu_mul(y, s_y[lane]) : __builtin_nanf("");
}

// grid (ceil(n_seg / 2)); block 64: codes of expert e in k order as the
// lane-per-row decoder of k_expert_seg reads them (0-bit columns are left as
// the caller's zero fill; padding slots are skipped).
__global__ __launch_bounds__(64) void k_dump_codes(const uint8_t* __restrict__ blob,
                                                   uint64_t blob_bytes, int E, int dout, int r,
                                                   int e, uint16_t* __restrict__ codes) {
  DirRec d;
  const int lane = threadIdx.x;
  const int seg = 2 * (int)blockIdx.x + (lane >> 5);
  const int row = lane & 31;
  const int orow = seg * kSegRows + row;
  if (orow >= dout) return;
  if (!load_dir(blob, blob_bytes, e, E, dout, r, d)) {
    for (int k = 0; k < r; ++k) codes[(size_t)k * dout + orow] = 0xFFFFu;
    return;
  }
  const uint8_t* blk = blob + d.block_offset;
  const uint16_t* kidx = reinterpret_cast<const uint16_t*>(blk);
  const uint32_t* rec =
      reinterpret_cast<const uint32_t*>(blk + d.planes_off) + (size_t)seg * d.seg_words;
  const SlotGeo geo = slot_geo(d.count);
  uint32_t slot = 0, word = 0;
  for (int g = 0; g < kNumGroups; ++g) {
    const int w = kGroupWidth[g];
    for (uint32_t b = 0; b < geo.nb[g]; ++b, slot += 4, word += 4u * w) {
      for (int u = 0; u < 4; ++u) {
        if (4 * b + u >= d.count[g]) continue;  // padding slot
        const uint32_t k = kidx[slot + u];
        const uint32_t q = w == 16 ? decode_f16(rec + word, row, u)
                                   : decode_code(rec + word, w, row, u);
        if (k < (uint32_t)r) codes[(size_t)k * dout + orow] = (uint16_t)q;
      }
    }
  }
}

// Codes as the MFMA kernels' operand builders produce them.  grid (n_seg);
// block 64 (one wave per 32-row segment, read straight from the blob).
//  kPath 0: the one-launch kernel's int8 apply: a_i8<W> for widths 1..8 (the
//           A byte: the code, width 8: code ^ 0x80), a_tiles_f16 for 16-bit
//           slots, in that kernel's 64-slot steps (the last, odd K32 step
//           of a group taken as a half step);
//  kPath 1: the batched kernel's fp16 apply: a_tiles_uniform<W> (fp16 of the
//           code through codes_to_f16) and a_tiles_f16, in 32-slot steps.
// Each lane scatters the operand elements it holds to codes[k * dout + row]
// (k = the slot's component index); padding slots are skipped.
template <int kPath>
__global__ __launch_bounds__(64) void k_dump_operands(const uint8_t* __restrict__ blob,
                                                      uint64_t blob_bytes, int E, int dout, int r,
                                                      int e, uint16_t* __restrict__ codes) {
  using namespace seg;
  const int lane = threadIdx.x, seg_i = blockIdx.x;
  const DirRec d = load_rec_s(blob, e, E);
  const SegProj p = uniform_seg(make_seg(blob, blob_bytes, e, d, load_hdr(blob), E, dout, r));
  if (!p.ok) {
    const int orow = seg_i * kSegRows + (lane & 31);
    if (orow < dout)
      for (int k = lane >> 5; k < r; k += 2) codes[(size_t)k * dout + orow] = 0xFFFFu;
    return;
  }
  // (generic pointers into the blob, as the kernels' LDS copies are read)
  const uint32_t* base = (const uint32_t*)(p.planes + (size_t)seg_i * p.seg_words);
  const gu16* kidx = p.kidx;
  const int m = lane & 15, q = lane >> 4;
  const uint32_t gb[kNumGroups + 1] = {0u, p.b1, p.b2, p.b3, p.b4, p.b5, p.b6, p.n_blk};
  const uint32_t gw[kNumGroups] = {0u, p.w1, p.w2, p.w3, p.w4, p.w5, p.w6};
  // element (block blk of the segment's block list, slot u, row 16 tile + m)
  auto put = [&](int g, uint32_t blk, int u, int tile, uint32_t v) {
    if (4u * (blk - gb[g]) + (uint32_t)u >= d.count[g]) return;  // padding slot
    const uint32_t k = kidx[4u * blk + (uint32_t)u];
    const int orow = seg_i * kSegRows + 16 * tile + m;
    if (k < (uint32_t)r && orow < dout) codes[(size_t)k * dout + orow] = (uint16_t)v;
  };
  // fp16 operands of K32 step kb: this lane's blocks 8 kb + 2 q + t, element
  // 4 t + u of tile `tile`
  auto put_h8 = [&](int g, uint32_t kb, const h8& a0, const h8& a1) {
    const uint4 v0 = __builtin_bit_cast(uint4, a0), v1 = __builtin_bit_cast(uint4, a1);
    const uint32_t w0[4] = {v0.x, v0.y, v0.z, v0.w}, w1[4] = {v1.x, v1.y, v1.z, v1.w};
    for (int j = 0; j < 8; ++j) {
      const uint32_t blk = 8u * kb + 2u * (uint32_t)q + (uint32_t)(j >> 2);
      put(g, blk, j & 3, 0, (w0[j >> 1] >> (16 * (j & 1))) & 0xFFFFu);
      put(g, blk, j & 3, 1, (w1[j >> 1] >> (16 * (j & 1))) & 0xFFFFu);
    }
  };
  auto f16_steps = [&](int g, auto wc) {
    constexpr int W = decltype(wc)::value;
    constexpr uint32_t bw = 4u * (uint32_t)W;
    for (uint32_t kb = gb[g] / kBlkPerK; kb < gb[g + 1] / kBlkPerK; ++kb) {
      const uint32_t* rec0 = base + gw[g] + (kBlkPerK * kb - gb[g]) * bw + 2u * bw * (uint32_t)q;
      h8 a0, a1;
      if constexpr (W == 16)
        a_tiles_f16(rec0, m, a0, a1);
      else
        a_tiles_uniform<W>(rec0, m, a0, a1);
      put_h8(g, kb, a0, a1);
    }
  };
  auto i8_steps = [&](int g, auto wc) {
    constexpr int W = decltype(wc)::value;
    const uint32_t s = gb[g] / kBlkPerK, e_ = gb[g + 1] / kBlkPerK;
    for (uint32_t k = s; k < e_; k += 2) {
      if (!(q < 2 || k + 1 < e_)) continue;  // upper half of a trailing half step
      const uint32_t* rec = base + gw[g] + (8u * k + 4u * (uint32_t)q - gb[g]) * 4u * W;
      for (int tile = 0; tile < 2; ++tile) {
        const i32x4 a = a_i8<W>(rec, m, tile);
        for (int dd = 0; dd < 4; ++dd)
          for (int u = 0; u < 4; ++u)
            put(g, 8u * k + 4u * (uint32_t)q + (uint32_t)dd, u, tile,
                ((uint32_t)a[dd] >> (8 * u)) & 0xFFu);
      }
    }
  };
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;
  using I4 = std::integral_constant<int, 4>;
  using I6 = std::integral_constant<int, 6>;
  using I8 = std::integral_constant<int, 8>;
  using I16 = std::integral_constant<int, 16>;
  if constexpr (kPath == 0) {
    i8_steps(0, I1{});
    i8_steps(1, I2{});
    i8_steps(2, I3{});
    i8_steps(3, I4{});
    i8_steps(4, I6{});
    i8_steps(5, I8{});
  } else {
    f16_steps(0, I1{});
    f16_steps(1, I2{});
    f16_steps(2, I3{});
    f16_steps(3, I4{});
    f16_steps(4, I6{});
    f16_steps(5, I8{});
  }
  f16_steps(6, I16{});
}

__global__ __launch_bounds__(256) void k_zero_fill(uint4* __restrict__ p, size_t n16,
                                                   uint8_t* __restrict__ tail, int ntail) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride)
    p[i] = make_uint4(0, 0, 0, 0);
  if (blockIdx.x == 0 && (int)threadIdx.x < ntail) tail[threadIdx.x] = 0;
}

// ---------------------------------------------------------------------------
// host helpers
// ---------------------------------------------------------------------------
bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int launch_status(const char* what) {
  const hipError_t err = hipGetLastError();
  if (err != hipSuccess) return fail(BITSMOE_EHIP, "%s: %s", what, hipGetErrorString(err));
  return BITSMOE_OK;
}

int check_blob_arg(const void* blob, size_t bytes, int E, int r, const char* name) {
  if (!blob) return fail(BITSMOE_EINVAL, "%s is null", name);
  if (!aligned16(blob)) return fail(BITSMOE_EINVAL, "%s is not 16-byte aligned", name);
  if (bytes < first_block_offset((uint64_t)E, (uint64_t)r))
    return fail(BITSMOE_ENOSPC, "%s: %zu bytes cannot hold header, directory and slot index",
                name, bytes);
  return BITSMOE_OK;
}

int check_layer_dims(int E, int dout, int r) {
  if (E <= 0 || dout <= 0 || r <= 0)
    return fail(BITSMOE_ESHAPE, "E=%d dout=%d r=%d must be positive", E, dout, r);
  if (r > 65535) return fail(BITSMOE_ESHAPE, "r=%d exceeds 65535", r);
  if (dout > (1 << 24)) return fail(BITSMOE_ESHAPE, "dout=%d too large", dout);
  return BITSMOE_OK;
}

int proj_args(const void* phi, const void* x, const float* z, int T, int din, int R) {
  if (!phi || !x || !z) return fail(BITSMOE_EINVAL, "null pointer argument");
  if (!aligned16(phi) || !aligned16(x) || !aligned16(z))
    return fail(BITSMOE_EINVAL, "phi, x and z must be 16-byte aligned");
  if (T < 1) return fail(BITSMOE_EINVAL, "T=%d < 1", T);
  if (din <= 0 || R <= 0) return fail(BITSMOE_ESHAPE, "din=%d r_total=%d", din, R);
  if (din % 8) return fail(BITSMOE_ESHAPE, "din=%d is not a multiple of 8", din);
  return BITSMOE_OK;
}

// z = Phi^T x; zpart (may be null; din <= 4096 only) gets max |z| per
// 16-row work-group and token.  A route job (may be null) runs in the same
// launch when the projection takes the matrix-core kernel and E <=
// kRouteFuseMaxE; *routed tells whether it did.
int launch_proj(const void* phi, const void* x, float* z, float* zpart, int T, int din, int R,
                hipStream_t s, const RouteJob* route = nullptr, bool* routed = nullptr,
                bool x_f32 = false) {
  const int din8 = din / 8;
  if (routed) *routed = false;
  if (x_f32 && ((T >= 16 && din % 32 == 0) || din8 > kPMaxU * kWave || ((uintptr_t)x & 15u)))
    return fail(BITSMOE_EINVAL, "float32 x needs T < 16 or din %% 32 != 0, din <= 4096, 16-byte x");
  if (T >= 64 && din % kQK == 0 && !x_f32) {  // (x_f32 is refused above for T >= 16)
    const int nzp = (R + kProjRowsPerBlock - 1) / kProjRowsPerBlock;
    RouteJob rj{};
    const bool fuse = route && route->E <= kRouteFuseMaxE;
    if (fuse) rj = *route;
    // (row blocks grouped by XCD, each with all of its token tiles; one
    // more work-group for the route job)
    const long long nmb = (R + kQM - 1) / kQM, ntb = (T + kQN - 1) / kQN;
    const long long nmain = 8 * ((nmb + 7) / 8) * ntb;
    hipLaunchKernelGGL(k_proj_gemm, dim3((unsigned)(nmain + (fuse ? 1 : 0))),
                       dim3(kQWaves * kWave), 0, s, (const uint4*)phi, (const uint4*)x, z, zpart,
                       T, din8, R, nzp, rj);
    if (routed) *routed = fuse;
    return launch_status("spectral projection launch");
  }
  if (T >= 16 && din % 32 == 0) {
    const int nzp = (R + kProjRowsPerBlock - 1) / kProjRowsPerBlock;
    RouteJob rj{};
    const bool fuse = route && route->E <= kRouteFuseMaxE;
    if (fuse) rj = *route;
    hipLaunchKernelGGL(k_proj_mfma,
                       dim3((unsigned)(nzp + (fuse ? 1 : 0)),
                            (unsigned)((T + 16 * kPMBlocks - 1) / (16 * kPMBlocks))),
                       dim3(kPMWaves * kWave), 0, s, (const uint4*)phi, (const uint4*)x, z, zpart,
                       T, din8, R, nzp, rj);
    if (routed) *routed = fuse;
    return launch_status("spectral projection launch");
  }
  const uint4* p4 = (const uint4*)phi;
  const uint4* x4 = (const uint4*)x;
  const dim3 block(kProjWaves * kWave);
  if (din8 <= kPMaxU * kWave) {
    RouteJob rj{};
    const bool fuse = route && route->E <= kRouteFuseMaxE;
    if (fuse) rj = *route;
    const dim3 grid((R + kProjWaves * kPRW - 1) / (kProjWaves * kPRW) + (fuse ? 1 : 0));
#define PROJ_ROWS(U)                                                                         \
  hipLaunchKernelGGL((x_f32 ? k_proj_rows<U, true> : k_proj_rows<U, false>), grid, block, 0, s, \
                     p4, x, z, zpart, T, din8, R, rj)
    if (din8 <= kWave)
      PROJ_ROWS(1);
    else if (din8 <= 2 * kWave)
      PROJ_ROWS(2);
    else if (din8 <= 4 * kWave)
      PROJ_ROWS(4);
    else
      PROJ_ROWS(8);
#undef PROJ_ROWS
    if (routed) *routed = fuse;
  } else
    hipLaunchKernelGGL(k_proj_gemv, dim3((R + kProjWaves - 1) / kProjWaves), block, 0, s, p4,
                       x4, z, T, din8, R);
  return launch_status("spectral projection launch");
}


}  // namespace

int launch_proj_maxima(const void* phi, const void* x, float* z, float* zpart, int T, int din,
                       int R, hipStream_t st, const RouteJob* route, bool* routed, bool x_f32) {
  return launch_proj(phi, x, z, zpart, T, din, R, st, route, routed, x_f32);
}

// Per-tile coefficient tables: hi and lo rows (with 256 slots of slack for
// the last row's 16-byte copies), the chunk sums and the flags.
size_t group_coef_bytes(int tcap, int r) {
  const size_t rpad = (size_t)group_rpad(r), nck = rpad / 256;
  const size_t rows = (size_t)tcap * 2 * kTile;
  return 2 * align_up(rows * rpad * 2 + 512, 256) + align_up((size_t)tcap * 2 * nck * kTile * 4, 256) +
         align_up((size_t)tcap * 2 * 4, 256) + align_up(rows * 4, 256);
}

void group_coef_tables(GroupArgs& gs, uint8_t* base, int r) {
  const size_t rpad = (size_t)group_rpad(r), nck = rpad / 256;
  const size_t rows = (size_t)gs.tcap * 2 * kTile;
  const size_t hb = align_up(rows * rpad * 2 + 512, 256);
  gs.thi = (_Float16*)base;
  gs.tlo = (_Float16*)(base + hb);
  gs.tbias = (float*)(base + 2 * hb);
  gs.tbad = (uint32_t*)(base + 2 * hb + align_up((size_t)gs.tcap * 2 * nck * kTile * 4, 256));
  gs.tsh = (int*)((uint8_t*)gs.tbad + align_up((size_t)gs.tcap * 2 * 4, 256));
  gs.rpad = (int)rpad;
  gs.nck = (int)nck;
}

int tile_cap(int T, int k, int E) {
  const long long P = (long long)T * k;
  const long long g = P < E ? P : E;
  const long long cap = g + (P + kTile - 1) / kTile;
  return (int)((cap + 7) / 8 * 8);
}

GateUpPlan gateup_plan(int T, int k, int E, int r) {
  GateUpPlan p;
  const size_t P = (size_t)T * k;
  const size_t nzp = ((size_t)2 * r + kProjRowsPerBlock - 1) / kProjRowsPerBlock;
  p.sync_off = 0;
  p.z_off = align_up(kSyncBytes, 256);
  p.zpart_off = align_up(p.z_off + (size_t)T * 2 * r * sizeof(float), 256);
  p.zt_off = align_up(p.zpart_off + (size_t)T * nzp * sizeof(float), 256);
  p.cw_off = align_up(p.zt_off + (size_t)kZRing * T * 2 * r * sizeof(uint64_t), 256);
  const size_t ncw = T == 1 && k <= kOneMaxK && r <= kOneMaxR
                         ? (size_t)kZRing * k * 2 * ((size_t)kOneSlots + r) * sizeof(uint64_t)
                         : 0;
  p.route_off = align_up(p.cw_off + ncw, 256);
  p.coef_off = align_up(p.route_off + route_ints(tile_cap(T, k, E), P) * sizeof(int), 256);
  p.total = p.coef_off + group_coef_bytes(tile_cap(T, k, E), r);
  return p;
}

}  // namespace bitsmoe

using namespace bitsmoe;

extern "C" {

int bitsmoe_spectral_proj(const void* phi_t_f16, const void* x_f16, float* z, int T, int din,
                          int r_total, bitsmoe_stream_t stream) {
  int st = proj_args(phi_t_f16, x_f16, z, T, din, r_total);
  if (st) return st;
  return launch_proj(phi_t_f16, x_f16, z, nullptr, T, din, r_total, (hipStream_t)stream);
}

int bitsmoe_expert_apply(const void* packed, size_t packed_bytes, int E, int dout, int r,
                         const float* z, int z_stride, const int32_t* ids, int T, int k,
                         float* y, void* ws, size_t ws_bytes, bitsmoe_stream_t stream) {
  (void)ws;
  (void)ws_bytes;
  int st = check_layer_dims(E, dout, r);
  if (st) return st;
  if ((st = check_blob_arg(packed, packed_bytes, E, r, "packed"))) return st;
  if (!z || !ids || !y) return fail(BITSMOE_EINVAL, "null pointer argument");
  if (!aligned16(z) || !aligned16(y) || ((uintptr_t)ids & 3u))
    return fail(BITSMOE_EINVAL, "misaligned z, y or ids");
  if (T < 1 || k < 1 || k > E) return fail(BITSMOE_EINVAL, "T=%d k=%d E=%d", T, k, E);
  if (z_stride < r) return fail(BITSMOE_ESHAPE, "z_stride=%d < r=%d", z_stride, r);
  if ((long long)T * k > (1LL << 24))
    return fail(BITSMOE_ESHAPE, "T*k=%lld too large", (long long)T * k);
  const int n_pairs_seg = (dout + 2 * kSegRows - 1) / (2 * kSegRows);
  hipLaunchKernelGGL(k_expert_seg<false>, dim3(T * k, n_pairs_seg), dim3(64), 0,
                     (hipStream_t)stream, (const uint8_t*)packed, (uint64_t)packed_bytes,
                     (const uint8_t*)packed, (uint64_t)packed_bytes, E, dout, r, z, z_stride, 0,
                     ids, k, y);
  return launch_status("expert apply launch");
}

int bitsmoe_moe_gateup_workspace_size(int T, int k, int E, int din, int dout, int r,
                                      size_t* bytes) {
  if (!bytes) return fail(BITSMOE_EINVAL, "bytes is null");
  int st = check_layer_dims(E, dout, r);
  if (st) return st;
  if (T < 1 || k < 1 || k > E) return fail(BITSMOE_EINVAL, "T=%d k=%d E=%d", T, k, E);
  if (din <= 0 || din % 8) return fail(BITSMOE_ESHAPE, "din=%d", din);
  *bytes = gateup_plan(T, k, E, r).total;
  return BITSMOE_OK;
}

}  // extern "C"

namespace {
// Host checks of a gate/up call.  static_ws: the workspace is the library's
// static array (ws is not checked; ws_bytes is its size).
int gateup_checks(const void* packed_gate, size_t gate_bytes, const void* packed_up,
                  size_t up_bytes, const void* phi_t_gateup_f16, const void* x_f16,
                  const int32_t* ids, int T, int k, int E, int din, int dout, int r,
                  const float* h, const void* ws, size_t ws_bytes, bool static_ws) {
  int st = check_layer_dims(E, dout, r);
  if (st) return st;
  if ((st = check_blob_arg(packed_gate, gate_bytes, E, r, "packed_gate"))) return st;
  if ((st = check_blob_arg(packed_up, up_bytes, E, r, "packed_up"))) return st;
  if (!ids || !h || (!static_ws && !ws)) return fail(BITSMOE_EINVAL, "null pointer argument");
  if (!aligned16(h) || (!static_ws && !aligned16(ws)) || ((uintptr_t)ids & 3u))
    return fail(BITSMOE_EINVAL, "misaligned h, ws or ids");
  if (k < 1 || k > E) return fail(BITSMOE_EINVAL, "k=%d E=%d", k, E);
  if ((st = proj_args(phi_t_gateup_f16, x_f16, h, T, din, 2 * r))) return st;
  if ((long long)T * k > (1LL << 24))
    return fail(BITSMOE_ESHAPE, "T*k=%lld too large", (long long)T * k);
  size_t need = 0;
  bitsmoe_moe_gateup_workspace_size(T, k, E, din, dout, r, &need);
  if (ws_bytes < need)
    return fail(BITSMOE_ENOSPC, static_ws ? "needs %zu bytes of workspace, above the %zu of "
                "the static one: use bitsmoe_moe_gateup with a workspace" : "ws_bytes=%zu < %zu",
                static_ws ? need : ws_bytes, static_ws ? ws_bytes : need);
  return BITSMOE_OK;
}
}  // namespace

extern "C" {

int bitsmoe_moe_gateup(const void* packed_gate, size_t gate_bytes, const void* packed_up,
                       size_t up_bytes, const void* phi_t_gateup_f16, const void* x_f16,
                       const int32_t* ids, int T, int k, int E, int din, int dout, int r,
                       float* h, void* ws, size_t ws_bytes, bitsmoe_stream_t stream) {
  int st = gateup_checks(packed_gate, gate_bytes, packed_up, up_bytes, phi_t_gateup_f16, x_f16,
                         ids, T, k, E, din, dout, r, h, ws, ws_bytes, false);
  if (st) return st;
  const GateUpPlan plan = gateup_plan(T, k, E, r);
  hipStream_t s = (hipStream_t)stream;
  uint8_t* wsb = (uint8_t*)ws;
  GateUpArgs a;
  a.blob_g = (const uint8_t*)packed_gate;
  a.blob_u = (const uint8_t*)packed_up;
  a.bytes_g = gate_bytes;
  a.bytes_u = up_bytes;
  a.E = E;
  a.dout = dout;
  a.r = r;
  a.ids = ids;
  a.ktop = k;
  a.npairs = T * k;
  a.h = h;
  a.n_seg = (dout + kSegRows - 1) / kSegRows;
  float* z = (float*)(wsb + plan.z_off);
  // One launch when every work-group can be resident at once (the groups
  // wait for each other's z); otherwise z first, then the expert kernels.
  const int fgrid = fused_grid();
  // (both one-launch kernels add 4 per work-group to the shared hint
  // counters, so they must use the same grid)
  const int ogrid = one_grid();
  const bool one = T == 1 && k <= kOneMaxK && r <= kOneMaxR && r % 4 == 0 &&
                   din <= kOneMaxDin && ogrid > 0 && ogrid == fgrid && 2 * r <= 32 * ogrid &&
                   (long long)k * a.n_seg <= ogrid;
  if (one || (T <= kFusedMaxTokens && r <= kFusedMaxR && fgrid > 0)) {
    FusedArgs fa;
    fa.g = a;
    fa.phi_t = (const uint4*)phi_t_gateup_f16;
    fa.x = (const uint4*)x_f16;
    fa.din8 = din / 8;
    fa.T = T;
    fa.zt = (uint64_t*)(wsb + plan.zt_off);
    fa.cw = (uint64_t*)(wsb + plan.cw_off);
    fa.bw = fa.cw + (size_t)kZRing * k * 2 * kOneSlots;
    fa.epoch = (uint32_t*)(wsb + plan.sync_off);
    fa.hint = fa.epoch + 32;
    fa.timeouts = fa.epoch + 1;
    fa.grid = fgrid;
    fa.spin = g_wait_limit.load(std::memory_order_relaxed);
    if (one)
      launch_gateup_one(fa, s);
    else
      launch_gateup_fused(fa, s);
    return launch_status("one-launch gate/up");
  }
  const bool grouped = r <= kGroupMaxR && E <= kGroupMaxE && din <= kGroupMaxDin;
  float* zpart = grouped ? (float*)(wsb + plan.zpart_off) : nullptr;
  if (!grouped) {
    if ((st = launch_proj(phi_t_gateup_f16, x_f16, z, zpart, T, din, 2 * r, s))) return st;
  } else {
    // batched tokens: pairs grouped by expert, each expert's planes read and
    // unpacked once per tile of up to 16 tokens
    GroupArgs gs;
    gs.g = a;
    gs.z = z;
    gs.zpart = zpart;
    gs.nzp = (2 * r + kProjRowsPerBlock - 1) / kProjRowsPerBlock;
    gs.tcap = tile_cap(T, k, E);
    gs.single = 0;
    route_lists_at(gs.rl, (int*)(wsb + plan.route_off), gs.tcap, (size_t)T * k);
    group_coef_tables(gs, wsb + plan.coef_off, r);
    const RouteJob rj{ids, T * k, E, dout, h, gs.rl, gs.tbad, gs.tcap * 2};
    bool routed = false;
    if ((st = launch_proj(phi_t_gateup_f16, x_f16, z, zpart, T, din, 2 * r, s, &rj, &routed)))
      return st;
    if (!routed) {
      launch_route_group(ids, T * k, E, dout, h, gs.rl, s, gs.tbad, gs.tcap * 2);
      if ((st = launch_status("route grouping launch"))) return st;
    }
    launch_group_coef(gs, s);
    if ((st = launch_status("tile coefficient launch"))) return st;
    launch_gateup_grouped(gs, s);
    return launch_status("grouped gate/up launch");
  }
  hipLaunchKernelGGL(k_expert_seg<true>,
                     dim3(T * k, (a.n_seg + 1) / 2), dim3(128), 0, s, a.blob_g, a.bytes_g,
                     a.blob_u, a.bytes_u, E, dout, r, (const float*)z, 2 * r, r, ids, k, h);
  return launch_status("gate/up expert launch");
}

int bitsmoe_workspace_init(void* ws, size_t ws_bytes, bitsmoe_stream_t stream) {
  if (!ws) return fail(BITSMOE_EINVAL, "ws is null");
  if (!aligned16(ws)) return fail(BITSMOE_EINVAL, "ws is not 16-byte aligned");
  const size_t n16 = ws_bytes / 16;
  const int ntail = (int)(ws_bytes % 16);
  size_t blocks = (n16 + 255) / 256;
  if (blocks < 1) blocks = 1;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(k_zero_fill, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream,
                     (uint4*)ws, n16, (uint8_t*)ws + n16 * 16, ntail);
  return launch_status("workspace fill launch");
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Allocation-free gate/up: the workspace is this file-scope array, one copy
// per device, kept (with the one-launch kernel's counters in its first bytes)
// until the process ends.  Host code never passes `scratch` itself to a
// kernel (on the host it only names the symbol): it uses the device address
// hipGetSymbolAddress returns, looked up once per device.
// ---------------------------------------------------------------------------
constexpr size_t kScratchBytes = BITSMOE_GATEUP_NOALLOC_MAX_WS;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {
constexpr int kScratchMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kScratchMaxDevices];

// Device address of this device's scratch array.  The first call on a device
// looks it up and zero-fills it on `s` (work enqueued after it on any stream
// of that device must come after that fill, as with bitsmoe_workspace_init).
int scratch_for_current_device(hipStream_t s, void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(BITSMOE_EHIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kScratchMaxDevices)
    return fail(BITSMOE_EHIP, "device %d outside [0,%d)", dev, kScratchMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(BITSMOE_EHIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
    const int st = bitsmoe_workspace_init(p, kScratchBytes, (bitsmoe_stream_t)s);
    if (st) return st;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return BITSMOE_OK;
}
}  // namespace

extern "C" {

int bitsmoe_moe_gateup_noalloc(const void* packed_gate, size_t gate_bytes, const void* packed_up,
                               size_t up_bytes, const void* phi_t_gateup_f16, const void* x_f16,
                               const int32_t* ids, int T, int k, int E, int din, int dout, int r,
                               float* h, bitsmoe_stream_t stream) {
  int st = gateup_checks(packed_gate, gate_bytes, packed_up, up_bytes, phi_t_gateup_f16, x_f16,
                         ids, T, k, E, din, dout, r, h, nullptr, kScratchBytes, true);
  if (st) return st;
  void* ws = nullptr;
  if ((st = scratch_for_current_device((hipStream_t)stream, &ws))) return st;
  return bitsmoe_moe_gateup(packed_gate, gate_bytes, packed_up, up_bytes, phi_t_gateup_f16,
                            x_f16, ids, T, k, E, din, dout, r, h, ws, kScratchBytes, stream);
}

uint32_t bitsmoe_debug_set_wait_limit(uint32_t spins) {
  return g_wait_limit.exchange(spins);
}

int bitsmoe_wait_timeouts(const void* ws, size_t ws_bytes, uint32_t* count,
                          bitsmoe_stream_t stream) {
  if (!count) return fail(BITSMOE_EINVAL, "count is null");
  hipStream_t s = (hipStream_t)stream;
  const uint8_t* w = (const uint8_t*)ws;
  if (!w) {
    void* p = nullptr;
    const int st = scratch_for_current_device(s, &p);
    if (st) return st;
    w = (const uint8_t*)p;
  } else if (ws_bytes < kSyncBytes) {
    return fail(BITSMOE_EINVAL, "ws_bytes=%zu below the %zu bytes of the sync words", ws_bytes,
                kSyncBytes);
  }
  // word 1 of the sync line (the epoch is word 0, the hint counters follow)
  hipError_t e = hipMemcpyAsync(count, w + sizeof(uint32_t), sizeof(uint32_t),
                                hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return fail(BITSMOE_EHIP, "reading the time-out count: %s",
                                   hipGetErrorString(e));
  return BITSMOE_OK;
}

int bitsmoe_dump_codes(const void* packed, size_t packed_bytes, int E, int dout, int r, int e,
                       int path, uint16_t* codes, bitsmoe_stream_t stream) {
  int st = check_layer_dims(E, dout, r);
  if (st) return st;
  if ((st = check_blob_arg(packed, packed_bytes, E, r, "packed"))) return st;
  if (!codes) return fail(BITSMOE_EINVAL, "codes is null");
  if (!aligned16(codes)) return fail(BITSMOE_EINVAL, "codes is not 16-byte aligned");
  if (e < 0 || e >= E) return fail(BITSMOE_EINVAL, "e=%d outside [0,%d)", e, E);
  if (path < 0 || path > 2) return fail(BITSMOE_EINVAL, "path=%d outside [0,2]", path);
  hipStream_t s = (hipStream_t)stream;
  if ((st = bitsmoe_workspace_init(codes, (size_t)r * dout * 2, stream))) return st;
  const int n_seg = (dout + kSegRows - 1) / kSegRows;
  const uint8_t* b = (const uint8_t*)packed;
  if (path == 0)
    hipLaunchKernelGGL(k_dump_operands<0>, dim3(n_seg), dim3(64), 0, s, b,
                       (uint64_t)packed_bytes, E, dout, r, e, codes);
  else if (path == 1)
    hipLaunchKernelGGL(k_dump_operands<1>, dim3(n_seg), dim3(64), 0, s, b,
                       (uint64_t)packed_bytes, E, dout, r, e, codes);
  else
    hipLaunchKernelGGL(k_dump_codes, dim3((n_seg + 1) / 2), dim3(64), 0, s, b,
                       (uint64_t)packed_bytes, E, dout, r, e, codes);
  return launch_status("code dump launch");
}

}  // extern "C"
