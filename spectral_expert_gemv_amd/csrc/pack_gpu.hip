// Device packer: quantizes and packs one linear type of a layer on the GPU
// and writes the same blob bytes as the host packer (format v3).
//
// BitsMoE blog note, Methodology: "second split" (unit directions p_{e,k}
// with magnitudes a_{e,k}), "Usage" (widths {0,1,2,3,4,6,8,16}) and
// "execution" (columns of one width stored together, plane by plane).
//
// gfx950 mapping.
//  * The host plans the layout from the widths (directory records, block
//    offsets, slot -> column order; the same planner as the host packer)
//    and copies the directory and the slot table to the device.
//  * k_pack_blocks: one wave per 4-slot block.  For 1..8-bit columns the
//    wave reduces min and max of its 4 columns over the rows, forms the fp16
//    scale and offset exactly as the host quantizer does (IEEE float32, no
//    contraction), then walks the rows 16 at a time: lane (octet half,
//    slot u, row rho) holds one code, and one 64-lane ballot per plane
//    yields the plane words of two row octets at once (bit 8u + rho of a
//    word is bit j of the code of row rho in slot u).  16-bit columns store
//    fp16 pairs directly.  The per-expert coefficient bound is an atomic max
//    on the record's float bits (all bounds are >= 0).
//  * k_crc_chunks: the CRC-32 of [128, total) in 4 KiB chunks, one lane
//    each (slicing by 4 with LDS tables, register start value 0); the host
//    folds the chunk values in order (a chunk's register value is linear in
//    the start value: appending n bytes multiplies it by x^(8n) modulo the
//    polynomial) and writes the header.
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>
#include <math.h>
#include <string.h>

#include <algorithm>
#include <vector>

#include "bitsmoe.h"
#include "common.h"
#include "format.h"
#include "pack_plan.h"

#pragma clang fp contract(off)

namespace bitsmoe {
namespace {

constexpr int kPkWaves = 4;                   // 4-slot blocks per work-group
constexpr int kPkB = 8;                       // 16-row steps per batch of loads
constexpr uint32_t kCrcChunk = 4096;          // bytes per CRC lane
constexpr uint32_t kCrcPoly = 0xEDB88320u;    // IEEE polynomial, reflected
constexpr float kPMax = 60000.0f;             // largest |p| the format accepts

enum : uint32_t { kBadP = 1u, kBadA = 2u };

__device__ __forceinline__ uint16_t f16_bits(float x) {
  return __half_as_ushort(__float2half_rn(x));
}
__device__ __forceinline__ float f16_val(uint16_t b) {
  return __half2float(__ushort_as_half(b));
}

// Minimum with -0 below +0 (IEEE minimum): the sign of a zero minimum does
// not depend on the reduction order.
__device__ __forceinline__ float min_signed(float v, float o) {
  return (o < v || (o == v && signbit(o))) ? o : v;
}

__global__ __launch_bounds__(kPkWaves * 64) void k_pack_blocks(
    const float* __restrict__ p, const float* __restrict__ a, uint8_t* __restrict__ blob,
    const uint32_t* __restrict__ slot_base, const int32_t* __restrict__ cols, int E, int dout,
    int r, uint32_t n_seg, uint32_t* __restrict__ flags) {
  const int e = (int)blockIdx.y;
  const int lane = (int)threadIdx.x & 63;
  const int wv = (int)threadIdx.x >> 6;
  DirRec* dir = reinterpret_cast<DirRec*>(blob + kHeaderBytes) + e;
  uint16_t cnt[kNumGroups];
#pragma unroll
  for (int g = 0; g < kNumGroups; ++g) cnt[g] = dir->count[g];
  const SlotGeo geo = slot_geo(cnt);
  if (blockIdx.x == 0) {  // every magnitude must be finite, stored or not
    for (int k = (int)threadIdx.x; k < r; k += (int)blockDim.x)
      if (!isfinite(a[(size_t)e * r + k])) atomicOr(flags, kBadA);
  }
  const uint32_t b = blockIdx.x * kPkWaves + (uint32_t)wv;
  if (b >= geo.n_slot / 4u) return;
  int g = 0;
  uint32_t gb0 = 0, word0 = 0;  // the group's first block and its first word in a segment record
  while (g < kNumGroups - 1 && b >= gb0 + geo.nb[g]) {
    gb0 += geo.nb[g];
    word0 += 4u * geo.nb[g] * (uint32_t)kGroupWidth[g];
    ++g;
  }
  const int w = kGroupWidth[g];
  const uint32_t wordb = word0 + (b - gb0) * 4u * (uint32_t)w;
  const uint64_t boff = dir->block_offset;
  uint8_t* blk = blob + boff;
  uint16_t* kidx = reinterpret_cast<uint16_t*>(blk);
  float* A = reinterpret_cast<float*>(blk + dir->a_off);
  uint16_t* S = reinterpret_cast<uint16_t*>(blk + dir->s_off);
  uint16_t* M = reinterpret_cast<uint16_t*>(blk + dir->m_off);
  uint32_t* P = reinterpret_cast<uint32_t*>(blk + dir->planes_off);
  const uint32_t seg_words = dir->seg_words;

  int col[4];
  float av[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    col[u] = cols[slot_base[e] + 4u * b + (uint32_t)u];
    av[u] = col[u] >= 0 ? a[(size_t)e * r + col[u]] : 0.f;
  }
  if (lane < 4) {
    kidx[4u * b + lane] = (uint16_t)(col[lane] >= 0 ? col[lane] : 0);
    A[4u * b + lane] = av[lane];
  }
  const float* pc[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) pc[u] = p + ((size_t)e * r + (col[u] >= 0 ? col[u] : 0)) * dout;

  bool bad = false;
  if (w == 16) {
    // word (octet i, 2 rho + h): fp16 of row 8 i + rho in slots 2h (low) and 2h + 1
    const int rho = lane & 7, h = (lane >> 3) & 1, oc = lane >> 4;
    const int c0 = h ? col[2] : col[0], c1 = h ? col[3] : col[1];
    const float* p0 = h ? pc[2] : pc[0];
    const float* p1 = h ? pc[3] : pc[1];
    for (uint32_t sg = 0; sg < n_seg; ++sg) {
      const uint32_t row = sg * kSegRows + 8u * (uint32_t)oc + (uint32_t)rho;
      uint32_t lo = 0, hi = 0;
      if (row < (uint32_t)dout) {
        if (c0 >= 0) {
          const float v = p0[row];
          bad |= !(fabsf(v) <= kPMax);
          lo = f16_bits(v);
        }
        if (c1 >= 0) {
          const float v = p1[row];
          bad |= !(fabsf(v) <= kPMax);
          hi = f16_bits(v);
        }
      }
      P[(size_t)sg * seg_words + wordb + 16u * (uint32_t)oc + 2u * (uint32_t)rho + (uint32_t)h] =
          lo | (hi << 16);
    }
    if (lane == 0) {
      float bound = 0.f;
      for (int u = 0; u < 4; ++u)
        if (col[u] >= 0) bound = fmaxf(bound, fabsf(av[u]));
      atomicMax(reinterpret_cast<unsigned int*>(&dir->cmax), __float_as_uint(bound));
    }
  } else {
    // lane = 32 half + 8 u + rho holds rows 16 it + 8 half + rho of slot u;
    // both passes walk the rows in batches of kPkB steps with all loads of a
    // batch issued first (the second pass finds the column in the cache)
    const int u = (lane >> 3) & 3, rho = lane & 7, half = lane >> 5;
    const int cu = u == 0 ? col[0] : u == 1 ? col[1] : u == 2 ? col[2] : col[3];
    const float* pu = u == 0 ? pc[0] : u == 1 ? pc[1] : u == 2 ? pc[2] : pc[3];
    const uint32_t nit = 2u * n_seg;  // 16-row steps
    float lo = INFINITY, hi = -INFINITY;
    for (uint32_t it0 = 0; it0 < nit; it0 += kPkB) {
      float v[kPkB];
#pragma unroll
      for (int j = 0; j < kPkB; ++j) {
        const uint32_t row = 16u * (it0 + j) + 8u * (uint32_t)half + (uint32_t)rho;
        v[j] = (cu >= 0 && it0 + j < nit && row < (uint32_t)dout) ? pu[row] : NAN;
      }
#pragma unroll
      for (int j = 0; j < kPkB; ++j) {
        const uint32_t row = 16u * (it0 + j) + 8u * (uint32_t)half + (uint32_t)rho;
        if (cu >= 0 && it0 + j < nit && row < (uint32_t)dout) {
          bad |= !(fabsf(v[j]) <= kPMax);
          lo = min_signed(lo, v[j]);
          hi = fmaxf(hi, v[j]);
        }
      }
    }
    // the 16 lanes of one slot: rho (lane bits 0-2) and half (bit 5)
#pragma unroll
    for (int o = 1; o <= 32; o <<= 1) {
      if (o == 8 || o == 16) continue;
      lo = min_signed(lo, __shfl_xor(lo, o, 64));
      hi = fmaxf(hi, __shfl_xor(hi, o, 64));
    }
    // scale and offset as the host quantizer forms them
    const float L = (float)((1 << w) - 1);
    uint16_t sb = 0, mb = 0;
    float bound = 0.f;
    if (cu >= 0) {
      sb = f16_bits((hi - lo) / L);
      if ((sb & 0x7FFFu) == 0) sb = 0x3C00u;  // scale rounded to zero: use 1
      mb = f16_bits(lo);
      const float au = u == 0 ? av[0] : u == 1 ? av[1] : u == 2 ? av[2] : av[3];
      bound = fabsf(au) * f16_val(sb);
    }
    const float su = f16_val(sb), mu = f16_val(mb);
    if (lane < 32 && rho == 0) {
      S[4u * b + (uint32_t)u] = sb;
      M[4u * b + (uint32_t)u] = mb;
    }
    bound = fmaxf(fmaxf(__shfl(bound, 0, 64), __shfl(bound, 8, 64)),
                  fmaxf(__shfl(bound, 16, 64), __shfl(bound, 24, 64)));
    if (lane == 0) atomicMax(reinterpret_cast<unsigned int*>(&dir->cmax), __float_as_uint(bound));
    // codes; one ballot per plane gives the words of two octets
    const int jw = lane & 31;  // the plane this lane writes (lanes with jw < w)
    for (uint32_t it0 = 0; it0 < nit; it0 += kPkB) {
      float v[kPkB];
#pragma unroll
      for (int j = 0; j < kPkB; ++j) {
        const uint32_t row = 16u * (it0 + j) + 8u * (uint32_t)half + (uint32_t)rho;
        v[j] = (cu >= 0 && it0 + j < nit && row < (uint32_t)dout) ? pu[row] : NAN;
      }
#pragma unroll
      for (int j = 0; j < kPkB; ++j) {
        if (it0 + j >= nit) break;  // uniform
        const uint32_t oct = 2u * (it0 + j) + (uint32_t)half;
        const uint32_t row = 8u * oct + (uint32_t)rho;
        uint32_t q = 0;
        if (cu >= 0 && row < (uint32_t)dout) {
          float c = rintf((v[j] - mu) / su);
          c = c < 0.0f ? 0.0f : (c > L ? L : c);
          q = (uint32_t)c;
        }
        uint32_t word = 0;
        for (int pj = 0; pj < w; ++pj) {
          const uint64_t m = __ballot((q >> pj) & 1u);
          if (jw == pj) word = half ? (uint32_t)(m >> 32) : (uint32_t)m;
        }
        if (jw < w)
          P[(size_t)(oct >> 2) * seg_words + wordb + (oct & 3u) * (uint32_t)w + (uint32_t)jw] =
              word;
      }
    }
  }
  if (bad) atomicOr(flags, kBadP);
}

// Register value of the CRC over each 4 KiB chunk of data[0, n) from a
// start value of 0 (n and the chunk starts are multiples of 16).
// The component table's values (s, m, a, cmax) of expert blockIdx.y, copied
// from its block's slot arrays once k_pack_blocks has written them (the
// slot array of the table is already in place): one thread per slot.
__global__ __launch_bounds__(256) void k_pack_ctab(uint8_t* __restrict__ blob, int E, int r) {
  const int e = (int)blockIdx.y;
  const DirRec* dir = reinterpret_cast<const DirRec*>(blob + kHeaderBytes) + e;
  uint16_t cnt[kNumGroups];
#pragma unroll
  for (int g = 0; g < kNumGroups; ++g) cnt[g] = dir->count[g];
  const SlotGeo geo = slot_geo(cnt);
  uint8_t* ct = blob + ctab_offset((uint64_t)E) + (size_t)e * ctab_stride((uint64_t)r);
  const uint32_t q = blockIdx.x * blockDim.x + threadIdx.x;
  if (q == 0) *reinterpret_cast<float*>(ct + ctab_cmax_off(r)) = dir->cmax;
  if (q >= geo.n_slot) return;
  uint32_t gs = 0;
  int g = 0;
  while (g < kNumGroups - 1 && q >= gs + 4u * geo.nb[g]) {
    gs += 4u * geo.nb[g];
    ++g;
  }
  if (q - gs >= cnt[g]) return;  // a padding slot
  const uint8_t* blk = blob + dir->block_offset;
  const uint32_t k = reinterpret_cast<const uint16_t*>(blk)[q];
  if (k >= (uint32_t)r) return;
  reinterpret_cast<uint32_t*>(ct + ctab_a_off(r))[k] =
      reinterpret_cast<const uint32_t*>(blk + dir->a_off)[q];
  if (g < kNumQGroups) {
    reinterpret_cast<uint16_t*>(ct + ctab_s_off(r))[k] =
        reinterpret_cast<const uint16_t*>(blk + dir->s_off)[q];
    reinterpret_cast<uint16_t*>(ct + ctab_m_off(r))[k] =
        reinterpret_cast<const uint16_t*>(blk + dir->m_off)[q];
  }
}

__global__ __launch_bounds__(256) void k_crc_chunks(const uint8_t* __restrict__ data, uint64_t n,
                                                    uint32_t* __restrict__ out) {
  __shared__ uint32_t T[4][256];
  {
    uint32_t c = threadIdx.x;
    for (int k = 0; k < 8; ++k) c = (c & 1u) ? kCrcPoly ^ (c >> 1) : c >> 1;
    T[0][threadIdx.x] = c;
  }
  __syncthreads();
  for (int t = 1; t < 4; ++t) {  // T[t][i]: byte i followed by t zero bytes
    const uint32_t prev = T[t - 1][threadIdx.x];
    T[t][threadIdx.x] = (prev >> 8) ^ T[0][prev & 0xFFu];
    __syncthreads();
  }
  const uint64_t chunk = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const uint64_t beg = chunk * kCrcChunk;
  if (beg >= n) return;
  const uint64_t end = beg + kCrcChunk < n ? beg + kCrcChunk : n;
  uint32_t c = 0;
  for (uint64_t off = beg; off < end; off += 16) {
    const uint4 v = *reinterpret_cast<const uint4*>(data + off);
    const uint32_t wv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t x = c ^ wv[i];
      c = T[3][x & 0xFFu] ^ T[2][(x >> 8) & 0xFFu] ^ T[1][(x >> 16) & 0xFFu] ^ T[0][x >> 24];
    }
  }
  out[chunk] = c;
}

// a(x) b(x) mod the CRC polynomial, reflected representation (bit 31 holds
// the coefficient of x^0).
uint32_t crc_mulmod(uint32_t a, uint32_t b) {
  uint32_t prod = 0;
  for (int i = 0; i < 32; ++i) {
    if (a & (0x80000000u >> i)) prod ^= b;
    b = (b & 1u) ? (b >> 1) ^ kCrcPoly : b >> 1;  // b *= x
  }
  return prod;
}

// x^(8 n) mod the polynomial: the effect of n zero bytes on the register.
uint32_t crc_x8n(uint64_t n) {
  uint32_t result = 0x80000000u;  // 1
  uint32_t base = 0x00800000u;    // x^8
  while (n) {
    if (n & 1u) result = crc_mulmod(result, base);
    base = crc_mulmod(base, base);
    n >>= 1;
  }
  return result;
}

struct PackWsLayout {
  size_t flags, slot_base, cols, crc, total;
};
PackWsLayout pack_ws_layout(int E, uint64_t n_slots, uint64_t blob_total) {
  PackWsLayout l;
  const uint64_t nchunks = (blob_total - kHeaderBytes + kCrcChunk - 1) / kCrcChunk;
  l.flags = 0;
  l.slot_base = 16;
  l.cols = align_up(l.slot_base + 4ull * (E + 1), 16);
  l.crc = align_up(l.cols + 4ull * n_slots, 16);
  l.total = align_up(l.crc + 4ull * nchunks, 16);
  return l;
}

int hip_status(hipError_t err, const char* what) {
  if (err != hipSuccess) return fail(BITSMOE_EHIP, "%s: %s", what, hipGetErrorString(err));
  return BITSMOE_OK;
}

}  // namespace
}  // namespace bitsmoe

using namespace bitsmoe;

extern "C" {

int bitsmoe_pack_device_workspace_size(int E, int dout, int r, const uint8_t* bits,
                                       size_t* bytes) {
  if (!bytes) return fail(BITSMOE_EINVAL, "bytes is null");
  std::vector<DirRec> dirs;
  uint64_t total = 0;
  const int st = pack_plan(E, dout, r, bits, dirs, total);
  if (st) return st;
  uint64_t n_slots = 0;
  for (const DirRec& d : dirs) n_slots += slot_geo(d.count).n_slot;
  *bytes = (size_t)pack_ws_layout(E, n_slots, total).total;
  return BITSMOE_OK;
}

int bitsmoe_pack_device(int E, int dout, int r, const float* p, const float* a,
                        const uint8_t* bits, void* out, size_t out_bytes, void* ws,
                        size_t ws_bytes, bitsmoe_stream_t stream) {
  if (!p || !a || !out || !ws) return fail(BITSMOE_EINVAL, "null pointer argument");
  if (E > 65535) return fail(BITSMOE_ESHAPE, "E=%d exceeds 65535 (device packer)", E);
  if (((uintptr_t)out & 15u) || ((uintptr_t)ws & 15u) || ((uintptr_t)p & 3u) ||
      ((uintptr_t)a & 3u))
    return fail(BITSMOE_EINVAL, "misaligned pointer (out, ws: 16 bytes; p, a: 4 bytes)");
  std::vector<DirRec> dirs;
  uint64_t total = 0;
  int st = pack_plan(E, dout, r, bits, dirs, total);
  if (st) return st;
  if (out_bytes < total)
    return fail(BITSMOE_ENOSPC, "out_bytes=%zu < %llu", out_bytes, (unsigned long long)total);
  std::vector<uint32_t> slot_base(E + 1);
  std::vector<int32_t> cols;
  uint32_t max_blk = 0;
  for (int e = 0; e < E; ++e) {
    slot_base[e] = (uint32_t)cols.size();
    const std::vector<int> c = pack_slot_columns(bits + (size_t)e * r, r);
    cols.insert(cols.end(), c.begin(), c.end());
    max_blk = std::max<uint32_t>(max_blk, (uint32_t)c.size() / 4u);
  }
  slot_base[E] = (uint32_t)cols.size();
  const PackWsLayout wl = pack_ws_layout(E, cols.size(), total);
  if (ws_bytes < wl.total)
    return fail(BITSMOE_ENOSPC, "ws_bytes=%zu < %zu", ws_bytes, wl.total);
  const hipStream_t s = (hipStream_t)stream;
  uint8_t* blob = (uint8_t*)out;
  uint8_t* w8 = (uint8_t*)ws;
  const uint32_t n_seg = (uint32_t)(align_up(dout, kSegRows) / kSegRows);

  if ((st = bitsmoe_workspace_init(blob, (size_t)total, stream))) return st;
  if ((st = bitsmoe_workspace_init(w8, 16, stream))) return st;
  // every copy below reads host memory that lives until this call returns
  if ((st = hip_status(hipMemcpyAsync(blob + kHeaderBytes, dirs.data(), sizeof(DirRec) * E,
                                      hipMemcpyHostToDevice, s),
                       "directory copy")))
    return st;
  std::vector<uint8_t> ctab((size_t)E * ctab_stride((uint64_t)r));
  pack_ctab_slots(E, r, bits, ctab.data());
  if ((st = hip_status(hipMemcpyAsync(blob + ctab_offset((uint64_t)E), ctab.data(), ctab.size(),
                                      hipMemcpyHostToDevice, s),
                       "component table copy")))
    return st;
  if ((st = hip_status(hipMemcpyAsync(w8 + wl.slot_base, slot_base.data(), 4ull * (E + 1),
                                      hipMemcpyHostToDevice, s),
                       "slot table copy")))
    return st;
  if (!cols.empty() &&
      (st = hip_status(hipMemcpyAsync(w8 + wl.cols, cols.data(), 4ull * cols.size(),
                                      hipMemcpyHostToDevice, s),
                       "slot table copy")))
    return st;
  const unsigned gx = std::max<unsigned>(1u, (max_blk + kPkWaves - 1) / kPkWaves);
  hipLaunchKernelGGL(k_pack_blocks, dim3(gx, (unsigned)E), dim3(kPkWaves * 64), 0, s, p, a, blob,
                     (const uint32_t*)(w8 + wl.slot_base), (const int32_t*)(w8 + wl.cols), E,
                     dout, r, n_seg, (uint32_t*)w8);
  if ((st = hip_status(hipGetLastError(), "pack launch"))) return st;
  hipLaunchKernelGGL(k_pack_ctab, dim3((4u * max_blk + 255u) / 256u, (unsigned)E), dim3(256), 0,
                     s, blob, E, r);
  if ((st = hip_status(hipGetLastError(), "component table launch"))) return st;
  const uint64_t nbody = total - kHeaderBytes;
  const uint64_t nchunks = (nbody + kCrcChunk - 1) / kCrcChunk;
  hipLaunchKernelGGL(k_crc_chunks, dim3((unsigned)((nchunks + 255) / 256)), dim3(256), 0, s,
                     blob + kHeaderBytes, nbody, (uint32_t*)(w8 + wl.crc));
  if ((st = hip_status(hipGetLastError(), "checksum launch"))) return st;
  std::vector<uint32_t> chunk_crc(nchunks);
  uint32_t flags = 0;
  if ((st = hip_status(hipMemcpyAsync(chunk_crc.data(), w8 + wl.crc, 4ull * nchunks,
                                      hipMemcpyDeviceToHost, s),
                       "checksum copy")) ||
      (st = hip_status(hipMemcpyAsync(&flags, w8, 4, hipMemcpyDeviceToHost, s), "flag copy")) ||
      (st = hip_status(hipStreamSynchronize(s), "pack")))
    return st;
  if (flags & kBadA) return fail(BITSMOE_EBITS, "a magnitude is not finite");
  if (flags & kBadP) return fail(BITSMOE_EBITS, "a stored p value is not finite or |p| > 60000");
  // fold: register(start, A B) = register(start, A) x^(8|B|) + register(0, B).
  // Multiplying by the fixed x^(8 * chunk) is linear in the register, so it
  // is four byte-table lookups.
  const uint32_t x_chunk = crc_x8n(kCrcChunk);
  std::vector<uint32_t> mt(4 * 256);
  for (int j = 0; j < 4; ++j)
    for (uint32_t v = 0; v < 256; ++v) mt[256 * j + v] = crc_mulmod(v << (8 * j), x_chunk);
  uint32_t reg = 0xFFFFFFFFu;
  for (uint64_t i = 0; i < nchunks; ++i) {
    const uint64_t len = std::min<uint64_t>(kCrcChunk, nbody - i * kCrcChunk);
    const uint32_t sh = len == kCrcChunk
                            ? mt[reg & 0xFFu] ^ mt[256 + ((reg >> 8) & 0xFFu)] ^
                                  mt[512 + ((reg >> 16) & 0xFFu)] ^ mt[768 + (reg >> 24)]
                            : crc_mulmod(reg, crc_x8n(len));
    reg = sh ^ chunk_crc[i];
  }
  Header h;
  memset(&h, 0, sizeof(h));
  h.magic = kMagic;
  h.version = kVersion;
  h.E = (uint32_t)E;
  h.dout = (uint32_t)dout;
  h.r = (uint32_t)r;
  h.dout_pad = n_seg * kSegRows;
  h.n_seg = n_seg;
  h.header_bytes = kHeaderBytes;
  h.total_bytes = total;
  h.dir_offset = kHeaderBytes;
  h.ctab_offset = ctab_offset((uint64_t)E);
  h.crc32 = reg ^ 0xFFFFFFFFu;
  if ((st = hip_status(hipMemcpyAsync(blob, &h, sizeof(h), hipMemcpyHostToDevice, s),
                       "header copy")) ||
      (st = hip_status(hipStreamSynchronize(s), "pack")))
    return st;
  return BITSMOE_OK;
}

}  // extern "C"
