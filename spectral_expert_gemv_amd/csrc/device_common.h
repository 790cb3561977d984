// Device-side helpers shared by the gfx950 kernels: blob directory access
// with bounds checks, the lane-per-row code decoder, wave reductions.
#pragma once
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "format.h"

namespace bitsmoe {

constexpr int kWave = 64;

// Header fields a directory record is checked against.
struct HdrF {
  uint32_t magic, version, E, dout, r, n_seg;
};

// Scalar loads (constant address space): the header is the same for all lanes.
__device__ inline HdrF load_hdr(const uint8_t* __restrict__ blob) {
  typedef __attribute__((address_space(4))) const Header CHeader;
  CHeader* h = (CHeader*)(blob);
  HdrF f;
  f.magic = h->magic;
  f.version = h->version;
  f.E = h->E;
  f.dout = h->dout;
  f.r = h->r;
  f.n_seg = h->n_seg;
  return f;
}

// Directory record of expert e, loaded from e clamped into [0, E) (always
// inside the directory the host size check guarantees); check_dir decides
// whether it may be used.
__device__ inline DirRec load_rec(const uint8_t* __restrict__ blob, int e, int E) {
  const int ec = e < 0 ? 0 : (e >= E ? E - 1 : e);
  return reinterpret_cast<const DirRec*>(blob + kHeaderBytes)[ec];
}

// Validates a record against the dimensions the host passed and against the
// blob size.  Returns false when the blob cannot be read safely.
__device__ inline bool check_dir(const HdrF& h, const DirRec& d, uint64_t blob_bytes, int e,
                                 int E, int dout, int r) {
  if (h.magic != kMagic || h.version != kVersion || h.E != (uint32_t)E ||
      h.dout != (uint32_t)dout || h.r != (uint32_t)r)
    return false;
  if (e < 0 || e >= E) return false;
  const uint64_t n_seg = h.n_seg;
  if (n_seg != (uint64_t)((dout + kSegRows - 1) / kSegRows)) return false;
  if (d.block_offset + d.block_bytes > blob_bytes) return false;
  const SlotGeo g = slot_geo(d.count);
  uint32_t n_nz = 0;
#pragma unroll
  for (int i = 0; i < kNumGroups; ++i) n_nz += d.count[i];
  if (n_nz != d.n_nz || d.n_16 != d.count[kNumGroups - 1] || d.n_q + d.n_16 != n_nz ||
      g.seg_words != d.seg_words || n_nz > (uint32_t)r)
    return false;
  if (2ull * g.n_slot > d.a_off || (uint64_t)d.a_off + 4ull * g.n_slot > d.s_off ||
      (uint64_t)d.s_off + 2ull * g.n_qslot > d.m_off ||
      (uint64_t)d.m_off + 2ull * g.n_qslot > d.planes_off ||
      (uint64_t)d.planes_off + 4ull * n_seg * g.seg_words + 16 > d.block_bytes ||
      (d.a_off & 15u) || (d.s_off & 15u) || (d.m_off & 15u) || (d.planes_off & 15u) ||
      (d.block_offset & 15u))
    return false;
  return true;
}

// Directory record of expert e of a device blob, loaded and validated.
__device__ inline bool load_dir(const uint8_t* __restrict__ blob, uint64_t blob_bytes,
                                int e, int E, int dout, int r, DirRec& d) {
  d = load_rec(blob, e, E);
  return check_dir(load_hdr(blob), d, blob_bytes, e, E, dout, r);
}

// Code of segment row `row` (0..31) in slot u (0..3) of a block of width
// w <= 8 whose record starts at `rec`: bit j from word (row / 8, j), bit
// 8 u + row % 8.  Used by the lane-per-row kernels and the code dump.
__device__ inline uint32_t decode_code(const uint32_t* __restrict__ rec, int w, int row, int u) {
  const uint32_t* oct = rec + (row >> 3) * w;
  const int sh = 8 * u + (row & 7);
  uint32_t q = 0;
  for (int j = 0; j < w; ++j) q |= ((oct[j] >> sh) & 1u) << j;
  return q;
}

// fp16 bit pattern of segment row `row` in slot u of a 16-bit block.
__device__ inline uint32_t decode_f16(const uint32_t* __restrict__ rec, int row, int u) {
  const uint32_t wv = rec[(row >> 3) * 16 + 2 * (row & 7) + (u >> 1)];
  return (u & 1) ? (wv >> 16) : (wv & 0xFFFFu);
}

// Wave-wide sum and max through DPP row operations (no LDS round trips):
// two quad permutes, the half-row and row mirrors leave every row's total in
// all its lanes, then row broadcasts 15 (into rows 1, 3) and 31 (into rows
// 2, 3) leave the wave total in lane 63, read back as a uniform value.
template <int kCtrl, int kRowMask = 0xF>
__device__ __forceinline__ float dpp_move(float v, float fill) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, fill),
                                                                __builtin_bit_cast(int, v), kCtrl,
                                                                kRowMask, 0xF, false));
}
__device__ inline float wave_sum_dpp(float v) {
  v += dpp_move<0xB1>(v, 0.f);        // quad_perm [1,0,3,2]
  v += dpp_move<0x4E>(v, 0.f);        // quad_perm [2,3,0,1]
  v += dpp_move<0x141>(v, 0.f);       // row_half_mirror
  v += dpp_move<0x140>(v, 0.f);       // row_mirror
  v += dpp_move<0x142, 0xA>(v, 0.f);  // row_bcast:15
  v += dpp_move<0x143, 0xC>(v, 0.f);  // row_bcast:31
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}
// (v >= 0 in every lane)
__device__ inline float wave_max_dpp(float v) {
  v = fmaxf(v, dpp_move<0xB1>(v, 0.f));
  v = fmaxf(v, dpp_move<0x4E>(v, 0.f));
  v = fmaxf(v, dpp_move<0x141>(v, 0.f));
  v = fmaxf(v, dpp_move<0x140>(v, 0.f));
  v = fmaxf(v, dpp_move<0x142, 0xA>(v, 0.f));
  v = fmaxf(v, dpp_move<0x143, 0xC>(v, 0.f));
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}

// Wave-wide sum of unsigned words (modulo 2^32), same DPP pattern.
template <int kCtrl, int kRowMask = 0xF>
__device__ __forceinline__ uint32_t dpp_move_u(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kCtrl, kRowMask, 0xF, false);
}
__device__ inline uint32_t wave_sum_u32_dpp(uint32_t v) {
  v += dpp_move_u<0xB1>(v);
  v += dpp_move_u<0x4E>(v);
  v += dpp_move_u<0x141>(v);
  v += dpp_move_u<0x140>(v);
  v += dpp_move_u<0x142, 0xA>(v);
  v += dpp_move_u<0x143, 0xC>(v);
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

__device__ inline float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

__device__ inline float silu_mul(float g, float u) { return g / (1.0f + expf(-g)) * u; }

}  // namespace bitsmoe
