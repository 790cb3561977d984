// Device-side helpers shared by the gfx950 kernels: blob directory access
// with bounds checks, the bit-plane code decoder, wave reductions.
#pragma once
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "format.h"

namespace bitsmoe {

constexpr int kWave = 64;

// Header fields a directory record is checked against.
struct HdrF {
  uint32_t magic, version, E, dout, r, n_slabs;
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
  f.n_slabs = h->n_slabs;
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
  const uint64_t n_slabs = h.n_slabs;
  const uint64_t dout_pad = n_slabs * 64;
  if (n_slabs != (uint64_t)((dout + 63) / 64)) return false;
  if (d.block_offset + d.block_bytes > blob_bytes) return false;
  uint32_t n_nz = 0, mps = 0;
#pragma unroll
  for (int g = 0; g < kNumGroups; ++g) {
    n_nz += d.count[g];
    if (g < kNumQGroups) mps += (uint32_t)d.count[g] * kGroupWidth[g];
  }
  if (n_nz != d.n_nz || d.n_16 != d.count[kNumGroups - 1] || d.n_q + d.n_16 != n_nz ||
      mps != d.masks_per_slab || n_nz > (uint32_t)r)
    return false;
  if ((uint64_t)d.a_off + 4ull * n_nz > d.block_bytes || 2ull * n_nz > d.a_off ||
      (uint64_t)d.s_off + 2ull * d.n_q > d.block_bytes ||
      (uint64_t)d.m_off + 2ull * d.n_q > d.block_bytes ||
      (uint64_t)d.planes_off + 8ull * n_slabs * mps + 16 > d.f16_off ||
      (uint64_t)d.f16_off + 2ull * d.n_16 * dout_pad > d.block_bytes ||
      (d.a_off & 3u) || (d.s_off & 1u) || (d.m_off & 1u) || (d.planes_off & 7u) ||
      (d.f16_off & 15u))
    return false;
  return true;
}

// Directory record of expert e of a device blob, loaded and validated.
__device__ inline bool load_dir(const uint8_t* __restrict__ blob, uint64_t blob_bytes,
                                int e, int E, int dout, int r, DirRec& d) {
  d = load_rec(blob, e, E);
  return check_dir(load_hdr(blob), d, blob_bytes, e, E, dout, r);
}

// Code of row `lane` of one 1..8-bit column in a 64-row slab: bit j comes
// from plane j's 64-bit mask (bit `lane`).  Every kernel decodes codes with
// this routine, including the code dump used by the bit-exact tests.
__device__ inline uint32_t decode_code(const uint64_t* __restrict__ masks, int b, int lane) {
  uint32_t q = 0;
  for (int j = 0; j < b; ++j) q |= (uint32_t)((masks[j] >> lane) & 1ull) << j;
  return q;
}

__device__ inline float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

__device__ inline float silu_mul(float g, float u) { return g / (1.0f + expf(-g)) * u; }

}  // namespace bitsmoe
