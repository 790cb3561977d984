// Host packer and blob checker (format v3, documented in include/bitsmoe.h).
//
// Quantizes each unit direction p_{e,k} at its own width and stores the
// columns grouped by width, each 1..8-bit group as bit planes ("second
// split", "Usage" and "execution" of the BitsMoE blog note's Methodology).
// A plane word covers 8 rows x 4 adjacent slots: byte u holds the 8 rows'
// bits of slot u, so a lane that owns a row rotates its bits into the low
// bit of every byte and gets 4 codes per plane with two operations; the
// lane reads a contiguous run of words per block.  The quantizer runs in IEEE float32 with no contraction so that its
// codes are reproducible bit for bit.
#include <math.h>
#include <string.h>

#include <algorithm>
#include <thread>
#include <vector>

#include "bitsmoe.h"
#include "common.h"
#include "format.h"
#include "pack_plan.h"

#pragma clang fp contract(off)

namespace bitsmoe {
namespace {

// float32 -> binary16, round to nearest, ties to even (IEEE 754 conversion).
uint16_t f32_to_f16(float f) {
  uint32_t x;
  memcpy(&x, &f, 4);
  const uint32_t sign = (x >> 16) & 0x8000u;
  const uint32_t ax = x & 0x7FFFFFFFu;
  if (ax >= 0x7F800000u) return sign | 0x7C00u | (ax > 0x7F800000u ? 0x200u : 0u);
  if (ax >= 0x477FF000u) return sign | 0x7C00u;          // >= 65520 rounds to inf
  if (ax < 0x38800000u) {                                 // below 2^-14: subnormal
    if (ax < 0x33000000u) return sign;                    // below 2^-25: zero
    const uint32_t e = ax >> 23;
    const uint32_t mant = (ax & 0x7FFFFFu) | 0x800000u;
    const uint32_t shift = 126u - e;                      // 14..24
    uint32_t h = mant >> shift;
    const uint32_t rem = mant & ((1u << shift) - 1u);
    const uint32_t half = 1u << (shift - 1u);
    if (rem > half || (rem == half && (h & 1u))) ++h;
    return sign | h;
  }
  uint32_t h = (ax >> 13) - 0x1C000u;                     // rebias exponent 127 -> 15
  const uint32_t rem = ax & 0x1FFFu;
  if (rem > 0x1000u || (rem == 0x1000u && (h & 1u))) ++h;
  return sign | h;
}

float f16_to_f32(uint16_t h) {
  const uint32_t sign = (uint32_t)(h & 0x8000u) << 16;
  const uint32_t e = (h >> 10) & 0x1Fu;
  const uint32_t m = h & 0x3FFu;
  uint32_t x;
  if (e == 0) {
    if (m == 0) {
      x = sign;
    } else {  // subnormal: m * 2^-24, exact in float32
      float v = (float)m * 5.9604644775390625e-8f;
      memcpy(&x, &v, 4);
      x |= sign;
    }
  } else if (e == 31) {
    x = sign | 0x7F800000u | (m << 13);
  } else {
    x = sign | ((e + 112u) << 23) | (m << 13);
  }
  float f;
  memcpy(&f, &x, 4);
  return f;
}

struct CrcTable {
  uint32_t t[256];
  CrcTable() {
    for (uint32_t i = 0; i < 256; ++i) {
      uint32_t c = i;
      for (int k = 0; k < 8; ++k) c = (c & 1u) ? 0xEDB88320u ^ (c >> 1) : c >> 1;
      t[i] = c;
    }
  }
};

// CRC-32 with the reflected IEEE polynomial (the zlib/PNG checksum).
uint32_t crc32_ieee(const uint8_t* p, size_t n) {
  static const CrcTable tab;  // thread-safe static initialisation
  const uint32_t* table = tab.t;
  uint32_t c = 0xFFFFFFFFu;
  for (size_t i = 0; i < n; ++i) c = table[(c ^ p[i]) & 0xFFu] ^ (c >> 8);
  return c ^ 0xFFFFFFFFu;
}

// width -> group index; 0-bit columns map to kNumGroups, invalid widths to
// kNumGroups + 1 (one table lookup per column instead of a search)
struct GroupLut {
  uint8_t g[256];
  GroupLut() {
    for (int b = 0; b < 256; ++b) g[b] = kNumGroups + 1;
    g[0] = kNumGroups;
    for (int i = 0; i < kNumGroups; ++i) g[kGroupWidth[i]] = (uint8_t)i;
  }
};
const GroupLut& group_lut() {
  static const GroupLut lut;  // thread-safe static initialisation
  return lut;
}

// Canonical block layout of one expert from its per-width column counts
// (cmax and block_offset are filled in by the caller).
DirRec block_layout(const uint16_t count[kNumGroups], uint32_t n_seg) {
  DirRec d;
  memset(&d, 0, sizeof(d));
  const SlotGeo g = slot_geo(count);
  uint32_t n_nz = 0;
  for (int i = 0; i < kNumGroups; ++i) {
    d.count[i] = count[i];
    n_nz += count[i];
  }
  d.n_nz = n_nz;
  d.n_16 = count[kNumGroups - 1];
  d.n_q = n_nz - d.n_16;
  d.seg_words = g.seg_words;
  d.a_off = (uint32_t)align_up(2ull * g.n_slot, 16);
  d.s_off = (uint32_t)align_up(d.a_off + 4ull * g.n_slot, 16);
  d.m_off = (uint32_t)align_up(d.s_off + 2ull * g.n_qslot, 16);
  d.planes_off = (uint32_t)align_up(d.m_off + 2ull * g.n_qslot, 256);
  // at least 16 zero bytes follow the planes, so 16-byte reads of the last
  // words stay inside the block
  d.block_bytes = (uint32_t)align_up(d.planes_off + 4ull * n_seg * g.seg_words + 16, 256);
  return d;
}

int check_dims(int E, int dout, int r) {
  if (E <= 0 || dout <= 0 || r <= 0)
    return fail(BITSMOE_ESHAPE, "E=%d dout=%d r=%d must be positive", E, dout, r);
  if (r > 65535) return fail(BITSMOE_ESHAPE, "r=%d exceeds 65535", r);
  if (dout > (1 << 24)) return fail(BITSMOE_ESHAPE, "dout=%d too large", dout);
  return BITSMOE_OK;
}

}  // namespace

// Per-expert directory records and the total size; validates widths.
int pack_plan(int E, int dout, int r, const uint8_t* bits, std::vector<DirRec>& dirs,
         uint64_t& total) {
  int st = check_dims(E, dout, r);
  if (st) return st;
  if (!bits) return fail(BITSMOE_EINVAL, "bits is null");
  const uint32_t n_seg = (uint32_t)(align_up(dout, kSegRows) / kSegRows);
  dirs.resize(E);
  uint64_t pos = first_block_offset((uint64_t)E, (uint64_t)r);
  const uint8_t* lut = group_lut().g;
  for (int e = 0; e < E; ++e) {
    uint32_t c[kNumGroups + 2] = {0, 0, 0, 0, 0, 0, 0, 0, 0};
    const uint8_t* be = bits + (size_t)e * r;
    for (int k = 0; k < r; ++k) ++c[lut[be[k]]];
    if (c[kNumGroups + 1]) {
      for (int k = 0; k < r; ++k)
        if (lut[be[k]] == kNumGroups + 1)
          return fail(BITSMOE_EBITS, "bits[%d,%d]=%d not in {0,1,2,3,4,6,8,16}", e, k, be[k]);
    }
    uint16_t count[kNumGroups];
    for (int g = 0; g < kNumGroups; ++g) count[g] = (uint16_t)c[g];
    const SlotGeo g = slot_geo(count);
    if (align_up(2ull * g.n_slot + 8ull * g.n_slot, 256) + 4ull * n_seg * g.seg_words + 512 >
        0xFFFFFFFFull)
      return fail(BITSMOE_ESHAPE, "expert %d block exceeds 4 GiB", e);
    dirs[e] = block_layout(count, n_seg);
    dirs[e].block_offset = pos;
    pos += dirs[e].block_bytes;
  }
  total = pos;
  return BITSMOE_OK;
}

namespace {

void quantize_col(const float* p, int dout, int b, uint8_t* q, uint16_t* s_bits,
                  uint16_t* m_bits) {
  float lo = p[0], hi = p[0];
  for (int i = 1; i < dout; ++i) {
    // -0 counts as below +0 (IEEE minimum), so the sign of a zero minimum
    // does not depend on the order of the rows
    if (p[i] < lo || (p[i] == lo && signbit(p[i]))) lo = p[i];
    hi = std::max(hi, p[i]);
  }
  const float L = (float)((1 << b) - 1);
  const float s32 = (hi - lo) / L;
  uint16_t sb = f32_to_f16(s32);
  if ((sb & 0x7FFFu) == 0) sb = 0x3C00u;  // scale rounded to zero: use 1
  const uint16_t mb = f32_to_f16(lo);
  const float s = f16_to_f32(sb), m = f16_to_f32(mb);
  for (int i = 0; i < dout; ++i) {
    float v = nearbyintf((p[i] - m) / s);
    v = v < 0.0f ? 0.0f : (v > L ? L : v);
    q[i] = (uint8_t)v;
  }
  *s_bits = sb;
  *m_bits = mb;
}

}  // namespace

// Slot -> column list of one expert: groups of width 1,2,3,4,6,8,16, columns
// in ascending k, each group padded with -1 to a multiple of 32.
std::vector<int> pack_slot_columns(const uint8_t* bits_e, int r) {
  const uint8_t* lut = group_lut().g;
  uint32_t count[kNumGroups + 2] = {0, 0, 0, 0, 0, 0, 0, 0, 0};
  for (int k = 0; k < r; ++k) ++count[lut[bits_e[k]]];
  uint32_t pos[kNumGroups + 2], n = 0;
  for (int g = 0; g < kNumGroups; ++g) {
    pos[g] = n;
    n += (count[g] + kGroupSlots - 1) / kGroupSlots * kGroupSlots;
  }
  std::vector<int> cols(n, -1);
  for (int k = 0; k < r; ++k) {
    const uint32_t g = lut[bits_e[k]];
    if (g < (uint32_t)kNumGroups) cols[pos[g]++] = k;
  }
  return cols;
}

void pack_ctab_slots(int E, int r, const uint8_t* bits, uint8_t* dst) {
  const uint64_t stride = ctab_stride((uint64_t)r);
  memset(dst, 0, (size_t)(E * stride));
  for (int e = 0; e < E; ++e) {
    uint16_t* slot = (uint16_t*)(dst + (size_t)e * stride);
    for (int k = 0; k < r; ++k) slot[k] = kNoSlot;
    const std::vector<int> cols = pack_slot_columns(bits + (size_t)e * r, r);
    for (size_t sl = 0; sl < cols.size(); ++sl)
      if (cols[sl] >= 0) slot[cols[sl]] = (uint16_t)sl;
  }
}

namespace {

// s, m, a and cmax of one expert's component table, read back from its
// block's slot arrays (the slot array is already in place).
void fill_ctab_values(const DirRec& d, const uint8_t* blk, int r, uint8_t* ct) {
  const SlotGeo geo = slot_geo(d.count);
  const uint16_t* kidx = (const uint16_t*)blk;
  const uint32_t* A = (const uint32_t*)(blk + d.a_off);
  const uint16_t* S = (const uint16_t*)(blk + d.s_off);
  const uint16_t* M = (const uint16_t*)(blk + d.m_off);
  uint16_t* cs = (uint16_t*)(ct + ctab_s_off(r));
  uint16_t* cm = (uint16_t*)(ct + ctab_m_off(r));
  uint32_t* ca = (uint32_t*)(ct + ctab_a_off(r));
  uint32_t sl = 0;
  for (int g = 0; g < kNumGroups; ++g) {
    for (uint32_t u = 0; u < d.count[g]; ++u) {
      const uint32_t q = sl + u, k = kidx[q];
      ca[k] = A[q];
      if (g < kNumQGroups) {
        cs[k] = S[q];
        cm[k] = M[q];
      }
    }
    sl += 4u * geo.nb[g];
  }
  memcpy(ct + ctab_cmax_off(r), &d.cmax, 4);
}

void fill_block(DirRec& d, int e, int dout, int r, uint32_t n_seg, const float* p,
                const float* a, const uint8_t* bits, uint8_t* blk) {
  const SlotGeo geo = slot_geo(d.count);
  const std::vector<int> cols = pack_slot_columns(bits + (size_t)e * r, r);
  uint16_t* kidx = (uint16_t*)blk;
  float* A = (float*)(blk + d.a_off);
  uint16_t* S = (uint16_t*)(blk + d.s_off);
  uint16_t* M = (uint16_t*)(blk + d.m_off);
  uint32_t* P = (uint32_t*)(blk + d.planes_off);
  const uint32_t dout_pad = n_seg * kSegRows;
  // codes (1..8 bits) or fp16 bit patterns (16 bits) of the 4 slots of a block
  std::vector<uint16_t> q4(4 * (size_t)dout_pad);
  std::vector<uint8_t> q(dout_pad);
  float cmax = 0.0f;
  uint32_t slot = 0, word = 0;  // word: offset of the block inside a segment record
  for (int g = 0; g < kNumGroups; ++g) {
    const int w = kGroupWidth[g];
    for (uint32_t blkno = 0; blkno < geo.nb[g]; ++blkno, slot += 4, word += 4u * w) {
      std::fill(q4.begin(), q4.end(), 0);
      for (int u = 0; u < 4; ++u) {
        const int k = cols[slot + u];
        if (k < 0) continue;  // padding slot: everything stays 0
        const float* pc = p + ((size_t)e * r + k) * dout;
        const float ak = a[(size_t)e * r + k];
        kidx[slot + u] = (uint16_t)k;
        A[slot + u] = ak;
        uint16_t* qs = &q4[(size_t)u * dout_pad];
        if (w == 16) {
          for (int i = 0; i < dout; ++i) qs[i] = f32_to_f16(pc[i]);
          cmax = std::max(cmax, fabsf(ak));
        } else {
          quantize_col(pc, dout, w, q.data(), &S[slot + u], &M[slot + u]);
          for (int i = 0; i < dout; ++i) qs[i] = q[i];
          const float bound = fabsf(ak) * f16_to_f32(S[slot + u]);
          cmax = std::max(cmax, bound);
        }
      }
      for (uint32_t sg = 0; sg < n_seg; ++sg) {
        uint32_t* rec = P + (size_t)sg * d.seg_words + word;
        for (int oct = 0; oct < 4; ++oct) {
          const uint32_t row0 = sg * kSegRows + 8u * oct;
          if (w == 16) {
            for (int rho = 0; rho < 8; ++rho)
              for (int h = 0; h < 2; ++h)
                rec[oct * 16 + 2 * rho + h] =
                    (uint32_t)q4[(size_t)(2 * h) * dout_pad + row0 + rho] |
                    ((uint32_t)q4[(size_t)(2 * h + 1) * dout_pad + row0 + rho] << 16);
            continue;
          }
          for (int j = 0; j < w; ++j) {
            uint32_t v = 0;
            for (int rho = 0; rho < 8; ++rho)
              for (int u = 0; u < 4; ++u)
                v |= (uint32_t)((q4[(size_t)u * dout_pad + row0 + rho] >> j) & 1u)
                     << (8 * u + rho);
            rec[oct * w + j] = v;
          }
        }
      }
    }
  }
  d.cmax = cmax;
}

}  // namespace
}  // namespace bitsmoe

using namespace bitsmoe;

extern "C" {

int bitsmoe_pack_size(int E, int dout, int r, const uint8_t* bits, size_t* out_bytes) {
  if (!out_bytes) return fail(BITSMOE_EINVAL, "out_bytes is null");
  std::vector<DirRec> dirs;
  uint64_t total = 0;
  const int st = pack_plan(E, dout, r, bits, dirs, total);
  if (st) return st;
  *out_bytes = (size_t)total;
  return BITSMOE_OK;
}

int bitsmoe_pack(int E, int dout, int r, const float* p, const float* a,
                 const uint8_t* bits, void* out, size_t out_bytes) {
  if (!p || !a || !out) return fail(BITSMOE_EINVAL, "null pointer argument");
  std::vector<DirRec> dirs;
  uint64_t total = 0;
  int st = pack_plan(E, dout, r, bits, dirs, total);
  if (st) return st;
  if (out_bytes < total)
    return fail(BITSMOE_ENOSPC, "out_bytes=%zu < %llu", out_bytes, (unsigned long long)total);
  const size_t n = (size_t)E * r;
  for (size_t i = 0; i < n; ++i) {
    if (!isfinite(a[i])) return fail(BITSMOE_EBITS, "a[%zu] is not finite", i);
    if (bits[i] == 0) continue;
    const float* pc = p + i * dout;
    for (int j = 0; j < dout; ++j)
      if (!isfinite(pc[j]) || fabsf(pc[j]) > 60000.0f)
        return fail(BITSMOE_EBITS, "p[%zu,%d] is not finite or |p| > 60000", i, j);
  }
  uint8_t* blob = (uint8_t*)out;
  memset(blob, 0, total);
  pack_ctab_slots(E, r, bits, blob + ctab_offset((uint64_t)E));
  const uint32_t n_seg = (uint32_t)(align_up(dout, kSegRows) / kSegRows);
  unsigned nt = std::max(1u, std::min(16u, std::thread::hardware_concurrency()));
  nt = std::min<unsigned>(nt, (unsigned)E);
  std::vector<std::thread> pool;
  for (unsigned w = 0; w < nt; ++w) {
    pool.emplace_back([&, w]() {
      for (int e = (int)w; e < E; e += (int)nt) {
        fill_block(dirs[e], e, dout, r, n_seg, p, a, bits, blob + dirs[e].block_offset);
        fill_ctab_values(dirs[e], blob + dirs[e].block_offset, r,
                         blob + ctab_offset((uint64_t)E) + (size_t)e * ctab_stride((uint64_t)r));
      }
    });
  }
  for (auto& t : pool) t.join();
  memcpy(blob + kHeaderBytes, dirs.data(), sizeof(DirRec) * dirs.size());
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
  h.crc32 = crc32_ieee(blob + kHeaderBytes, total - kHeaderBytes);
  memcpy(blob, &h, sizeof(h));
  return BITSMOE_OK;
}

int bitsmoe_blob_check(const void* blob_v, size_t bytes, int* E_out, int* dout_out,
                       int* r_out) {
  if (!blob_v) return fail(BITSMOE_EINVAL, "blob is null");
  if (bytes < kHeaderBytes) return fail(BITSMOE_EFORMAT, "blob shorter than its header");
  const uint8_t* blob = (const uint8_t*)blob_v;
  Header h;
  memcpy(&h, blob, sizeof(h));
  if (h.magic != kMagic) return fail(BITSMOE_EFORMAT, "bad magic");
  if (h.version != kVersion) return fail(BITSMOE_EFORMAT, "unsupported version %u", h.version);
  if (h.header_bytes != kHeaderBytes || h.dir_offset != kHeaderBytes ||
      h.ctab_offset != ctab_offset(h.E))
    return fail(BITSMOE_EFORMAT, "bad header size, directory or component table offset");
  if (check_dims((int)h.E, (int)h.dout, (int)h.r) || h.E > (1u << 20))
    return fail(BITSMOE_EFORMAT, "bad dimensions in header");
  if (h.dout_pad != align_up(h.dout, kSegRows) || h.n_seg != h.dout_pad / kSegRows)
    return fail(BITSMOE_EFORMAT, "bad dout_pad / n_seg");
  if (h.total_bytes > bytes || h.total_bytes < first_block_offset(h.E, h.r))
    return fail(BITSMOE_EFORMAT, "total_bytes %llu inconsistent with buffer %zu",
                (unsigned long long)h.total_bytes, bytes);
  if (crc32_ieee(blob + kHeaderBytes, h.total_bytes - kHeaderBytes) != h.crc32)
    return fail(BITSMOE_EFORMAT, "CRC mismatch");
  uint64_t pos = first_block_offset(h.E, h.r);
  const uint64_t cstride = ctab_stride(h.r);
  for (uint32_t e = 0; e < h.E; ++e) {
    DirRec d;
    memcpy(&d, blob + kHeaderBytes + (size_t)kDirRecBytes * e, sizeof(d));
    DirRec c = block_layout(d.count, h.n_seg);
    c.block_offset = pos;
    c.cmax = d.cmax;
    if (!(d.cmax >= 0.0f) || !isfinite(d.cmax))
      return fail(BITSMOE_EFORMAT, "directory record %u: bad coefficient bound", e);
    if (memcmp(&c, &d, sizeof(d)) != 0 || c.n_nz > h.r)
      return fail(BITSMOE_EFORMAT, "directory record %u inconsistent", e);
    pos += d.block_bytes;
    if (pos > h.total_bytes) return fail(BITSMOE_EFORMAT, "block %u beyond total_bytes", e);
    const uint16_t* kidx = (const uint16_t*)(blob + d.block_offset);
    const SlotGeo geo = slot_geo(d.count);
    for (uint32_t c2 = 0; c2 < geo.n_slot; ++c2)
      if (kidx[c2] >= h.r) return fail(BITSMOE_EFORMAT, "expert %u column index out of range", e);
    // the component table is the stored columns' values in component
    // order: every stored slot maps back, nothing else is indexed, and the
    // other bytes are zero
    std::vector<uint8_t> want((size_t)cstride, 0);
    {
      uint16_t* ws = (uint16_t*)want.data();
      for (uint32_t k = 0; k < h.r; ++k) ws[k] = kNoSlot;
      uint32_t sl = 0;
      for (int g = 0; g < kNumGroups; ++g) {
        for (uint32_t u = 0; u < d.count[g]; ++u) ws[kidx[sl + u]] = (uint16_t)(sl + u);
        sl += 4u * geo.nb[g];
      }
      fill_ctab_values(d, blob + d.block_offset, (int)h.r, want.data());
    }
    if (memcmp(want.data(), blob + h.ctab_offset + cstride * e, (size_t)cstride) != 0)
      return fail(BITSMOE_EFORMAT, "expert %u component table does not match its block", e);
  }
  if (pos != h.total_bytes) return fail(BITSMOE_EFORMAT, "total_bytes does not match blocks");
  if (E_out) *E_out = (int)h.E;
  if (dout_out) *dout_out = (int)h.dout;
  if (r_out) *r_out = (int)h.r;
  return BITSMOE_OK;
}

}  // extern "C"
