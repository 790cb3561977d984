// Packed blob format v4: constants and the directory record shared by the
// host packer, the host checker and the device kernels.  The layout is
// documented in include/bitsmoe.h.
#pragma once
#include <stdint.h>

#if defined(__HIPCC__) || defined(__HIP__)
#define BM_HD __host__ __device__
#else
#define BM_HD
#endif

namespace bitsmoe {

constexpr uint32_t kMagic = 0x454F4D42u;  // bytes 'B','M','O','E'
constexpr uint32_t kVersion = 4;
constexpr int kSegRows = 32;                        // rows of one segment record
constexpr uint32_t kHeaderBytes = 128;
constexpr uint32_t kDirRecBytes = 64;
constexpr int kNumGroups = 7;                       // widths 1,2,3,4,6,8,16
constexpr int kNumQGroups = 6;                      // widths 1..8
constexpr int kGroupWidth[kNumGroups] = {1, 2, 3, 4, 6, 8, 16};

struct Header {
  uint32_t magic, version, E, dout, r, dout_pad, n_seg, header_bytes;
  uint64_t total_bytes, dir_offset;
  uint32_t crc32, reserved0;
  uint64_t ctab_offset;  // the component table (see ctab_offset())
  uint32_t pad[16];
};
static_assert(sizeof(Header) == 128, "header is 128 bytes");

struct DirRec {
  uint64_t block_offset;
  uint32_t n_nz, n_q, n_16, seg_words;
  uint32_t a_off, s_off, m_off, planes_off;
  float cmax;  // max |a_k| s_k (1..8 bits) or |a_k| (16 bits) over stored columns
  uint32_t block_bytes;
  uint16_t count[kNumGroups];
  uint16_t reserved;
};
static_assert(sizeof(DirRec) == 64, "directory record is 64 bytes");

BM_HD constexpr inline uint64_t align_up(uint64_t x, uint64_t a) {
  return (x + a - 1) / a * a;
}

// Component table: after the directory, for every expert the values of its
// components in component (k) order, so that whoever holds z_k can form
// the coefficient of every routed expert without a directory lookup:
//   u16 slot[r]  slot of component k in the expert's slot order, kNoSlot
//                for a 0-bit component
//   f16 s[r], f16 m[r]  scale and offset of a 1..8-bit component (0 for 16-
//                and 0-bit components: s == 0 marks a 16-bit one)
//   f32 a[r]     magnitude (0 for a 0-bit component)
//   f32 cmax     the directory's coefficient bound, then 12 zero bytes
// each array padded to 16 bytes; the expert blocks follow.  Its place
// depends only on E and r.
constexpr uint16_t kNoSlot = 0xFFFFu;
BM_HD constexpr inline uint64_t ctab_offset(uint64_t E) {
  return align_up(kHeaderBytes + (uint64_t)kDirRecBytes * E, 256);
}
BM_HD constexpr inline uint64_t ctab_s_off(uint64_t r) { return align_up(2 * r, 16); }
BM_HD constexpr inline uint64_t ctab_m_off(uint64_t r) { return 2 * align_up(2 * r, 16); }
BM_HD constexpr inline uint64_t ctab_a_off(uint64_t r) { return 3 * align_up(2 * r, 16); }
BM_HD constexpr inline uint64_t ctab_cmax_off(uint64_t r) {
  return 3 * align_up(2 * r, 16) + align_up(4 * r, 16);
}
BM_HD constexpr inline uint64_t ctab_stride(uint64_t r) { return ctab_cmax_off(r) + 16; }
BM_HD constexpr inline uint64_t first_block_offset(uint64_t E, uint64_t r) {
  return align_up(ctab_offset(E) + E * ctab_stride(r), 256);
}

constexpr uint32_t kGroupSlots = 32;  // width groups are padded to a multiple of this

// Slot geometry of one expert, derived from its per-width column counts:
// each width group is padded to a multiple of 32 slots (8 blocks of 4), so
// that a 32-slot step never mixes two widths.
struct SlotGeo {
  uint32_t nb[kNumGroups];  // blocks per group
  uint32_t n_slot, n_qslot, seg_words;
};
BM_HD inline SlotGeo slot_geo(const uint16_t count[kNumGroups]) {
  SlotGeo g;
  g.n_slot = g.n_qslot = g.seg_words = 0;
  for (int i = 0; i < kNumGroups; ++i) {
    g.nb[i] = ((uint32_t)count[i] + kGroupSlots - 1u) / kGroupSlots * (kGroupSlots / 4u);
    g.n_slot += 4u * g.nb[i];
    if (i < kNumQGroups) g.n_qslot += 4u * g.nb[i];
    g.seg_words += 4u * g.nb[i] * (uint32_t)kGroupWidth[i];
  }
  return g;
}

}  // namespace bitsmoe
