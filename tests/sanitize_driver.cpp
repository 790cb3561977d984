// Host-side driver of the library's host C++ (packer, blob check, status
// strings), built by tests/test_host_sanitized.py with AddressSanitizer and
// UndefinedBehaviorSanitizer.  It packs the layer read from a file, writes
// the blob back (the test compares it with the oracle packer's bytes), and
// exercises the checks on corrupted blobs and bad arguments.  Exit status 0
// when every expectation holds; each miss is printed.
//
//   sanitize_driver E dout r in.bin out.bin
//   in.bin: p (E*r*dout float32), a (E*r float32), bits (E*r uint8)
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <vector>

#include "bitsmoe.h"

static int g_miss = 0;
#define EXPECT(cond, what)                                              \
  do {                                                                  \
    if (!(cond)) {                                                      \
      fprintf(stderr, "MISS %s (line %d): %s\n", what, __LINE__, #cond); \
      ++g_miss;                                                         \
    }                                                                   \
  } while (0)

// CRC-32 (IEEE 802.3, reflected, polynomial 0xEDB88320), bit by bit: used to
// re-seal a blob after a planted directory change, so the check reaches the
// directory validation.
static uint32_t crc32_bitwise(const uint8_t* p, size_t n) {
  uint32_t c = 0xFFFFFFFFu;
  for (size_t i = 0; i < n; ++i) {
    c ^= p[i];
    for (int k = 0; k < 8; ++k) c = (c >> 1) ^ (0xEDB88320u & (0u - (c & 1u)));
  }
  return ~c;
}

static void reseal(std::vector<uint8_t>& b) {
  uint64_t total;
  memcpy(&total, b.data() + 32, 8);
  const uint32_t c = crc32_bitwise(b.data() + 128, (size_t)(total - 128));
  memcpy(b.data() + 48, &c, 4);
}

int main(int argc, char** argv) {
  if (argc != 6) {
    fprintf(stderr, "usage: %s E dout r in.bin out.bin\n", argv[0]);
    return 2;
  }
  const int E = atoi(argv[1]), dout = atoi(argv[2]), r = atoi(argv[3]);
  const size_t n = (size_t)E * r;
  std::vector<float> p(n * dout), a(n);
  std::vector<uint8_t> bits(n);
  FILE* f = fopen(argv[4], "rb");
  if (!f) return 2;
  const bool ok_read = fread(p.data(), 4, p.size(), f) == p.size() &&
                       fread(a.data(), 4, a.size(), f) == a.size() &&
                       fread(bits.data(), 1, bits.size(), f) == bits.size();
  fclose(f);
  if (!ok_read) return 2;

  size_t need = 0;
  EXPECT(bitsmoe_pack_size(E, dout, r, bits.data(), &need) == BITSMOE_OK, "pack_size");
  std::vector<uint8_t> blob(need + 64, 0xAB);
  EXPECT(bitsmoe_pack(E, dout, r, p.data(), a.data(), bits.data(), blob.data(), need - 1) ==
             BITSMOE_ENOSPC, "pack into a short buffer");
  EXPECT(bitsmoe_pack(E, dout, r, p.data(), a.data(), bits.data(), blob.data(), need) ==
             BITSMOE_OK, "pack");
  for (size_t i = need; i < blob.size(); ++i) EXPECT(blob[i] == 0xAB, "write past the blob");
  blob.resize(need);
  f = fopen(argv[5], "wb");
  if (!f || fwrite(blob.data(), 1, blob.size(), f) != blob.size()) return 2;
  fclose(f);

  int e2 = 0, d2 = 0, r2 = 0;
  EXPECT(bitsmoe_blob_check(blob.data(), blob.size(), &e2, &d2, &r2) == BITSMOE_OK, "check");
  EXPECT(e2 == E && d2 == dout && r2 == r, "check dims");
  EXPECT(bitsmoe_blob_check(blob.data(), blob.size() - 1, 0, 0, 0) != BITSMOE_OK, "truncated");
  EXPECT(bitsmoe_blob_check(blob.data(), 100, 0, 0, 0) == BITSMOE_EFORMAT, "short header");
  EXPECT(bitsmoe_blob_check(nullptr, blob.size(), 0, 0, 0) == BITSMOE_EINVAL, "null blob");

  // a flipped bit anywhere past the header fails the checksum
  const size_t step = need > 4096 ? need / 997 : 1;
  for (size_t i = 128; i < need; i += step) {
    blob[i] ^= 0x10;
    EXPECT(bitsmoe_blob_check(blob.data(), blob.size(), 0, 0, 0) != BITSMOE_OK, "bit flip");
    blob[i] ^= 0x10;
  }
  // header fields.  Not r (16): a larger rank still describes a consistent
  // blob whose extra components are 0-bit everywhere, and the device kernels
  // compare it with the call's r.  dout (12) flipped by 32 rows, across a
  // segment: a change inside the last segment's padding is consistent too.
  const int fields[][2] = {{0, 1},  {4, 1},  {8, 1},  {12, 32}, {20, 1}, {24, 1},
                           {28, 1}, {32, 1}, {40, 1}, {48, 1}, {56, 16}};
  for (const auto& fm : fields) {
    blob[fm[0]] ^= (uint8_t)fm[1];
    EXPECT(bitsmoe_blob_check(blob.data(), blob.size(), 0, 0, 0) != BITSMOE_OK, "header field");
    blob[fm[0]] ^= (uint8_t)fm[1];
  }
  // directory records changed and re-sealed: every byte but the float bound
  // (40..43, only required finite and >= 0) must be caught by the check
  for (int e = 0; e < E && e < 4; ++e)
    for (int b = 0; b < 64; ++b) {
      std::vector<uint8_t> c = blob;
      c[128 + 64 * e + b] ^= 0xFF;
      reseal(c);
      const int st = bitsmoe_blob_check(c.data(), c.size(), 0, 0, 0);
      if (b < 40 || b >= 44) EXPECT(st != BITSMOE_OK, "directory byte");
    }
  // a column index out of range, re-sealed
  {
    std::vector<uint8_t> c = blob;
    uint64_t off0;
    memcpy(&off0, c.data() + 128, 8);
    uint32_t n_nz;
    memcpy(&n_nz, c.data() + 128 + 8, 4);
    if (n_nz > 0) {
      c[off0] = 0xFF;
      c[off0 + 1] = 0xFF;
      reseal(c);
      EXPECT(bitsmoe_blob_check(c.data(), c.size(), 0, 0, 0) == BITSMOE_EFORMAT, "kidx range");
    }
  }

  // the component -> slot index, changed and re-sealed: an entry moved to
  // another slot, and a dropped component given a slot
  {
    const size_t io = (128 + 64 * (size_t)E + 255) / 256 * 256;
    uint16_t* idx0 = nullptr;
    std::vector<uint8_t> c = blob;
    idx0 = (uint16_t*)(c.data() + io);
    int k_stored = -1, k_dropped = -1;
    for (int k = 0; k < r; ++k) {
      if (idx0[k] != 0xFFFF && k_stored < 0) k_stored = k;
      if (idx0[k] == 0xFFFF && k_dropped < 0) k_dropped = k;
    }
    if (k_stored >= 0) {
      idx0[k_stored] ^= 1;
      reseal(c);
      EXPECT(bitsmoe_blob_check(c.data(), c.size(), 0, 0, 0) == BITSMOE_EFORMAT, "slot index");
    }
    if (k_dropped >= 0) {
      c = blob;
      idx0 = (uint16_t*)(c.data() + io);
      idx0[k_dropped] = 0;
      reseal(c);
      EXPECT(bitsmoe_blob_check(c.data(), c.size(), 0, 0, 0) == BITSMOE_EFORMAT,
             "slot index extra");
    }
  }

  // bad arguments
  size_t tmp = 0;
  EXPECT(bitsmoe_pack_size(0, dout, r, bits.data(), &tmp) == BITSMOE_ESHAPE, "E = 0");
  EXPECT(bitsmoe_pack_size(E, dout, r, bits.data(), nullptr) == BITSMOE_EINVAL, "null size");
  EXPECT(bitsmoe_pack(E, dout, r, nullptr, a.data(), bits.data(), blob.data(), need) ==
             BITSMOE_EINVAL, "null p");
  {
    std::vector<uint8_t> b2 = bits;
    b2[0] = 5;
    EXPECT(bitsmoe_pack_size(E, dout, r, b2.data(), &tmp) == BITSMOE_EBITS, "width 5");
  }
  {
    size_t k = 0;
    while (k < n && bits[k] == 0) ++k;
    if (k < n) {
      std::vector<float> p2 = p;
      p2[k * dout] = 1.0f / 0.0f;
      EXPECT(bitsmoe_pack(E, dout, r, p2.data(), a.data(), bits.data(), blob.data(), need) ==
                 BITSMOE_EBITS, "infinite p");
      p2[k * dout] = 70000.0f;
      EXPECT(bitsmoe_pack(E, dout, r, p2.data(), a.data(), bits.data(), blob.data(), need) ==
                 BITSMOE_EBITS, "|p| > 60000");
    }
  }
  for (int s = -8; s <= 1; ++s) EXPECT(bitsmoe_strerror(s) != nullptr, "strerror");
  EXPECT(bitsmoe_last_error_detail() != nullptr, "detail");
  EXPECT(bitsmoe_version() > 0, "version");
  if (g_miss) fprintf(stderr, "%d expectation(s) missed\n", g_miss);
  return g_miss ? 1 : 0;
}
