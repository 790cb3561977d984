"""Independent writer and reader of the packed spectral-expert blob (format v1).

Source: BitsMoE blog note, "Methodology / execution": components of the same
width are placed together and then packed by bit plane so that a GPU can
process the mixed widths regularly.  The concrete byte layout below is this
project's own (the pages give none); the HIP library's packer writes the same
bytes from its own C++ code, and the tests compare the two.

Layout (little-endian; offsets in bytes from the blob base):

Header, 128 bytes
  0 'BMOE' | 4 u32 version=1 | 8 u32 E | 12 u32 dout | 16 u32 r
  20 u32 dout_pad = 64*ceil(dout/64) | 24 u32 n_slabs = dout_pad/64
  28 u32 header_bytes=128 | 32 u64 total_bytes | 40 u64 dir_offset=128
  48 u32 CRC-32 (IEEE, as zlib) of bytes [128, total_bytes) | rest zero
Directory, E records of 64 bytes at dir_offset
  0 u64 block_offset | 8 u32 n_nz | 12 u32 n_q | 16 u32 n_16
  20 u32 masks_per_slab = sum of b over the 1..8-bit columns
  24 u32 a_off | 28 u32 s_off | 32 u32 m_off | 36 u32 planes_off
  40 u32 f16_off | 44 u32 block_bytes (offsets relative to block_offset)
  48 u16 count of columns of width 1,2,3,4,6,8,16 (7 values) | 62 u16 0
Expert block (first at align256(128 + 64 E), blocks back to back)
  column order: width groups 1,2,3,4,6,8,16, ascending k inside a group;
  0-bit columns have no entry at all
  kidx   u16[n_nz]                 at 0
  a      f32[n_nz]                 at a_off      = align16(2 n_nz)
  s      f16[n_q]                  at s_off      = align16(a_off + 4 n_nz)
  m      f16[n_q]                  at m_off      = align16(s_off + 2 n_q)
  planes u64[n_slabs][masks_per_slab] at planes_off = align256(m_off + 2 n_q)
         per 64-row slab, for each 1..8-bit column in order and each plane
         j = 0..b-1 (j = 0 is the least significant code bit): one u64 whose
         bit t is bit j of q[64*slab + t] (0 for rows >= dout)
  f16    f16[n_16][dout_pad]       at f16_off = align256(planes_off + 8 n_slabs mps + 16)
         fp16 values of the 16-bit columns (rows >= dout are 0)
  block_bytes = align256(f16_off + 2 n_16 dout_pad)
All padding bytes are zero.
"""
import struct
import zlib

import numpy as np

from .quantize import quantize_expert

MAGIC = b"BMOE"
VERSION = 1
HEADER_BYTES = 128
DIR_REC = 64
GROUP_WIDTHS = (1, 2, 3, 4, 6, 8, 16)


def _al(x: int, a: int) -> int:
    return (x + a - 1) // a * a


def _block_layout(bits_e: np.ndarray, n_slabs: int, dout_pad: int):
    cnt = [int(np.count_nonzero(bits_e == w)) for w in GROUP_WIDTHS]
    n_nz = sum(cnt)
    n_16 = cnt[-1]
    n_q = n_nz - n_16
    mps = sum(w * c for w, c in zip(GROUP_WIDTHS[:-1], cnt[:-1]))
    a_off = _al(2 * n_nz, 16)
    s_off = _al(a_off + 4 * n_nz, 16)
    m_off = _al(s_off + 2 * n_q, 16)
    p_off = _al(m_off + 2 * n_q, 256)
    f_off = _al(p_off + 8 * n_slabs * mps + 16, 256)
    nbytes = _al(f_off + 2 * n_16 * dout_pad, 256)
    return dict(cnt=cnt, n_nz=n_nz, n_q=n_q, n_16=n_16, mps=mps, a_off=a_off,
                s_off=s_off, m_off=m_off, p_off=p_off, f_off=f_off, nbytes=nbytes)


def _column_order(bits_e: np.ndarray):
    return np.concatenate([np.nonzero(bits_e == w)[0] for w in GROUP_WIDTHS]).astype(np.int64)


def pack(p: np.ndarray, a: np.ndarray, bits: np.ndarray) -> bytes:
    """Quantize (oracle quantizer) and pack one linear type.

    p: E x r x dout float32 unit columns, a: E x r float32, bits: E x r.
    """
    E, r, dout = p.shape
    dout_pad = _al(dout, 64)
    n_slabs = dout_pad // 64
    lays = [_block_layout(bits[e], n_slabs, dout_pad) for e in range(E)]
    first = _al(HEADER_BYTES + DIR_REC * E, 256)
    offs = []
    pos = first
    for L in lays:
        offs.append(pos)
        pos += L["nbytes"]
    total = pos
    buf = bytearray(total)
    for e in range(E):
        L = lays[e]
        base = offs[e]
        order = _column_order(bits[e])
        qe = quantize_expert(p[e], bits[e])
        struct.pack_into("<QIIIIIIIIII", buf, HEADER_BYTES + DIR_REC * e,
                         base, L["n_nz"], L["n_q"], L["n_16"], L["mps"],
                         L["a_off"], L["s_off"], L["m_off"], L["p_off"],
                         L["f_off"], L["nbytes"])
        struct.pack_into("<7H", buf, HEADER_BYTES + DIR_REC * e + 48, *L["cnt"])
        n_nz, n_q = L["n_nz"], L["n_q"]
        buf[base:base + 2 * n_nz] = order.astype("<u2").tobytes()
        buf[base + L["a_off"]:base + L["a_off"] + 4 * n_nz] = \
            a[e][order].astype("<f4").tobytes()
        qorder = order[:n_q]
        buf[base + L["s_off"]:base + L["s_off"] + 2 * n_q] = qe["s"][qorder].astype("<f2").tobytes()
        buf[base + L["m_off"]:base + L["m_off"] + 2 * n_q] = qe["m"][qorder].astype("<f2").tobytes()
        # bit planes: codes padded to dout_pad rows
        planes = np.zeros((n_slabs, L["mps"]), dtype="<u8")
        col = 0
        for w in GROUP_WIDTHS[:-1]:
            g = np.nonzero(bits[e] == w)[0]
            if g.size == 0:
                continue
            Q = np.zeros((g.size, dout_pad), dtype=np.uint16)
            Q[:, :dout] = qe["q"][g]
            for j in range(w):
                bj = ((Q >> j) & 1).astype(np.uint8).reshape(g.size, n_slabs, 64)
                packed = np.packbits(bj, axis=2, bitorder="little")  # g x slabs x 8
                words = packed.reshape(g.size, n_slabs * 8).view("<u8").reshape(g.size, n_slabs)
                planes[:, col + j:col + w * g.size:w] = words.T
            col += w * g.size
        assert col == L["mps"]
        buf[base + L["p_off"]:base + L["p_off"] + planes.nbytes] = planes.tobytes()
        g16 = np.nonzero(bits[e] == 16)[0]
        if g16.size:
            F = np.zeros((g16.size, dout_pad), dtype="<u2")
            F[:, :dout] = qe["q"][g16]
            buf[base + L["f_off"]:base + L["f_off"] + F.nbytes] = F.tobytes()
    struct.pack_into("<4sIIIIIII", buf, 0, MAGIC, VERSION, E, dout, r,
                     dout_pad, n_slabs, HEADER_BYTES)
    struct.pack_into("<QQ", buf, 32, total, HEADER_BYTES)
    struct.pack_into("<I", buf, 48, zlib.crc32(memoryview(buf)[HEADER_BYTES:]) & 0xFFFFFFFF)
    return bytes(buf)


def read_header(blob) -> dict:
    mv = memoryview(blob)
    magic, ver, E, dout, r, dout_pad, n_slabs, hb = struct.unpack_from("<4sIIIIIII", mv, 0)
    total, dir_off = struct.unpack_from("<QQ", mv, 32)
    crc, = struct.unpack_from("<I", mv, 48)
    return dict(magic=magic, version=ver, E=E, dout=dout, r=r, dout_pad=dout_pad,
                n_slabs=n_slabs, header_bytes=hb, total_bytes=total,
                dir_offset=dir_off, crc32=crc)


def unpack(blob) -> dict:
    """Read codes back: returns dict with per-expert arrays in k order.

    'q'   E x r x dout uint16 (codes; fp16 bit patterns for b = 16; 0 for b = 0)
    's','m' E x r float16, 'a' E x r float32 (0 for b = 0), 'bits' E x r uint8
    """
    H = read_header(blob)
    if H["magic"] != MAGIC or H["version"] != VERSION:
        raise ValueError("not a v1 BMOE blob")
    if zlib.crc32(memoryview(blob)[HEADER_BYTES:H["total_bytes"]]) & 0xFFFFFFFF != H["crc32"]:
        raise ValueError("CRC mismatch")
    E, r, dout, dp, ns = H["E"], H["r"], H["dout"], H["dout_pad"], H["n_slabs"]
    q = np.zeros((E, r, dout), dtype=np.uint16)
    s = np.ones((E, r), dtype=np.float16)
    m = np.zeros((E, r), dtype=np.float16)
    a = np.zeros((E, r), dtype=np.float32)
    bits = np.zeros((E, r), dtype=np.uint8)
    buf = np.frombuffer(blob, dtype=np.uint8)
    for e in range(E):
        (base, n_nz, n_q, n_16, mps, a_off, s_off, m_off, p_off, f_off,
         nbytes) = struct.unpack_from("<QIIIIIIIIII", blob, H["dir_offset"] + DIR_REC * e)
        cnt = struct.unpack_from("<7H", blob, H["dir_offset"] + DIR_REC * e + 48)
        order = buf[base:base + 2 * n_nz].view("<u2").astype(np.int64)
        a[e, order] = buf[base + a_off:base + a_off + 4 * n_nz].view("<f4")
        qo = order[:n_q]
        s[e, qo] = buf[base + s_off:base + s_off + 2 * n_q].view("<f2")
        m[e, qo] = buf[base + m_off:base + m_off + 2 * n_q].view("<f2")
        planes = buf[base + p_off:base + p_off + 8 * ns * mps].view("<u8").reshape(ns, mps)
        col = 0
        ci = 0
        for w, c in zip(GROUP_WIDTHS, cnt):
            ks = order[ci:ci + c]
            ci += c
            if c == 0:
                continue
            bits[e, ks] = w
            if w == 16:
                continue
            Q = np.zeros((c, dp), dtype=np.uint16)
            for j in range(w):
                words = np.ascontiguousarray(planes[:, col + j:col + w * c:w].T)  # c x ns
                bj = np.unpackbits(words.view(np.uint8).reshape(c, ns, 8), axis=2,
                                   bitorder="little").reshape(c, dp)
                Q |= (bj.astype(np.uint16) << j)
            q[e, ks] = Q[:, :dout]
            col += w * c
        if n_16:
            F = buf[base + f_off:base + f_off + 2 * n_16 * dp].view("<u2").reshape(n_16, dp)
            q[e, order[n_q:]] = F[:, :dout]
    return dict(header=H, q=q, s=s, m=m, a=a, bits=bits)
