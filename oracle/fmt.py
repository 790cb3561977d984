"""Independent writer and reader of the packed spectral-expert blob (format v4).

Test infrastructure: only the tests, the smoke check and the benchmark's CPU
baseline use this module; the HIP library never imports it.

Source: BitsMoE blog note, "Methodology / execution": components of the same
width are placed together and then packed by bit plane so that a GPU can
process the mixed widths regularly.  The concrete byte layout below is this
project's own (the pages give none); the HIP library's packer writes the same
bytes from its own C++ code, and the tests compare the two.

Layout (little-endian; offsets in bytes from the blob base):

Header, 128 bytes
  0 'BMOE' | 4 u32 version=4 | 8 u32 E | 12 u32 dout | 16 u32 r
  20 u32 dout_pad = 32*ceil(dout/32) | 24 u32 n_seg = dout_pad/32
  28 u32 header_bytes=128 | 32 u64 total_bytes | 40 u64 dir_offset=128
  48 u32 CRC-32 (IEEE, as zlib) of bytes [128, total_bytes)
  56 u64 ctab_offset = align256(128 + 64 E) | rest zero
Directory, E records of 64 bytes at dir_offset
  0 u64 block_offset | 8 u32 n_nz | 12 u32 n_q | 16 u32 n_16
  20 u32 seg_words (u32 words of one 32-row segment record)
  24 u32 a_off | 28 u32 s_off | 32 u32 m_off | 36 u32 planes_off
  40 f32 cmax | 44 u32 block_bytes (offsets relative to block_offset)
  48 u16 count of columns of width 1,2,3,4,6,8,16 (7 values) | 62 u16 0
  cmax = max over the expert's stored columns of |a_k| * s_k (1..8 bits,
  float32 product) or |a_k| (16 bits); 0 when the expert stores none.
Component table at ctab_offset: for expert e, at e * stride, with
  R2 = align16(2 r), stride = 3 R2 + align16(4 r) + 16:
  0      u16 slot[r]: slot of component k in expert e's slot order (below),
         0xFFFF when component k has width 0
  R2     f16 s[r], 2 R2: f16 m[r]: scale and offset of 1..8-bit components
         (0 for 16-bit and 0-bit ones)
  3 R2   f32 a[r] (0 for 0-bit components)
  3 R2 + align16(4 r): f32 cmax (as in the directory), then 12 zero bytes
  (the same values as the expert block's slot arrays, in component order)
Expert block (first at align256(ctab_offset + E stride), blocks back to
back)
  slot order: width groups 1,2,3,4,6,8,16; inside a group the columns in
  ascending k, then zero slots up to a multiple of 32 (nb_w = 8 ceil(n_w /
  32) blocks of 4 slots per group, so that a 32-slot step never mixes
  widths); 0-bit columns have no slot at all.
  n_slot = 4 * sum nb_w, n_qslot = 4 * sum of nb_w over widths 1..8.
  kidx   u16[n_slot]  at 0                   (0 in padding slots)
  a      f32[n_slot]  at a_off  = align16(2 n_slot)          (0 in padding)
  s      f16[n_qslot] at s_off  = align16(a_off + 4 n_slot)  (0 in padding)
  m      f16[n_qslot] at m_off  = align16(s_off + 2 n_qslot) (0 in padding)
  planes u32[n_seg][seg_words] at planes_off = align256(m_off + 2 n_qslot)
         one record per 32-row segment; inside it, block after block in slot
         order, 4*w words per block of width w: for row octet i = 0..3
         (segment rows 8i..8i+7) w words.
         w <= 8: word (i, j), j = 0..w-1 is plane j; its bit 8*u + rho is
         bit j (j = 0 least significant) of the code of segment row 8i + rho
         in slot 4*beta + u.
         w = 16: word (i, 2*rho + h) holds the fp16 values of segment row
         8i + rho in slots 4*beta + 2h (low half) and 4*beta + 2h + 1.
         seg_words = 4 * sum over blocks of w.  Rows >= dout are 0.
  block_bytes = align256(planes_off + 4 n_seg seg_words + 16)
All padding bytes are zero.
"""
import struct
import zlib

import numpy as np

from .quantize import quantize_expert

MAGIC = b"BMOE"
VERSION = 4
HEADER_BYTES = 128
DIR_REC = 64
SEG_ROWS = 32
GROUP_WIDTHS = (1, 2, 3, 4, 6, 8, 16)


def _al(x: int, a: int) -> int:
    return (x + a - 1) // a * a


def ctab_offset(E: int) -> int:
    return _al(HEADER_BYTES + DIR_REC * E, 256)


def ctab_layout(r: int) -> dict:
    """Byte offsets of the component table's arrays inside one expert's entry."""
    r2 = _al(2 * r, 16)
    return dict(slot=0, s=r2, m=2 * r2, a=3 * r2, cmax=3 * r2 + _al(4 * r, 16),
                stride=3 * r2 + _al(4 * r, 16) + 16)


def plane_bit(rho, u):
    """Bit position of (row rho of an octet, slot u of a block) in a plane word:
    byte u holds the octet's 8 rows of slot u."""
    return 8 * u + rho


GROUP_SLOTS = 32   # each width group is padded to a multiple of this


def _block_layout(cnt, n_seg: int):
    nb = [(c + GROUP_SLOTS - 1) // GROUP_SLOTS * (GROUP_SLOTS // 4) for c in cnt]
    n_nz = sum(cnt)
    n_16 = cnt[-1]
    n_q = n_nz - n_16
    n_slot = 4 * sum(nb)
    n_qslot = 4 * sum(nb[:-1])
    seg_words = 4 * sum(n * w for n, w in zip(nb, GROUP_WIDTHS))
    a_off = _al(2 * n_slot, 16)
    s_off = _al(a_off + 4 * n_slot, 16)
    m_off = _al(s_off + 2 * n_qslot, 16)
    p_off = _al(m_off + 2 * n_qslot, 256)
    nbytes = _al(p_off + 4 * n_seg * seg_words + 16, 256)
    return dict(cnt=list(cnt), nb=nb, n_nz=n_nz, n_q=n_q, n_16=n_16, n_slot=n_slot,
                n_qslot=n_qslot, seg_words=seg_words, a_off=a_off, s_off=s_off,
                m_off=m_off, p_off=p_off, nbytes=nbytes)


def _slots(bits_e: np.ndarray):
    """Column index per slot (-1 for padding), group after group."""
    out = []
    for w in GROUP_WIDTHS:
        cols = np.nonzero(bits_e == w)[0]
        pad = (-cols.size) % GROUP_SLOTS
        out.append(np.concatenate([cols, np.full(pad, -1)]))
    return np.concatenate(out).astype(np.int64)


def _plane_words(Q: np.ndarray, w: int, n_seg: int) -> np.ndarray:
    """Segment records of one width group: n_seg x (nb * 4 * w) uint32.

    Q: (4 nb) x dout_pad codes (w <= 8) or fp16 bit patterns (w = 16),
    one row per slot of the group.
    """
    nb = Q.shape[0] // 4
    if w == 16:
        # [beta][pair h][low/high][seg][octet i][rho]
        F = Q.astype(np.uint32).reshape(nb, 2, 2, n_seg, 4, 8)
        word = F[:, :, 0] | (F[:, :, 1] << 16)            # beta, h, seg, i, rho
        return np.ascontiguousarray(word.transpose(2, 0, 3, 4, 1)).reshape(n_seg, nb * 64)
    # [beta][u][seg][octet i][rho]
    V = Q.astype(np.uint32).reshape(nb, 4, n_seg, 4, 8)
    rho = np.arange(8).reshape(1, 1, 1, 1, 8)
    u = np.arange(4).reshape(1, 4, 1, 1, 1)
    sh = plane_bit(rho, u).astype(np.uint32)
    planes = []
    for j in range(w):
        bit = (V >> j) & 1
        planes.append(np.bitwise_or.reduce(bit << sh, axis=(1, 4)))  # beta, seg, i
    P = np.stack(planes, axis=-1)                          # beta, seg, i, j
    return np.ascontiguousarray(P.transpose(1, 0, 2, 3)).reshape(n_seg, nb * 4 * w)


def pack(p: np.ndarray, a: np.ndarray, bits: np.ndarray) -> bytes:
    """Quantize (oracle quantizer) and pack one linear type.

    p: E x r x dout float32 unit columns, a: E x r float32, bits: E x r.
    """
    E, r, dout = p.shape
    dout_pad = _al(dout, SEG_ROWS)
    n_seg = dout_pad // SEG_ROWS
    lays = []
    for e in range(E):
        cnt = [int(np.count_nonzero(bits[e] == w)) for w in GROUP_WIDTHS]
        lays.append(_block_layout(cnt, n_seg))
    CT = ctab_layout(r)
    first = _al(ctab_offset(E) + E * CT["stride"], 256)
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
        slots = _slots(bits[e])
        real = slots >= 0

        ks = np.where(real, slots, 0)
        qe = quantize_expert(p[e], bits[e])
        a_s = np.where(real, a[e][ks], np.float32(0)).astype("<f4")
        qs = L["n_qslot"]
        s_s = np.where(real[:qs], qe["s"][ks[:qs]], np.float16(0)).astype("<f2")
        m_s = np.where(real[:qs], qe["m"][ks[:qs]], np.float16(0)).astype("<f2")
        # coefficient bound: |a| * s (float32 product) or |a| for 16-bit columns
        cmax = np.float32(0)
        if real[:qs].any():
            cmax = max(cmax, np.max(np.abs(a_s[:qs][real[:qs]]) *
                                    s_s[real[:qs]].astype(np.float32)))
        if real[qs:].any():
            cmax = max(cmax, np.max(np.abs(a_s[qs:][real[qs:]])))
        struct.pack_into("<QIIIIIIIIfI", buf, HEADER_BYTES + DIR_REC * e,
                         base, L["n_nz"], L["n_q"], L["n_16"], L["seg_words"],
                         L["a_off"], L["s_off"], L["m_off"], L["p_off"],
                         float(cmax), L["nbytes"])
        struct.pack_into("<7H", buf, HEADER_BYTES + DIR_REC * e + 48, *L["cnt"])
        # component table: the stored slots' values in component order
        cslot = np.full(r, 0xFFFF, dtype="<u2")
        cs = np.zeros(r, dtype="<f2")
        cm = np.zeros(r, dtype="<f2")
        ca = np.zeros(r, dtype="<f4")
        sl_real = np.nonzero(real)[0]
        cslot[slots[sl_real]] = sl_real
        ca[slots[sl_real]] = a_s[sl_real]
        q_real = sl_real[sl_real < qs]
        cs[slots[q_real]] = s_s[q_real]
        cm[slots[q_real]] = m_s[q_real]
        co = ctab_offset(E) + e * CT["stride"]
        buf[co + CT["slot"]:co + CT["slot"] + 2 * r] = cslot.tobytes()
        buf[co + CT["s"]:co + CT["s"] + 2 * r] = cs.tobytes()
        buf[co + CT["m"]:co + CT["m"] + 2 * r] = cm.tobytes()
        buf[co + CT["a"]:co + CT["a"] + 4 * r] = ca.tobytes()
        struct.pack_into("<f", buf, co + CT["cmax"], float(cmax))
        n_slot = L["n_slot"]
        buf[base:base + 2 * n_slot] = ks.astype("<u2").tobytes()
        buf[base + L["a_off"]:base + L["a_off"] + 4 * n_slot] = a_s.tobytes()
        buf[base + L["s_off"]:base + L["s_off"] + 2 * qs] = s_s.tobytes()
        buf[base + L["m_off"]:base + L["m_off"] + 2 * qs] = m_s.tobytes()
        planes = np.zeros((n_seg, L["seg_words"]), dtype="<u4")
        col = 0   # word offset inside a segment record
        sl = 0    # first slot of the group
        for w, nb in zip(GROUP_WIDTHS, L["nb"]):
            if nb == 0:
                continue
            gs = slots[sl:sl + 4 * nb]
            Q = np.zeros((4 * nb, dout_pad), dtype=np.uint16)
            Q[gs >= 0, :dout] = qe["q"][gs[gs >= 0]]
            planes[:, col:col + 4 * w * nb] = _plane_words(Q, w, n_seg)
            col += 4 * w * nb
            sl += 4 * nb
        assert col == L["seg_words"]
        buf[base + L["p_off"]:base + L["p_off"] + planes.nbytes] = planes.tobytes()
    struct.pack_into("<4sIIIIIII", buf, 0, MAGIC, VERSION, E, dout, r,
                     dout_pad, n_seg, HEADER_BYTES)
    struct.pack_into("<QQ", buf, 32, total, HEADER_BYTES)
    struct.pack_into("<Q", buf, 56, ctab_offset(E))
    struct.pack_into("<I", buf, 48, zlib.crc32(memoryview(buf)[HEADER_BYTES:]) & 0xFFFFFFFF)
    return bytes(buf)


def read_header(blob) -> dict:
    mv = memoryview(blob)
    magic, ver, E, dout, r, dout_pad, n_seg, hb = struct.unpack_from("<4sIIIIIII", mv, 0)
    total, dir_off = struct.unpack_from("<QQ", mv, 32)
    crc, = struct.unpack_from("<I", mv, 48)
    cto, = struct.unpack_from("<Q", mv, 56)
    return dict(magic=magic, version=ver, E=E, dout=dout, r=r, dout_pad=dout_pad,
                n_seg=n_seg, header_bytes=hb, total_bytes=total,
                dir_offset=dir_off, crc32=crc, ctab_offset=cto)


def read_ctab(blob, e: int) -> dict:
    """Expert e's component table: 'slot' int64 (-1 for width 0), 's', 'm'
    float16, 'a' float32 (component order) and 'cmax' float32."""
    H = read_header(blob)
    CT = ctab_layout(H["r"])
    r = H["r"]
    o = H["ctab_offset"] + e * CT["stride"]
    slot = np.frombuffer(blob, dtype="<u2", count=r, offset=o + CT["slot"]).astype(np.int64)
    return dict(slot=np.where(slot == 0xFFFF, -1, slot),
                s=np.frombuffer(blob, dtype="<f2", count=r, offset=o + CT["s"]),
                m=np.frombuffer(blob, dtype="<f2", count=r, offset=o + CT["m"]),
                a=np.frombuffer(blob, dtype="<f4", count=r, offset=o + CT["a"]),
                cmax=np.frombuffer(blob, dtype="<f4", count=1, offset=o + CT["cmax"])[0])


def read_dir(blob, e: int) -> dict:
    H = read_header(blob)
    off = H["dir_offset"] + DIR_REC * e
    (base, n_nz, n_q, n_16, seg_words, a_off, s_off, m_off, p_off, cmax,
     nbytes) = struct.unpack_from("<QIIIIIIIIfI", blob, off)
    cnt = struct.unpack_from("<7H", blob, off + 48)
    return dict(block_offset=base, n_nz=n_nz, n_q=n_q, n_16=n_16, seg_words=seg_words,
                a_off=a_off, s_off=s_off, m_off=m_off, p_off=p_off, cmax=cmax,
                block_bytes=nbytes, count=cnt)


def _plane_codes(words: np.ndarray, w: int, nb: int, n_seg: int) -> np.ndarray:
    """Inverse of _plane_words: (4 nb) x dout_pad codes / fp16 bit patterns."""
    if w == 16:
        Wd = words.reshape(n_seg, nb, 4, 8, 2)             # seg, beta, i, rho, h
        lo = (Wd & 0xFFFF).astype(np.uint16)
        hi = (Wd >> 16).astype(np.uint16)
        F = np.stack([lo, hi], axis=-1)                    # seg, beta, i, rho, h, lh
        return np.ascontiguousarray(F.transpose(1, 4, 5, 0, 2, 3)).reshape(4 * nb, n_seg * 32)
    Wd = words.reshape(n_seg, nb, 4, w)                    # seg, beta, i, j
    Q = np.zeros((nb, 4, n_seg, 4, 8), dtype=np.uint16)    # beta, u, seg, i, rho
    for j in range(w):
        pj = Wd[:, :, :, j].transpose(1, 0, 2)             # beta, seg, i
        for u in range(4):
            for rho in range(8):
                bit = (pj >> plane_bit(rho, u)) & 1
                Q[:, u, :, :, rho] |= (bit.astype(np.uint16) << j)
    return Q.reshape(4 * nb, n_seg * 32)


def unpack(blob, experts=None) -> dict:
    """Read codes back: returns dict with per-expert arrays in k order.

    'q'   E x r x dout uint16 (codes; fp16 bit patterns for b = 16; 0 for b = 0)
    's','m' E x r float16, 'a' E x r float32 (0 for b = 0), 'bits' E x r uint8,
    'cmax' E float32 (the directory's coefficient bound)
    experts: None for all, else a list of expert ids; row i of every array
    then belongs to experts[i].
    """
    H = read_header(blob)
    if H["magic"] != MAGIC or H["version"] != VERSION:
        raise ValueError("not a v%d BMOE blob" % VERSION)
    if H["ctab_offset"] != ctab_offset(H["E"]):
        raise ValueError("component table offset %d, expected %d" % (H["ctab_offset"],
                                                                     ctab_offset(H["E"])))
    if zlib.crc32(memoryview(blob)[HEADER_BYTES:H["total_bytes"]]) & 0xFFFFFFFF != H["crc32"]:
        raise ValueError("CRC mismatch")
    E, r, dout, dp, ns = H["E"], H["r"], H["dout"], H["dout_pad"], H["n_seg"]
    sel = list(range(E)) if experts is None else [int(e) for e in experts]
    if any(e < 0 or e >= E for e in sel):
        raise ValueError("expert id outside [0, %d)" % E)
    n = len(sel)
    q = np.zeros((n, r, dout), dtype=np.uint16)
    s = np.ones((n, r), dtype=np.float16)
    m = np.zeros((n, r), dtype=np.float16)
    a = np.zeros((n, r), dtype=np.float32)
    bits = np.zeros((n, r), dtype=np.uint8)
    cmax = np.zeros(n, dtype=np.float32)
    buf = np.frombuffer(blob, dtype=np.uint8)
    for e, ex in enumerate(sel):
        D = read_dir(blob, ex)
        cmax[e] = D["cmax"]
        L = _block_layout(list(D["count"]), ns)
        base = D["block_offset"]
        n_slot, qs = L["n_slot"], L["n_qslot"]
        kidx = buf[base:base + 2 * n_slot].view("<u2").astype(np.int64)
        a_s = buf[base + D["a_off"]:base + D["a_off"] + 4 * n_slot].view("<f4")
        s_s = buf[base + D["s_off"]:base + D["s_off"] + 2 * qs].view("<f2")
        m_s = buf[base + D["m_off"]:base + D["m_off"] + 2 * qs].view("<f2")
        planes = buf[base + D["p_off"]:base + D["p_off"] + 4 * ns * L["seg_words"]]
        planes = planes.view("<u4").reshape(ns, L["seg_words"])
        CTe = read_ctab(blob, ex)
        sidx = CTe["slot"]
        if np.count_nonzero(sidx >= 0) != D["n_nz"]:
            raise ValueError("expert %d: component table has extra entries" % ex)
        col = 0
        sl = 0
        for w, c, nb in zip(GROUP_WIDTHS, D["count"], L["nb"]):
            if nb == 0:
                continue
            ks = kidx[sl:sl + c]
            if not np.array_equal(sidx[ks], np.arange(sl, sl + c)) or \
                    not np.array_equal(CTe["a"][ks].view("<u4"), a_s[sl:sl + c].view("<u4")):
                raise ValueError("expert %d: component table does not match its columns" % ex)
            if w != 16 and not (np.array_equal(CTe["s"][ks].view("<u2"), s_s[sl:sl + c].view("<u2"))
                                and np.array_equal(CTe["m"][ks].view("<u2"),
                                                   m_s[sl:sl + c].view("<u2"))):
                raise ValueError("expert %d: component table does not match its columns" % ex)
            bits[e, ks] = w
            a[e, ks] = a_s[sl:sl + c]
            if w != 16:
                s[e, ks] = s_s[sl:sl + c]
                m[e, ks] = m_s[sl:sl + c]
            Q = _plane_codes(planes[:, col:col + 4 * w * nb], w, nb, ns)
            q[e, ks] = Q[:c, :dout]
            col += 4 * w * nb
            sl += 4 * nb
    return dict(header=H, q=q, s=s, m=m, a=a, bits=bits, cmax=cmax)
