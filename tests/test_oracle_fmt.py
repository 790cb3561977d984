"""Pins of the oracle's independent packer/reader (oracle/fmt.py).

A hand-built one-expert blob whose plane words were worked out by hand, the
round trip unpack(pack(q)) == q over every width, the 96-row tail, empty
groups, all-0 and all-16 experts, header fields, alignment and the CRC.
"""
import struct
import zlib

import numpy as np
import pytest

from oracle import fmt
from oracle.quantize import quantize_expert


def test_hand_built_planes():
    # one expert, r = 3: column 0 at 2 bits with codes [0,1,2,3] (the first
    # hand-derived quantizer case), column 1 dropped, column 2 at 1 bit.
    p = np.zeros((1, 3, 4), np.float32)
    p[0, 0] = [-0.5, -0.1, 0.2, 0.5]
    p[0, 1] = [1, 0, 0, 0]
    p[0, 2] = [0.25, 0.5, 0.375, 0.25]   # codes [0,1,0,0]
    a = np.array([[2.0, 3.0, 0.5]], np.float32)
    bits = np.array([[2, 0, 1]], np.uint8)
    blob = fmt.pack(p, a, bits)
    H = fmt.read_header(blob)
    assert H["magic"] == b"BMOE" and H["version"] == 4
    assert H["dout_pad"] == 32 and H["n_seg"] == 1
    base, n_nz, n_q, n_16, seg_words = struct.unpack_from("<QIIII", blob, 128)
    # each used group padded to 32 slots = 8 blocks: 4 * 8 * (1 + 2) words
    assert (n_nz, n_q, n_16, seg_words) == (2, 2, 0, 96)
    # the component table sits at align256(128 + 64) = 256: slots column 0
    # -> 32 (the width-2 group starts after the 32 slots of the width-1
    # group), column 1 dropped, column 2 -> slot 0; then s, m (16 bytes
    # each) and a (16 bytes) in component order, then cmax
    assert H["ctab_offset"] == 256
    assert struct.unpack_from("<3H", blob, 256) == (32, 0xFFFF, 0)
    assert blob[256 + 6:256 + 16] == bytes(10)
    assert struct.unpack_from("<3e", blob, 256 + 16) == (0.333251953125, 0.0, 0.25)
    assert struct.unpack_from("<3e", blob, 256 + 32) == (-0.5, 0.0, 0.25)
    assert struct.unpack_from("<3f", blob, 256 + 48) == (2.0, 0.0, 0.5)
    assert struct.unpack_from("<f", blob, 256 + 64)[0] == np.float32(2.0) * np.float32(0.333251953125)
    assert base == 512  # align256(256 + 3 * 16 + 16 + 16)
    cnt = struct.unpack_from("<7H", blob, 128 + 48)
    assert cnt == (1, 1, 0, 0, 0, 0, 0)
    # width group 1 first (column 2 + 31 padding slots), then width 2 (column 0)
    kidx = struct.unpack_from("<64H", blob, base)
    assert kidx[0] == 2 and kidx[32] == 0 and not any(kidx[1:32]) and not any(kidx[33:])
    a_off, s_off, m_off, p_off = struct.unpack_from("<IIII", blob, 128 + 24)
    a_s = struct.unpack_from("<64f", blob, base + a_off)
    assert (a_s[0], a_s[32]) == (0.5, 2.0) and sum(map(abs, a_s)) == 2.5
    # s of column 0 is fp16(1/3) = 0.333251953125; of column 2, 0.25
    s = struct.unpack_from("<64e", blob, base + s_off)
    assert (s[0], s[32]) == (0.25, 0.333251953125) and sum(s) == 0.25 + 0.333251953125
    cmax, = struct.unpack_from("<f", blob, 128 + 40)
    assert cmax == np.float32(2.0) * np.float32(0.333251953125)
    words = struct.unpack_from("<96I", blob, base + p_off)
    # group 1 (width 1), block 0, octet 0: slot 0 (column 2, u = 0) has
    #   code 1 in row 1 -> bit 8*0 + 1; octets 1-3 are rows 8..31 (padding)
    #   -> 0; blocks 1-7 of the group are padding (4 words each)
    # group 2 (width 2) starts at word 4 * 8 * 1 = 32; its block 0, octet 0:
    #   slot 32 (column 0, u = 0) codes [0,1,2,3] in rows 0..3
    #   plane 0: rows 1, 3 -> bits 1, 3; plane 1: rows 2, 3 -> bits 2, 3
    expect = [0] * 96
    expect[0] = 0x2
    expect[32], expect[33] = 0xA, 0xC
    assert words == tuple(expect)


def test_hand_built_fp16_block():
    # one 16-bit column among 5: its block holds row-major fp16 pairs
    dout = 40
    p = np.zeros((1, 5, dout), np.float32)
    for k in range(5):
        p[0, k, :] = (np.arange(dout) + 100 * k) / 1024.0   # exact in fp16
    a = np.ones((1, 5), np.float32)
    bits = np.array([[0, 16, 16, 0, 16]], np.uint8)
    blob = fmt.pack(p, a, bits)
    H = fmt.read_header(blob)
    assert (H["dout_pad"], H["n_seg"]) == (64, 2)
    base, n_nz, n_q, n_16, seg_words = struct.unpack_from("<QIIII", blob, 128)
    assert (n_nz, n_q, n_16, seg_words) == (3, 0, 3, 4 * 8 * 16)
    p_off, = struct.unpack_from("<I", blob, 128 + 36)
    W = np.frombuffer(blob, "<u4", count=2 * 512, offset=base + p_off).reshape(2, 512)
    f16 = lambda v: int(np.float16(v).view(np.uint16))
    # segment 1, octet 0, rho 2 = row 34; word 2*rho + h, h = 1 -> slots 2, 3
    # slot 2 is column 4, slot 3 is padding
    assert W[1, 0 * 16 + 2 * 2 + 1] == f16((34 + 400) / 1024.0)
    # h = 0 -> slots 0 (column 1) and 1 (column 2)
    assert W[1, 2 * 2] == f16((34 + 100) / 1024.0) | (f16((34 + 200) / 1024.0) << 16)
    # rows >= dout (segment 1, octet 1, rows 40..47) are 0
    assert np.all(W[1, 16:32] == 0)


def _random_layer(E, r, dout, bits, seed):
    g = np.random.default_rng(seed).standard_normal((E, r, dout))
    p = (g / np.linalg.norm(g, axis=2, keepdims=True)).astype(np.float32)
    a = np.random.default_rng(seed + 1).lognormal(0, 0.3, (E, r)).astype(np.float32)
    return p, a, bits.astype(np.uint8)


@pytest.mark.parametrize("dout", [96, 64, 130, 33])
def test_round_trip_all_widths(dout):
    E, r = 4, 24
    rng = np.random.default_rng(dout)
    bits = rng.choice([0, 1, 2, 3, 4, 6, 8, 16], size=(E, r))
    bits[1] = 0          # all-0 expert
    bits[2] = 16         # all-16 expert
    bits[3, :] = rng.choice([1, 2, 8], size=r)   # empty groups 3, 4, 6, 16
    p, a, bits = _random_layer(E, r, dout, bits, dout)
    blob = fmt.pack(p, a, bits)
    out = fmt.unpack(blob)
    assert np.array_equal(out["bits"], bits)
    for e in range(E):
        qe = quantize_expert(p[e], bits[e])
        nz = bits[e] > 0
        assert np.array_equal(out["q"][e][nz], qe["q"][nz])
        qm = (bits[e] > 0) & (bits[e] <= 8)
        assert np.array_equal(out["s"][e][qm], qe["s"][qm])
        assert np.array_equal(out["m"][e][qm], qe["m"][qm])
        assert np.array_equal(out["a"][e][nz], a[e][nz])
        assert np.all(out["a"][e][~nz] == 0)


def test_unpack_subset_of_experts():
    """unpack(blob, experts) gives the same rows as the full unpack, in the
    order asked for, and refuses ids outside [0, E)."""
    E, r, dout = 4, 24, 70
    rng = np.random.default_rng(7)
    bits = rng.choice([0, 1, 2, 3, 4, 6, 8, 16], size=(E, r))
    p, a, bits = _random_layer(E, r, dout, bits, 7)
    blob = fmt.pack(p, a, bits)
    full = fmt.unpack(blob)
    sub = fmt.unpack(blob, experts=[2, 0])
    for key in ("q", "s", "m", "a", "bits", "cmax"):
        assert np.array_equal(sub[key], full[key][[2, 0]]), key
    with pytest.raises(ValueError):
        fmt.unpack(blob, experts=[4])


def test_header_alignment_and_crc():
    p, a, bits = _random_layer(3, 16, 96, np.random.default_rng(5).choice(
        [0, 1, 2, 3, 4, 6, 8, 16], size=(3, 16)), 5)
    blob = fmt.pack(p, a, bits)
    H = fmt.read_header(blob)
    assert H["total_bytes"] == len(blob) and H["total_bytes"] % 256 == 0
    assert H["crc32"] == zlib.crc32(blob[128:]) & 0xFFFFFFFF
    for e in range(3):
        base, = struct.unpack_from("<Q", blob, 128 + 64 * e)
        assert base % 256 == 0
        offs = struct.unpack_from("<4I", blob, 128 + 64 * e + 24)
        nbytes, = struct.unpack_from("<I", blob, 128 + 64 * e + 44)
        assert offs[3] % 256 == 0 and nbytes % 256 == 0
    bad = bytearray(blob)
    bad[-300] ^= 1
    with pytest.raises(ValueError):
        fmt.unpack(bytes(bad))


def test_zero_width_column_is_invisible():
    """Changing a and p of a 0-bit column does not change a single byte."""
    E, r, dout = 2, 12, 96
    bits = np.random.default_rng(2).choice([0, 1, 2, 3, 16], size=(E, r))
    bits[0, 5] = 0
    p, a, bits = _random_layer(E, r, dout, bits, 11)
    b1 = fmt.pack(p, a, bits)
    p2, a2 = p.copy(), a.copy()
    p2[0, 5] = -p2[0, 5]
    a2[0, 5] = 123.0
    assert fmt.pack(p2, a2, bits) == b1
