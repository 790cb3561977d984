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
    assert H["magic"] == b"BMOE" and H["dout_pad"] == 64 and H["n_slabs"] == 1
    base, n_nz, n_q, n_16, mps = struct.unpack_from("<QIIII", blob, 128)
    assert (n_nz, n_q, n_16, mps) == (2, 2, 0, 3)
    assert base == 256  # align256(128 + 64)
    cnt = struct.unpack_from("<7H", blob, 128 + 48)
    assert cnt == (1, 1, 0, 0, 0, 0, 0)
    # width group 1 first (column 2), then width 2 (column 0)
    assert struct.unpack_from("<2H", blob, base) == (2, 0)
    a_off, s_off, m_off, p_off = struct.unpack_from("<IIII", blob, 128 + 24)
    assert struct.unpack_from("<2f", blob, base + a_off) == (0.5, 2.0)
    words = struct.unpack_from("<3Q", blob, base + p_off)
    # column 2, plane 0: codes [0,1,0,0] -> bit 1 -> 0b0010
    # column 0, plane 0: codes&1 = [0,1,0,1] -> 0b1010; plane 1: [0,0,1,1] -> 0b1100
    assert words == (0b0010, 0b1010, 0b1100)


def _random_layer(E, r, dout, bits, seed):
    g = np.random.default_rng(seed).standard_normal((E, r, dout))
    p = (g / np.linalg.norm(g, axis=2, keepdims=True)).astype(np.float32)
    a = np.random.default_rng(seed + 1).lognormal(0, 0.3, (E, r)).astype(np.float32)
    return p, a, bits.astype(np.uint8)


@pytest.mark.parametrize("dout", [96, 64, 130])
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
        offs = struct.unpack_from("<6I", blob, 128 + 64 * e + 24)
        assert offs[3] % 256 == 0 and offs[4] % 256 == 0 and offs[5] % 256 == 0
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
