"""CPU checks of the C-ABI library: exports, host packer, host-side validation.

No kernel is launched: the packer and blob checker are host code, and every
device entry point below is called with arguments its host checks reject
before anything is enqueued.
"""
import ctypes
import os
import re
import struct

import numpy as np
import pytest

import synth
from oracle import fmt
from spectral_expert_gemv_amd import bitsmoe as bm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_symbols():
    names = set()
    for fn in os.listdir(os.path.join(ROOT, "include")):
        if fn.endswith(".h"):
            src = open(os.path.join(ROOT, "include", fn)).read()
            src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
            names |= set(re.findall(r"\b(bitsmoe_\w+)\s*\(", src))
    return sorted(names)


def test_exports_every_declared_symbol():
    lib = ctypes.CDLL(bm.LIB_PATH)
    decl = _declared_symbols()
    assert len(decl) >= 12
    for name in decl:
        assert hasattr(lib, name), name
    assert set(decl) == set(bm.EXPORTS)
    hdr = open(os.path.join(ROOT, "include", "bitsmoe.h")).read()
    m = re.search(r"#define BITSMOE_GATEUP_NOALLOC_MAX_WS \(\(size_t\)(\d+) << (\d+)\)", hdr)
    assert m and int(m.group(1)) << int(m.group(2)) == bm.GATEUP_NOALLOC_MAX_WS


def test_strerror_and_version():
    assert bm.version() == 10000
    for st in (0, -1, -2, -3, -4, -5, -6):
        assert bm._strerror(st) and bm._strerror(st) != "unknown status"


def _layer(E, r, dout, bits, seed):
    g = np.random.default_rng(seed).standard_normal((E, r, dout))
    p = (g / np.linalg.norm(g, axis=2, keepdims=True)).astype(np.float32)
    a = np.random.default_rng(seed + 7).lognormal(0, 0.5, (E, r)).astype(np.float32)
    return p, a, np.asarray(bits, np.uint8)


@pytest.mark.parametrize("dout", [96, 64, 1, 200])
def test_library_packer_matches_oracle_packer(dout):
    E, r = 5, 33
    rng = np.random.default_rng(dout)
    bits = rng.choice([0, 1, 2, 3, 4, 6, 8, 16], size=(E, r))
    bits[1] = 0
    bits[2] = 16
    bits[3] = rng.choice([2, 6], size=r)
    p, a, bits = _layer(E, r, dout, bits, dout)
    lib_blob = bm.pack(p, a, bits)
    assert bytes(lib_blob) == fmt.pack(p, a, bits)
    assert bm.blob_check(lib_blob) == (E, dout, r)


def test_library_packer_matches_oracle_on_tiny_layer():
    L = synth.make_layer(synth.LAYERS["tiny"])
    for proj in ("gate", "up"):
        assert bytes(bm.pack(L.p[proj], L.a[proj], L.bits[proj])) == \
            fmt.pack(L.p[proj], L.a[proj], L.bits[proj])


def test_library_packer_rounding_edge_values():
    # columns engineered to hit ties, zero ranges, fp16 subnormal scales and
    # offsets that round above the minimum
    cols = [
        [0.25, 0.5, 0.375, 0.25], [0.0, 0.375, 0.75, 0.0], [0.1, 0.1, 0.1, 0.1],
        [0.7, 0.8, 0.75, 0.7], [1e-6, 2e-6, 3e-6, 1.5e-6], [-1e-7, 1e-7, 0, 0],
        [-0.5, -0.1, 0.2, 0.5], [6e-5, 6.1e-5, 6.2e-5, 6.3e-5],
        [0.0, -0.0, 0.5, 0.25], [-0.0, 0.0, 0.5, 0.25], [-0.0, -0.0, -0.0, -0.0],
        [30000.0, -30000.0, 1.0, 0.0],
    ]
    p = np.array(cols, np.float32)[None]
    for b in (1, 2, 3, 4, 6, 8, 16):
        bits = np.full((1, len(cols)), b, np.uint8)
        a = np.ones((1, len(cols)), np.float32)
        assert bytes(bm.pack(p, a, bits)) == fmt.pack(p, a, bits), b


def test_packer_status_codes():
    p, a, bits = _layer(2, 4, 8, np.full((2, 4), 2), 0)
    bad = bits.copy()
    bad[1, 2] = 5
    with pytest.raises(bm.BitsMoEError) as ei:
        bm.pack(p, a, bad)
    assert ei.value.status == bm.EBITS
    n = bm.pack_size(2, 8, 4, bits)
    out = np.zeros(n - 1, np.uint8)
    st = bm._lib.bitsmoe_pack(2, 8, 4, p.ctypes.data, a.ctypes.data, bits.ctypes.data,
                              out.ctypes.data, out.nbytes)
    assert st == bm.ENOSPC
    pn = p.copy()
    pn[0, 1, 3] = np.nan
    with pytest.raises(bm.BitsMoEError) as ei:
        bm.pack(pn, a, bits)
    assert ei.value.status == bm.EBITS
    with pytest.raises(bm.BitsMoEError) as ei:
        bm.pack_size(2, 8, 70000, np.zeros((2, 70000), np.uint8))
    assert ei.value.status == bm.ESHAPE
    assert bm._lib.bitsmoe_pack_size(0, 8, 4, bits.ctypes.data, None) == bm.EINVAL


def test_blob_check_rejects_corruption():
    p, a, bits = _layer(3, 16, 96, np.random.default_rng(1).choice(
        [0, 1, 2, 3, 4, 6, 8, 16], size=(3, 16)), 1)
    blob = bm.pack(p, a, bits)
    assert bm.blob_check(blob) == (3, 96, 16)
    for mutate in (lambda b: b.__setitem__(0, 0),                 # magic
                   lambda b: b.__setitem__(4, 1),                 # version
                   lambda b: b.__setitem__(len(b) - 300, b[len(b) - 300] ^ 1)):  # CRC
        bb = blob.copy()
        mutate(bb)
        with pytest.raises(bm.BitsMoEError) as ei:
            bm.blob_check(bb)
        assert ei.value.status == bm.EFORMAT
    # a directory edit with the CRC recomputed is still caught
    import zlib
    bb = bytearray(blob.tobytes())
    struct.pack_into("<I", bb, 128 + 8, struct.unpack_from("<I", bb, 128 + 8)[0] + 1)
    struct.pack_into("<I", bb, 48, zlib.crc32(bytes(bb[128:])) & 0xFFFFFFFF)
    with pytest.raises(bm.BitsMoEError) as ei:
        bm.blob_check(np.frombuffer(bytes(bb), np.uint8))
    assert ei.value.status == bm.EFORMAT
    with pytest.raises(bm.BitsMoEError) as ei:
        bm.blob_check(blob[:-256])
    assert ei.value.status == bm.EFORMAT


FAKE = 1 << 20   # a 16-byte aligned address; never dereferenced (checks fail first)


def test_device_entry_points_validate_before_launch():
    L = bm._lib
    # spectral projection
    assert L.bitsmoe_spectral_proj(None, FAKE, FAKE, 1, 64, 64, None) == bm.EINVAL
    assert L.bitsmoe_spectral_proj(FAKE + 2, FAKE, FAKE, 1, 64, 64, None) == bm.EINVAL
    assert L.bitsmoe_spectral_proj(FAKE, FAKE, FAKE, 0, 64, 64, None) == bm.EINVAL
    assert L.bitsmoe_spectral_proj(FAKE, FAKE, FAKE, 1, 60, 64, None) == bm.ESHAPE
    assert L.bitsmoe_spectral_proj(FAKE, FAKE, FAKE, 1, 64, 0, None) == bm.ESHAPE
    # expert apply
    args = dict(E=4, dout=96, r=64)
    def ea(packed=FAKE, nbytes=1 << 16, E=4, dout=96, r=64, z=FAKE, zs=64, ids=FAKE, T=1, k=2,
           y=FAKE):
        return L.bitsmoe_expert_apply(packed, nbytes, E, dout, r, z, zs, ids, T, k, y, None, 0,
                                      None)
    assert ea(packed=None) == bm.EINVAL
    assert ea(nbytes=100) == bm.ENOSPC
    assert ea(E=0) == bm.ESHAPE
    assert ea(r=70000, zs=70000) == bm.ESHAPE
    assert ea(k=5) == bm.EINVAL
    assert ea(zs=10) == bm.ESHAPE
    assert ea(ids=FAKE + 2) == bm.EINVAL
    assert ea(y=FAKE + 4) == bm.EINVAL
    # gate/up
    ws_need = bm.moe_gateup_workspace_size(8, 2, 4, 64, 96, 64)
    assert ws_need >= 8 * 2 * 64 * 4
    def gu(ws_bytes=ws_need, din=64, T=8, k=2, h=FAKE, ws=FAKE):
        return L.bitsmoe_moe_gateup(FAKE, 1 << 16, FAKE, 1 << 16, FAKE, FAKE, FAKE, T, k, 4,
                                    din, 96, 64, h, ws, ws_bytes, None)
    assert gu(ws_bytes=ws_need - 1) == bm.ENOSPC
    assert gu(din=60) == bm.ESHAPE
    assert gu(T=0) == bm.EINVAL
    assert gu(k=0) == bm.EINVAL
    assert gu(h=None) == bm.EINVAL
    assert gu(ws=FAKE + 8) == bm.EINVAL
    # gate/up on the static workspace: the same checks, and a call needing
    # more workspace than the static array holds is refused before any HIP call
    def gun(T=8, k=2, E=4, din=64, dout=96, r=64, h=FAKE):
        return L.bitsmoe_moe_gateup_noalloc(FAKE, 1 << 26, FAKE, 1 << 26, FAKE, FAKE, FAKE, T, k,
                                            E, din, dout, r, h, None)
    assert bm.moe_gateup_workspace_size(256, 8, 128, 2048, 768, 2048) > bm.GATEUP_NOALLOC_MAX_WS
    assert gun(T=256, k=8, E=128, din=2048, dout=768, r=2048) == bm.ENOSPC
    assert b"static" in bm._lib.bitsmoe_last_error_detail()
    assert gun(T=0) == bm.EINVAL
    assert gun(k=5) == bm.EINVAL
    assert gun(din=60) == bm.ESHAPE
    assert gun(h=None) == bm.EINVAL
    assert gun(h=FAKE + 4) == bm.EINVAL
    # code dump
    assert L.bitsmoe_dump_codes(FAKE, 1 << 16, 4, 96, 64, 4, 0, FAKE, None) == bm.EINVAL
    assert L.bitsmoe_dump_codes(FAKE, 1 << 16, 4, 96, 64, 0, 0, None, None) == bm.EINVAL
    assert L.bitsmoe_dump_codes(FAKE, 1 << 16, 4, 96, 64, 0, 3, FAKE, None) == bm.EINVAL
    assert L.bitsmoe_dump_codes(FAKE, 1 << 16, 4, 96, 64, 0, -1, FAKE, None) == bm.EINVAL
    assert L.bitsmoe_workspace_init(None, 16, None) == bm.EINVAL
    n = ctypes.c_uint32(7)
    assert L.bitsmoe_wait_timeouts(FAKE, 1 << 20, None, None) == bm.EINVAL
    assert L.bitsmoe_wait_timeouts(FAKE, 64, ctypes.byref(n), None) == bm.EINVAL
    assert n.value == 7
    assert bm._lib.bitsmoe_last_error_detail()


def test_device_packer_validates_before_launch():
    L = bm._lib
    E, dout, r = 2, 40, 8
    bits = np.full((E, r), 3, np.uint8)
    need = bm.pack_size(E, dout, r, bits)
    ws_need = bm.pack_device_workspace_size(E, dout, r, bits)
    assert ws_need >= 16 + 4 * (E + 1) + 4 * 2 * 32

    def pk(E=E, p=FAKE, a=FAKE, bits=bits, out=FAKE, out_bytes=need, ws=FAKE, ws_bytes=ws_need):
        return L.bitsmoe_pack_device(E, dout, r, p, a, bits.ctypes.data, out, out_bytes, ws,
                                     ws_bytes, None)
    assert pk(p=None) == bm.EINVAL
    assert pk(ws=None) == bm.EINVAL
    assert pk(out=FAKE + 8) == bm.EINVAL
    assert pk(a=FAKE + 2) == bm.EINVAL
    assert pk(out_bytes=need - 1) == bm.ENOSPC
    assert pk(ws_bytes=ws_need - 1) == bm.ENOSPC
    bad = bits.copy()
    bad[1, 3] = 7
    assert pk(bits=bad) == bm.EBITS
    assert pk(E=70000) == bm.ESHAPE
    assert L.bitsmoe_pack_device_workspace_size(E, dout, r, bits.ctypes.data, None) == bm.EINVAL


def test_fqcm_entry_points_validate_before_launch():
    L = bm._lib
    assert L.bitsmoe_fqcm_distortion(None, 2, 3, 4, FAKE, None) == bm.EINVAL
    assert L.bitsmoe_fqcm_distortion(FAKE, 0, 3, 4, FAKE, None) == bm.ESHAPE
    assert L.bitsmoe_fqcm_distortion(FAKE, 2, 3, 4, FAKE + 4, None) == bm.EINVAL
    assert L.bitsmoe_fqcm_beta(FAKE, 7, FAKE, FAKE, 4, 2, 3, 8, FAKE, None) == bm.ESHAPE
    assert L.bitsmoe_fqcm_beta(FAKE, 8, FAKE, FAKE, 0, 2, 3, 8, FAKE, None) == bm.EINVAL
    assert L.bitsmoe_fqcm_beta(None, 8, FAKE, FAKE, 4, 2, 3, 8, FAKE, None) == bm.EINVAL
    lam = ctypes.c_double()
    used = ctypes.c_uint64()
    def al(ws_bytes=bm.FQCM_WS_BYTES, ws=FAKE, bits=FAKE, E=2):
        return L.bitsmoe_fqcm_allocate(FAKE, FAKE, FAKE, E, 3, 4, 100, bits, ctypes.byref(lam),
                                       ctypes.byref(used), None, ws, ws_bytes, None)
    hdr = open(os.path.join(ROOT, "include", "bitsmoe.h")).read()
    m = re.search(r"#define BITSMOE_FQCM_WS_BYTES \(\(size_t\)(\d+) \+ (\d+) \* (\d+)\)", hdr)
    assert m and int(m.group(1)) + int(m.group(2)) * int(m.group(3)) == bm.FQCM_WS_BYTES
    assert al(ws_bytes=bm.FQCM_WS_BYTES - 1) == bm.ENOSPC
    assert al(ws=None) == bm.EINVAL
    assert al(bits=None) == bm.EINVAL
    assert al(E=0) == bm.ESHAPE


def test_down_entry_point_validates_before_launch():
    L = bm._lib
    need = bm.moe_down_workspace_size(2, 2, 4, 96, 64, 32)
    assert need >= 2 * 2 * (96 * 2 + 32 * 4 + 64 * 4)
    def dn(T=2, k=2, E=4, dout=96, ws=FAKE, ws_bytes=need, h=FAKE):
        return L.bitsmoe_moe_down(FAKE, 1 << 16, FAKE, h, FAKE, FAKE, T, k, E, dout, 64, 32,
                                  FAKE, ws, ws_bytes, None)
    assert dn(ws_bytes=need - 1) == bm.ENOSPC
    assert dn(dout=90) == bm.ESHAPE
    assert dn(T=0) == bm.EINVAL
    assert dn(k=5) == bm.EINVAL
    assert dn(ws=FAKE + 16) == bm.EINVAL
    assert dn(h=None) == bm.EINVAL


def test_ssd_entry_point_validates_before_launch():
    L = bm._lib
    need = bm.ssd_workspace_size(4, 10, 12, 12)
    assert need >= 2 * 12 * 12 * 8 + 4 * 10 * 12 * 8
    def sd(E=4, dout=10, din=12, r=12, ws=FAKE, ws_bytes=need, W=FAKE, sweeps=30):
        return L.bitsmoe_ssd(W, E, dout, din, r, FAKE, FAKE, FAKE, None, None, sweeps, ws,
                             ws_bytes, None)
    assert sd(ws_bytes=need - 1) == bm.ENOSPC
    assert sd(r=13) == bm.ESHAPE
    assert sd(din=9000, r=12) == bm.ESHAPE
    assert sd(W=None) == bm.EINVAL
    assert sd(ws=FAKE + 64) == bm.EINVAL
    assert sd(sweeps=0) == bm.EINVAL
