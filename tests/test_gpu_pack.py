"""GPU parity of the device packer (bitsmoe_pack_device) through the C ABI.

Bar: the blob is byte-identical to the oracle packer's (oracle.fmt.pack:
quantizer, layout, planes, directory and CRC written independently from the
format's definition), header and checksum included.  At the full Qwen3 layer
size the oracle packs a sample of experts on their own and their blocks are
compared byte for byte; the whole blob is also compared with the host
packer's and its CRC verified.
"""
import sys

import numpy as np
import pytest

import synth
from oracle import fmt

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="session")
def bm():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from spectral_expert_gemv_amd import bitsmoe
    return bitsmoe


def _dev_pack(bm, p, a, bits):
    pd = torch.from_numpy(np.ascontiguousarray(p, np.float32)).cuda()
    ad = torch.from_numpy(np.ascontiguousarray(a, np.float32)).cuda()
    blob = bm.pack_device(pd, ad, bits)
    return blob.cpu().numpy()


def _layer(E, r, dout, bits, seed):
    rng = np.random.default_rng(seed)
    p = rng.standard_normal((E, r, dout)).astype(np.float32)
    p /= np.linalg.norm(p, axis=2, keepdims=True)
    a = rng.lognormal(0, 0.5, (E, r)).astype(np.float32)
    return p, a, np.asarray(bits, np.uint8)


@pytest.mark.parametrize("dout", [96, 64, 1, 200, 33])
def test_device_packer_matches_oracle(bm, dout):
    E, r = 5, 37
    rng = np.random.default_rng(dout + 100)
    bits = rng.choice([0, 1, 2, 3, 4, 6, 8, 16], size=(E, r))
    bits[1] = 0                       # an expert with no stored column
    bits[2] = 16                      # fp16 only
    bits[3] = rng.choice([2, 6], size=r)
    p, a, bits = _layer(E, r, dout, bits, dout)
    _say("device pack dout=%d" % dout)
    assert bytes(_dev_pack(bm, p, a, bits)) == fmt.pack(p, a, bits)


def test_device_packer_tiny_layer(bm):
    L = synth.make_layer(synth.LAYERS["tiny"])
    for proj in ("gate", "up"):
        _say("device pack tiny %s" % proj)
        got = _dev_pack(bm, L.p[proj], L.a[proj], L.bits[proj])
        assert bytes(got) == fmt.pack(L.p[proj], L.a[proj], L.bits[proj]), proj


def test_device_packer_rounding_edge_values(bm):
    # ties, zero ranges, signed zero minima, fp16 subnormal scales and offsets
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
        _say("device pack edge values b=%d" % b)
        assert bytes(_dev_pack(bm, p, a, bits)) == fmt.pack(p, a, bits), b


def test_device_packer_rejects_bad_values(bm):
    p, a, bits = _layer(2, 8, 40, np.full((2, 8), 3), 5)
    for what, mutate in (("nan p", lambda p, a: p.__setitem__((1, 2, 7), np.nan)),
                         ("big p", lambda p, a: p.__setitem__((0, 5, 0), 70000.0)),
                         ("inf a", lambda p, a: a.__setitem__((1, 3), np.inf))):
        pp, aa = p.copy(), a.copy()
        mutate(pp, aa)
        _say("device pack rejects %s" % what)
        with pytest.raises(bm.BitsMoEError) as ei:
            _dev_pack(bm, pp, aa, bits)
        assert ei.value.status == bm.EBITS, what
    # a non-finite value in a 0-bit column is not stored and is accepted
    b0 = bits.copy()
    b0[0, 1] = 0
    pp = p.copy()
    pp[0, 1, :] = np.nan
    assert bytes(_dev_pack(bm, pp, a, b0)) == fmt.pack(pp, a, b0)


def test_device_packer_full_size_qwen(bm):
    L = synth.make_layer(synth.LAYERS["qwen3_30b_a3b"])
    for proj in ("gate", "up"):
        _say("device pack qwen %s (full size)" % proj)
        p, a, bits = L.p[proj], L.a[proj], L.bits[proj]
        got = _dev_pack(bm, p, a, bits)
        assert bm.blob_check(got) == (bits.shape[0], p.shape[2], bits.shape[1])
        assert np.array_equal(got, bm.pack(p, a, bits)), proj
        # sampled experts packed by the oracle alone: their blocks match
        for e in (0, 77, bits.shape[0] - 1):
            ref = fmt.pack(p[e:e + 1], a[e:e + 1], bits[e:e + 1])
            d_ref, d_got = fmt.read_dir(ref, 0), fmt.read_dir(got.tobytes(), e)
            n = d_ref["block_bytes"]
            assert d_got["block_bytes"] == n
            o_ref, o_got = d_ref["block_offset"], d_got["block_offset"]
            assert got[o_got:o_got + n].tobytes() == ref[o_ref:o_ref + n], (proj, e)
            for key in ("cmax", "count", "seg_words", "n_nz"):
                assert d_got[key] == d_ref[key], (proj, e, key)
