"""Pins of the plain C oracle (oracle/ref_decode.c) on the CPU.

* codes read back from the planes equal the Python oracle unpacker's
  (oracle/fmt.py) bit for bit: every expert and width of the tiny layer and
  of a ragged-dout layer with every width;
* h equals the float64 numpy oracle (oracle/path.py with the quantizer's own
  p_hat) to 1e-12 of max |h| per (token, slot): both take the same float64
  steps in k order; only z's sum over din is ordered differently (BLAS);
* the result does not depend on the thread count (bit for bit);
* an id outside [0, E) and a blob whose header disagrees give NaN rows.
"""
import numpy as np
import pytest

import synth
from oracle import fmt, path, ref_c
from oracle.quantize import quantize_expert


@pytest.fixture(scope="module", autouse=True)
def _built():
    import os
    if not os.path.exists(ref_c.LIB_PATH):
        from oracle import build_ref
        build_ref.build()


def _ragged_layer(seed=3, E=3, r=64, dout=100):
    rng = np.random.default_rng(seed)
    p = rng.standard_normal((E, r, dout)).astype(np.float32)
    p /= np.linalg.norm(p, axis=2, keepdims=True)
    a = rng.lognormal(0, 0.5, (E, r)).astype(np.float32)
    bits = rng.choice([0, 1, 2, 3, 4, 6, 8, 16], size=(E, r)).astype(np.uint8)
    return p.astype(np.float32), a, bits


def test_unpack_matches_oracle_unpacker():
    L = synth.make_layer(synth.LAYERS["tiny"])
    cases = [(L.p["gate"], L.a["gate"], L.bits["gate"]), _ragged_layer()]
    for p, a, bits in cases:
        E, r, dout = p.shape
        blob = np.frombuffer(fmt.pack(p, a, bits), np.uint8)
        ref = fmt.unpack(blob.tobytes())
        assert set(np.unique(bits).tolist()) >= {1, 2, 3, 4, 6, 8, 16}
        for e in range(E):
            got = ref_c.unpack_expert(blob, E, dout, r, e)
            assert np.array_equal(got, ref["q"][e]), e


def _numpy_h(L, x, ids):
    zg = path.spectral_proj(np.asarray(L.phi["gate"], np.float16), x)
    zu = path.spectral_proj(np.asarray(L.phi["up"], np.float16), x)
    T, K = ids.shape
    h = np.zeros((T, K, L.spec.dout))
    for t in range(T):
        for s in range(K):
            e = ids[t, s]
            y = {}
            for proj, z in (("gate", zg), ("up", zu)):
                ph = quantize_expert(L.p[proj][e], L.bits[proj][e])["phat"]
                y[proj] = path.expert_apply(z[t], L.a[proj][e], ph, L.bits[proj][e])[0]
            h[t, s] = path.silu(y["gate"]) * y["up"]
    return h


def _inputs(L, wl_name, step=0):
    wl = synth.workload(wl_name)
    x, ids = synth.make_batch(wl, L, step=step)
    blobs = [np.frombuffer(fmt.pack(L.p[p], L.a[p], L.bits[p]), np.uint8) for p in ("gate", "up")]
    phi_t = np.concatenate([np.asarray(L.phi["gate"], np.float16).T,
                            np.asarray(L.phi["up"], np.float16).T], axis=0)
    return x, ids, blobs, phi_t


def test_gateup_matches_numpy_oracle():
    L = synth.make_layer(synth.LAYERS["tiny"])
    spec = L.spec
    for wl_name, step in (("tiny_t8", 0), ("tiny_t8", 1), ("tiny_t1", 0)):
        x, ids, (bg, bu), phi_t = _inputs(L, wl_name, step)
        got = ref_c.gateup(bg, bu, phi_t, x, ids, spec.E, spec.dout, spec.r, threads=1)
        ref = _numpy_h(L, x, ids)
        scale = np.abs(ref).max(axis=2, keepdims=True)
        assert np.all(np.abs(got - ref) <= 1e-12 * scale), np.max(np.abs(got - ref) / scale)


def test_gateup_thread_count_and_bad_inputs():
    L = synth.make_layer(synth.LAYERS["tiny"])
    spec = L.spec
    x, ids, (bg, bu), phi_t = _inputs(L, "tiny_t8")
    h1 = ref_c.gateup(bg, bu, phi_t, x, ids, spec.E, spec.dout, spec.r, threads=1)
    h4 = ref_c.gateup(bg, bu, phi_t, x, ids, spec.E, spec.dout, spec.r, threads=4)
    assert np.array_equal(h1, h4)
    bad = ids.copy()
    bad[2, 1] = spec.E
    bad[3, 0] = -1
    hb = ref_c.gateup(bg, bu, phi_t, x, bad, spec.E, spec.dout, spec.r, threads=2)
    assert np.all(np.isnan(hb[2, 1])) and np.all(np.isnan(hb[3, 0]))
    keep = np.ones(ids.shape, bool)
    keep[2, 1] = keep[3, 0] = False
    assert np.array_equal(hb[keep], h1[keep])
    # the blobs describe E experts; a call that claims E + 1 is refused row by row
    hm = ref_c.gateup(bg, bu, phi_t, x, ids, spec.E + 1, spec.dout, spec.r, threads=1)
    assert np.all(np.isnan(hm))
