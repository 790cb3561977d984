"""GPU parity of the down projection + routing-weighted combine
(bitsmoe_moe_down) against the float64 oracle (oracle.path.moe_down).

Bar: max |d out| <= 5e-4 * max |out_oracle| per token (the per-pair
products accumulate in float32 over up to r_d terms of both signs, as the
expert apply; the combine adds k float32 terms; the fp16 rounding of h and
of Phi_down is the same on both sides).
"""
import sys

import numpy as np
import pytest

import synth
from oracle import path
from oracle.quantize import quantize_expert

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TOL = 5e-4


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="session")
def bm():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from spectral_expert_gemv_amd import bitsmoe
    return bitsmoe


def _cuda(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


_DOWN = {}


def _down(bm, name):
    if name not in _DOWN:
        L = synth.make_layer(synth.LAYERS[name])
        D = synth.make_down(L)
        phi16 = np.asarray(D.phi, np.float16)
        blob = _cuda(bm.pack(D.p, D.a, D.bits))
        _DOWN[name] = (L, D, phi16, blob, _cuda(np.ascontiguousarray(phi16.T)))
    return _DOWN[name]


def _run(bm, name, wl_name, T, seed, ids=None):
    L, D, phi16, blob, phit = _down(bm, name)
    spec = L.spec
    wl = synth.workload(wl_name)
    _, ids0 = synth.make_batch(wl, L, step=seed, T=T)
    ids = ids0 if ids is None else ids
    g = synth.make_gates(wl, L, step=seed, T=T)
    h = (np.random.default_rng(seed).standard_normal((T, spec.k, spec.dout)) * 0.3).astype(
        np.float32)
    rd = D.phi.shape[1]
    _say("down %s T=%d" % (name, T))
    out = bm.moe_down(blob, phit, _cuda(h), _cuda(ids.astype(np.int32)), _cuda(g), spec.E,
                      spec.din, rd).cpu().numpy()
    experts = sorted(set(int(e) for e in np.asarray(ids).ravel() if 0 <= e < spec.E))
    phat = np.zeros((spec.E, rd, spec.din))
    for e in experts:
        phat[e] = quantize_expert(D.p[e], D.bits[e])["phat"]
    ref = path.moe_down(phi16, D.a, phat, D.bits, h, ids, g)
    for t in range(T):
        err = np.abs(out[t] - ref[t]).max() / max(np.abs(ref[t]).max(), 1e-30)
        assert err <= TOL, (name, t, err)
    return out, ref


def test_down_tiny(bm):
    _run(bm, "tiny", "tiny_t8", 8, 0)


def test_down_tiny_invalid_id_contributes_nothing(bm):
    L = synth.make_layer(synth.LAYERS["tiny"])
    _, ids = synth.make_batch(synth.workload("tiny_t4"), L, step=3, T=4)
    ids = ids.copy()
    ids[1, 0] = L.spec.E + 2
    ids[2, 1] = -1
    _run(bm, "tiny", "tiny_t4", 4, 3, ids=ids)


@pytest.mark.parametrize("T", [1, 8])
def test_down_qwen_full_size(bm, T):
    _run(bm, "qwen3_30b_a3b", "qwen3_30b_a3b_t1" if T == 1 else "qwen3_30b_a3b_t32", T, 10 + T)


def test_gateup_then_down_chain(bm):
    # the device gate/up output feeds the device down projection: shapes,
    # finiteness and the combine's linearity in g
    from spectral_expert_gemv_amd import DeviceLayer
    L, D, phi16, blob, phit = _down(bm, "tiny")
    spec = L.spec
    wl = synth.workload("tiny_t8")
    x, ids = synth.make_batch(wl, L, step=1)
    dev = DeviceLayer.from_synth(L)
    h = dev.gateup(_cuda(x), _cuda(ids))
    g = synth.make_gates(wl, L, step=1)
    rd = D.phi.shape[1]
    out = bm.moe_down(blob, phit, h, _cuda(ids.astype(np.int32)), _cuda(g), spec.E, spec.din, rd)
    out2 = bm.moe_down(blob, phit, h, _cuda(ids.astype(np.int32)), _cuda(2 * g), spec.E,
                       spec.din, rd)
    torch.cuda.synchronize()
    o, o2 = out.cpu().numpy(), out2.cpu().numpy()
    assert o.shape == (ids.shape[0], spec.din) and np.all(np.isfinite(o))
    assert np.allclose(o2, 2 * o, rtol=1e-6, atol=0)
