"""GPU check of the allocation-free gate/up entry point (bitsmoe_moe_gateup_noalloc,
through the C ABI) against bitsmoe_moe_gateup with a caller-owned workspace.

Both run the same kernels on the same inputs; the bar is the gate/up parity
bar, max |dh| <= 2e-3 * max |h| per (token, slot).  Calls come in a row on one
stream with sizes going down and up again (T = 32: batched path; T = 1 and
T = 4: one-launch path), so each call finds the static workspace as the last
one left it.
"""
import sys

import numpy as np
import pytest

import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

H_TOL = 2e-3


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def qwen():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from spectral_expert_gemv_amd import DeviceLayer, bitsmoe
    _say("building layer qwen3_30b_a3b")
    L = synth.make_layer(synth.LAYERS["qwen3_30b_a3b"])
    return bitsmoe, L, DeviceLayer.from_synth(L)


def _cuda(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _noalloc(bm, dev, x, ids):
    T, k = ids.shape
    h = torch.full((T, k, dev.dout), float("nan"), dtype=torch.float32, device="cuda")
    bm.moe_gateup_noalloc(dev.blob_gate, dev.blob_up, dev.phi_t, x, ids, dev.E, dev.dout, dev.r,
                          h)
    return h


def test_noalloc_matches_workspace_entry_point(qwen):
    bm, L, dev = qwen
    for call, wl_name in enumerate(["qwen3_30b_a3b_t32", "qwen3_30b_a3b_t1",
                                    "qwen3_30b_a3b_t4", "qwen3_30b_a3b_t1"]):
        wl = synth.workload(wl_name)
        x, ids = synth.make_batch(wl, L, step=300 + call)
        xd, idd = _cuda(x), _cuda(ids)
        T, k = ids.shape
        need = bm.moe_gateup_workspace_size(T, k, dev.E, dev.din, dev.dout, dev.r)
        assert need <= bm.GATEUP_NOALLOC_MAX_WS
        _say("noalloc call %d: %s (T=%d, workspace %d bytes)" % (call, wl_name, T, need))
        got = _noalloc(bm, dev, xd, idd)
        torch.cuda.synchronize()
        ref = dev.gateup(xd, idd)
        torch.cuda.synchronize()
        got, ref = got.cpu().numpy(), ref.cpu().numpy()
        assert np.all(np.isfinite(got)), call
        scale = np.max(np.abs(ref), axis=2)
        err = np.max(np.abs(got - ref), axis=2)
        assert np.all(err <= H_TOL * scale), (call, float(np.max(err / np.maximum(scale, 1e-30))))


def test_noalloc_refuses_oversized_call(qwen):
    bm, L, dev = qwen
    T, k = 256, L.spec.k
    assert bm.moe_gateup_workspace_size(T, k, dev.E, dev.din, dev.dout, dev.r) > \
        bm.GATEUP_NOALLOC_MAX_WS
    x = torch.zeros((T, dev.din), dtype=torch.float16, device="cuda")
    ids = torch.zeros((T, k), dtype=torch.int32, device="cuda")
    h = torch.full((T, k, dev.dout), 7.0, dtype=torch.float32, device="cuda")
    with pytest.raises(bm.BitsMoEError) as e:
        bm.moe_gateup_noalloc(dev.blob_gate, dev.blob_up, dev.phi_t, x, ids, dev.E, dev.dout,
                              dev.r, h)
    assert e.value.status == bm.ENOSPC
    torch.cuda.synchronize()
    assert bool(torch.all(h == 7.0))  # nothing was launched
