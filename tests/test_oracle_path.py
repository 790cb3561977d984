"""Pins of the oracle path (oracle/path.py) and of the SSD (oracle/ssd.py)."""
import numpy as np
import pytest
from scipy.special import expit

import synth
from oracle import path, ssd
from oracle.quantize import quantize_expert


def _unit(shape, seed):
    g = np.random.default_rng(seed).standard_normal(shape)
    return (g / np.linalg.norm(g, axis=-1, keepdims=True)).astype(np.float32)


# ---- z = Phi^T x ---------------------------------------------------------

def test_identity_and_permutation_projection():
    x = np.random.default_rng(0).standard_normal((5, 32)).astype(np.float16)
    assert np.array_equal(path.spectral_proj(np.eye(32), x), x.astype(np.float64))
    perm = np.random.default_rng(1).permutation(32)
    Pm = np.eye(32)[:, perm]          # column k is e_{perm[k]}
    z = path.spectral_proj(Pm, x)
    assert np.array_equal(z, x.astype(np.float64)[:, perm])


def test_parseval_tiny_layer():
    L = synth.make_layer(synth.LAYERS["tiny"])
    x = np.random.default_rng(2).standard_normal((8, 64))
    for proj in ("gate", "up"):
        z = path.spectral_proj(L.phi[proj], x)
        assert np.allclose(np.linalg.norm(z, axis=1), np.linalg.norm(x, axis=1), rtol=1e-6)


# ---- y_e = sum_k a z p_hat ------------------------------------------------

def _expert(r=40, dout=96, din=40, seed=0, widths=(0, 1, 2, 3, 4, 6, 8, 16)):
    rng = np.random.default_rng(seed)
    p = _unit((r, dout), seed)
    a = rng.lognormal(0, 0.5, r).astype(np.float32)
    bits = rng.choice(widths, size=r).astype(np.uint8)
    phi = np.linalg.qr(rng.standard_normal((din, din)))[0][:, :r]
    return p, a, bits, phi


def test_brute_force_dense():
    p, a, bits, phi = _expert()
    qe = quantize_expert(p, bits)
    x = np.random.default_rng(9).standard_normal((3, phi.shape[0]))
    y = path.expert_apply(path.spectral_proj(phi, x), a, qe["phat"], bits)
    keep = (bits > 0).astype(np.float64)
    Wq = (qe["phat"].T * (a * keep)[None, :]) @ phi.T        # dout x din
    ref = x @ Wq.T
    assert np.allclose(y, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())


def test_one_hot_and_linearity():
    p, a, bits, phi = _expert(seed=3)
    bits[7] = 3
    qe = quantize_expert(p, bits)
    z = np.random.default_rng(4).standard_normal((2, 40))
    onehot = np.zeros_like(a)
    onehot[7] = a[7]
    y = path.expert_apply(z, onehot, qe["phat"], bits)
    assert np.array_equal(y, np.outer(a[7] * z[:, 7], qe["phat"][7]))
    z2 = np.random.default_rng(5).standard_normal((2, 40))
    y1 = path.expert_apply(z, a, qe["phat"], bits)
    y2 = path.expert_apply(z2, a, qe["phat"], bits)
    y12 = path.expert_apply(2 * z - 3 * z2, a, qe["phat"], bits)
    assert np.allclose(y12, 2 * y1 - 3 * y2, rtol=1e-12, atol=1e-12)
    ya = path.expert_apply(z, 2.5 * a.astype(np.float64), qe["phat"], bits)
    assert np.allclose(ya, 2.5 * y1, rtol=1e-13, atol=1e-13 * np.abs(y1).max())


def test_zero_bit_column_removable_bit_exact():
    p, a, bits, phi = _expert(seed=6)
    bits[[4, 11, 30]] = 0
    qe = quantize_expert(p, bits)
    z = np.random.default_rng(7).standard_normal((4, 40))
    y = path.expert_apply(z, a, qe["phat"], bits)
    keep = np.ones(40, bool)
    keep[[4, 11, 30]] = False
    y_del = path.expert_apply(z[:, keep], a[keep], qe["phat"][keep], bits[keep])
    assert np.array_equal(y, y_del)


def test_all_16_bit_reproduces_dense_product():
    """All-16-bit factors reproduce W_e x of a dense matrix given as input."""
    rng = np.random.default_rng(8)
    E, dout, din = 3, 24, 20
    W = rng.standard_normal((E, dout, din))
    phi, a, p = ssd.ssd(W)
    x = rng.standard_normal((4, din))
    z = path.spectral_proj(phi, x)
    bits = np.full(a.shape[1], 16, np.uint8)
    for e in range(E):
        qe = quantize_expert(p[e].astype(np.float32), bits)
        y = path.expert_apply(z, a[e], qe["phat"], bits)
        ref = x @ W[e].T
        # fp16 rounding of each p element: |dp| <= 2^-11 |p| (+ fp32 cast)
        bound = (2 ** -11 + 2 ** -23) * (np.abs(z * a[e][None, :]) @ np.abs(p[e])) + 1e-12
        assert np.all(np.abs(y - ref) <= bound)


# ---- SiLU and the gated product ------------------------------------------

def test_silu_identities():
    v = np.linspace(-30, 30, 1001)
    assert path.silu(np.array([0.0]))[0] == 0.0
    assert np.allclose(path.silu(v) - path.silu(-v), v, rtol=1e-14, atol=1e-12)
    assert np.allclose(path.silu(v), v * expit(v), rtol=1e-14, atol=1e-300)


def test_moe_gateup_against_dense_per_pair():
    rng = np.random.default_rng(10)
    E, din, dout, r, T, K = 5, 16, 24, 16, 6, 2
    phis, As, Ps, Bs, Wq = {}, {}, {}, {}, {}
    for proj in ("g", "u"):
        phis[proj] = np.linalg.qr(rng.standard_normal((din, din)))[0][:, :r]
        As[proj] = rng.lognormal(0, 0.4, (E, r)).astype(np.float32)
        Ps[proj] = _unit((E, r, dout), int(rng.integers(1000)))
        Bs[proj] = rng.choice([0, 1, 2, 3, 4, 6, 8, 16], size=(E, r)).astype(np.uint8)
    x = rng.standard_normal((T, din))
    ids = np.stack([rng.permutation(E)[:K] for _ in range(T)])
    ph = {k: path.dequantized_layer(Ps[k], Bs[k]) for k in ("g", "u")}
    h = path.moe_gateup(phis["g"], phis["u"], As["g"], As["u"], ph["g"], ph["u"],
                        Bs["g"], Bs["u"], x, ids)
    for t in range(T):
        for s in range(K):
            e = ids[t, s]
            W = {}
            for k in ("g", "u"):
                keep = (Bs[k][e] > 0) * As[k][e].astype(np.float64)
                W[k] = (ph[k][e].T * keep[None, :]) @ phis[k].T
            ref = (W["g"] @ x[t]) * expit(W["g"] @ x[t]) * (W["u"] @ x[t])
            assert np.allclose(h[t, s], ref, rtol=1e-11, atol=1e-12 * np.abs(ref).max())


# ---- SSD ---------------------------------------------------------------

def test_ssd_reconstruction_and_structure():
    rng = np.random.default_rng(12)
    E, dout, din = 4, 10, 12
    W = rng.standard_normal((E, dout, din))
    phi, a, p = ssd.ssd(W)
    assert np.allclose(phi.T @ phi, np.eye(phi.shape[1]), atol=1e-12)
    assert np.allclose(np.linalg.norm(p, axis=2), 1.0, atol=1e-12)
    assert np.allclose(ssd.reconstruct(phi, a, p), W, atol=1e-11)
    # the energy of spectral component k summed over experts is sigma_k^2
    sv = np.linalg.svd(W.reshape(E * dout, din), compute_uv=False)
    assert np.allclose(np.sqrt((a ** 2).sum(axis=0)), sv, rtol=1e-12)
    # fp32 factors: reconstruction within 1e-5 relative
    W32 = ssd.reconstruct(phi.astype(np.float32), a.astype(np.float32), p.astype(np.float32))
    assert np.linalg.norm(W32 - W) / np.linalg.norm(W) <= 1e-5


def test_reconstruct_tiny_layer_matches_matrix_product():
    L = synth.make_layer(synth.LAYERS["tiny"])
    for proj in ("gate", "up"):
        W = ssd.reconstruct(L.phi[proj], L.a[proj], L.p[proj])
        for e in range(L.spec.E):
            ref = (L.p[proj][e].astype(np.float64).T * L.a[proj][e].astype(np.float64)[None, :]) \
                @ L.phi[proj].astype(np.float64).T
            assert np.linalg.norm(W[e] - ref) / np.linalg.norm(ref) <= 1e-12


# ---- down projection and combine ------------------------------------------

def _down_case(seed=3, E=4, dout=40, din=24, rd=16, T=3, K=2):
    rng = np.random.default_rng(seed)
    phi = np.linalg.qr(rng.standard_normal((dout, dout)))[0][:, :rd]
    a = rng.lognormal(0, 0.5, (E, rd)).astype(np.float32)
    p = _unit((E, rd, din), seed + 1)
    bits = rng.choice([0, 1, 2, 3, 4, 6, 8, 16], size=(E, rd)).astype(np.uint8)
    phat = np.stack([quantize_expert(p[e], bits[e])["phat"] for e in range(E)])
    h = rng.standard_normal((T, K, dout)).astype(np.float32)   # not fp16-exact
    ids = np.stack([rng.choice(E, K, replace=False) for _ in range(T)])
    g = rng.random((T, K)).astype(np.float32)
    return phi, a, phat, bits, h, ids, g


def test_moe_down_against_dense_expert_matrices():
    phi, a, phat, bits, h, ids, g = _down_case()
    E = phat.shape[0]
    # W_e = sum_k a_k p_hat_k phi_k^T (din x dout), built densely
    Wd = np.zeros((E, phat.shape[2], phi.shape[0]))
    for e in range(E):
        for k in range(phi.shape[1]):
            if bits[e, k]:
                Wd[e] += np.float64(a[e, k]) * np.outer(phat[e, k], phi[:, k])
    h16 = h.astype(np.float16).astype(np.float64)
    ref = np.zeros((h.shape[0], phat.shape[2]))
    for t in range(h.shape[0]):
        for j in range(h.shape[1]):
            ref[t] += np.float64(g[t, j]) * (Wd[ids[t, j]] @ h16[t, j])
    out = path.moe_down(phi, a, phat, bits, h, ids, g)
    assert np.allclose(out, ref, rtol=1e-11, atol=1e-13 * np.abs(ref).max())


def test_moe_down_one_hot_gates_and_linearity():
    phi, a, phat, bits, h, ids, g = _down_case(seed=8)
    T, K = ids.shape
    one = np.zeros_like(g)
    one[:, 1] = 1.0
    out1 = path.moe_down(phi, a, phat, bits, h, ids, one)
    for t in range(T):
        z = path.spectral_proj(phi, h[t, 1].astype(np.float16))
        y = path.expert_apply(z, a[ids[t, 1]], phat[ids[t, 1]], bits[ids[t, 1]])[0]
        assert np.array_equal(out1[t], y)
    both = path.moe_down(phi, a, phat, bits, h, ids, g)
    sep = sum(path.moe_down(phi, a, phat, bits, h, ids, np.where(
        np.arange(K)[None, :] == j, g, 0).astype(np.float32)) for j in range(K))
    assert np.allclose(both, sep, rtol=1e-13, atol=0)
    bad = ids.copy()
    bad[0, 0] = phat.shape[0] + 5          # an id outside [0, E) contributes nothing
    only = np.where(np.arange(K)[None, :] == 0, 0, g).astype(np.float32)
    assert np.array_equal(path.moe_down(phi, a, phat, bits, h, bad, g)[0],
                          path.moe_down(phi, a, phat, bits, h, ids, only)[0])
