"""GPU parity of the shared-basis spectral decomposition (bitsmoe_ssd)
against the oracle (oracle.ssd: numpy's SVD of the stacked matrix, float64).

The decomposition is unique only up to the sign of each singular pair (and
a rotation inside a repeated singular value), so the comparison is on what
is unique: the squared singular values (relative 1e-10 of sigma_max^2), the
magnitudes a (float32 outputs: relative 1e-5), each phi_k and p_{e,k} up to
one common sign per k (1e-5), the reconstruction sum_k a p phi^T of W
(relative Frobenius error 1e-5, the float32 factors' own rounding),
orthonormal phi, unit p, and the sign rule (the first largest-magnitude
entry of every phi_k is positive).
"""
import sys

import numpy as np
import pytest

from oracle import ssd as ossd

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


def _run(bm, W, r):
    Wd = torch.from_numpy(np.ascontiguousarray(W, np.float32)).cuda()
    phi, a, p, s2, sweeps = bm.ssd(Wd, r)
    torch.cuda.synchronize()
    return phi.cpu().numpy(), a.cpu().numpy(), p.cpu().numpy(), s2, sweeps


def _check(bm, W, r, distinct=True):
    E, dout, din = W.shape
    _say("ssd E=%d dout=%d din=%d r=%d" % (E, dout, din, r))
    phi, a, p, s2, sweeps = _run(bm, W, r)
    W64 = np.asarray(W, np.float32).astype(np.float64)
    sv = np.linalg.svd(W64.reshape(E * dout, din), compute_uv=False)[:r]
    assert np.all(np.abs(s2 - sv ** 2) <= 1e-10 * sv[0] ** 2), np.abs(s2 - sv ** 2).max()
    assert np.allclose(phi.T.astype(np.float64) @ phi, np.eye(r), atol=1e-5)
    # sign rule
    for k in range(r):
        j = int(np.argmax(np.abs(phi[:, k])))
        assert phi[j, k] > 0
    rec = ossd.reconstruct(phi, a, p)
    if r == min(din, E * dout):
        err = np.linalg.norm(rec - W64) / np.linalg.norm(W64)
        assert err <= 1e-5, err
    if distinct:
        ophi, oa, op = ossd.ssd(W64, r)
        for k in range(r):
            sgn = np.sign(float(ophi[:, k] @ phi[:, k]))
            assert abs(abs(float(ophi[:, k] @ phi[:, k])) - 1.0) <= 1e-5, k
            assert np.allclose(phi[:, k], sgn * ophi[:, k], atol=1e-5), k
            assert np.allclose(a[:, k], oa[:, k], rtol=1e-5, atol=1e-6 * oa.max()), k
            live = oa[:, k] > 1e-6 * oa.max()
            assert np.allclose(p[live, k], sgn * op[live, k], atol=1e-4), k
    nz = a > 0
    assert np.allclose(np.linalg.norm(p, axis=2)[nz], 1.0, atol=1e-5)
    return sweeps


@pytest.mark.parametrize("shape", [(4, 10, 12), (3, 7, 13), (2, 64, 96)])
def test_ssd_matches_oracle_random(bm, shape):
    W = np.random.default_rng(sum(shape)).standard_normal(shape).astype(np.float32)
    _check(bm, W, shape[2] if shape[2] <= shape[0] * shape[1] else shape[0] * shape[1])


def test_ssd_truncated_rank(bm):
    W = np.random.default_rng(5).standard_normal((4, 32, 48)).astype(np.float32)
    _check(bm, W, 20)


def test_ssd_moderate_with_decaying_spectrum(bm):
    rng = np.random.default_rng(9)
    E, dout, din = 8, 128, 256
    U = np.linalg.qr(rng.standard_normal((E * dout, din)))[0]
    V = np.linalg.qr(rng.standard_normal((din, din)))[0]
    s = np.exp(-np.arange(din) / 40.0) + 0.01
    W = ((U * s[None, :]) @ V.T).reshape(E, dout, din).astype(np.float32)
    sweeps = _check(bm, W, din)
    assert sweeps <= 30


def test_ssd_rank_deficient(bm):
    # exact rank 5: the remaining squared singular values are ~0 and the
    # reconstruction still holds; a = 0 columns carry the unit vector e_0
    rng = np.random.default_rng(4)
    E, dout, din = 3, 8, 12
    W = (rng.standard_normal((E * dout, 5)) @ rng.standard_normal((5, din))).reshape(
        E, dout, din).astype(np.float32)
    phi, a, p, s2, _ = _run(bm, W, din)
    W64 = W.astype(np.float64)
    assert np.all(s2[5:] <= 1e-10 * s2[0])
    rec = ossd.reconstruct(phi, a, p)
    assert np.linalg.norm(rec - W64) / np.linalg.norm(W64) <= 1e-5
