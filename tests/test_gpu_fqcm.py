"""GPU parity of the FQCM entry points (distortion, beta, allocation)
against the float64 oracle (oracle/fqcm.py), through the C ABI.

Bars:
* eps: the per-element terms are formed identically (the same float32 codes,
  the same float64 operations); only the order of the float64 sums differs:
  |d eps| <= 1e-12 * eps(0) per column.
* beta: the same float64 operations in the same pair order: bit-exact.
* allocation: the integer program's minimum (the oracle's dynamic program
  over budget units): the widths and bits used bit-exact, except that two
  allocations whose float64 losses agree to 1e-12 (sums in another order)
  may be taken either way; the Lagrangian multiplier lam bit-exact (same
  float64 expressions); lp_gap = loss - the oracle's dual bound at lam.
"""
import sys

import numpy as np
import pytest

import synth
from oracle import fqcm

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


def _cuda(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _unit(E, r, dout, seed):
    rng = np.random.default_rng(seed)
    P = rng.standard_normal((E, r, dout)).astype(np.float32)
    return (P / np.linalg.norm(P, axis=2, keepdims=True)).astype(np.float32)


def _check_eps(got, ref, p):
    e0 = np.maximum(ref[..., :1], 1e-300)
    assert np.all(np.abs(got - ref) <= 1e-12 * e0), np.abs(got - ref).max()


@pytest.mark.parametrize("dout", [1, 33, 96, 200])
def test_distortion_matches_oracle(bm, dout):
    E, r = 3, 17
    P = _unit(E, r, dout, dout)
    P[0, 0] = 0.25                                   # constant column
    P[0, 1, ::2], P[0, 1, 1::2] = 0.25, 0.75         # two levels
    P[1, 2] = np.float16(P[1, 2]).astype(np.float32) # fp16-exact
    P[2, 3, :] = -0.0                                # signed zeros
    _say("distortion dout=%d" % dout)
    got = bm.fqcm_distortion(_cuda(P)).cpu().numpy()
    ref = fqcm.distortion(P.reshape(E * r, dout)).reshape(E, r, 8)
    _check_eps(got, ref, P)


def test_distortion_full_size_sampled(bm):
    L = synth.make_layer(synth.LAYERS["qwen3_30b_a3b"])
    P = L.p["gate"]
    E, r, dout = P.shape
    _say("distortion qwen gate (full size)")
    got = bm.fqcm_distortion(_cuda(P)).cpu().numpy()
    rng = np.random.default_rng(7)
    cols = [(int(e), int(k)) for e, k in zip(rng.integers(0, E, 64), rng.integers(0, r, 64))]
    cols += [(0, 0), (E - 1, r - 1)]
    ref = fqcm.distortion(np.stack([P[e, k] for e, k in cols]))
    _check_eps(np.stack([got[e, k] for e, k in cols]), ref, None)


def test_beta_matches_oracle_bit_exact(bm):
    rng = np.random.default_rng(3)
    T, k, E, r = 13, 3, 6, 37
    z = rng.standard_normal((T, r)).astype(np.float32)
    ids = rng.integers(0, E - 1, size=(T, k)).astype(np.int32)   # expert E-1 unrouted
    ids[4, 1] = E + 3                                           # outside [0, E): skipped
    ids[5, 0] = -1
    g = rng.random((T, k)).astype(np.float32)
    _say("beta tiny")
    got = bm.fqcm_beta(_cuda(z), _cuda(ids), _cuda(g), E).cpu().numpy()
    ref = fqcm.beta(z, ids, g, E)
    assert np.array_equal(got, ref)
    assert np.all(got[E - 1] == 0)


def test_beta_full_size_bit_exact(bm):
    spec = synth.LAYERS["qwen3_30b_a3b"]
    rng = np.random.default_rng(11)
    T, k = 256, spec.k
    z = (rng.standard_normal((T, spec.r)) * 0.05).astype(np.float32)
    ids = np.stack([rng.choice(spec.E, k, replace=False) for _ in range(T)]).astype(np.int32)
    w = rng.random((T, k)).astype(np.float32)
    g = (w / w.sum(axis=1, keepdims=True)).astype(np.float32)
    _say("beta qwen size")
    got = bm.fqcm_beta(_cuda(z), _cuda(ids), _cuda(g), spec.E).cpu().numpy()
    assert np.array_equal(got, fqcm.beta(z, ids, g, spec.E))


def _alloc_inputs(E, r, seed):
    rng = np.random.default_rng(seed)
    a = rng.lognormal(0, 0.8, (E, r)).astype(np.float32)
    bet = rng.lognormal(0, 1.5, (E, r))
    bet[rng.random((E, r)) < 0.02] = 0.0
    # eps(b) of unit columns: 1 at b = 0, falling about 4x per bit, fp16 tiny
    b = np.array(fqcm.WIDTHS, np.float64)
    eps = np.exp2(-2.0 * b)[None, None, :] * rng.uniform(0.5, 1.5, (E, r, 8))
    eps[..., 0] = 1.0
    eps[..., 7] = rng.uniform(1e-9, 3e-9, (E, r))
    return a, bet, eps


def _check_alloc(bm, a, bet, eps, dout, budget, got_bits, used, gap):
    rb, rused = fqcm.allocate(a, bet, eps, dout, budget)
    loss = fqcm.total_loss(a, bet, eps, got_bits)
    rloss = fqcm.total_loss(a, bet, eps, rb)
    assert used <= budget and used == int(got_bits.astype(np.int64).sum()) * dout
    if not np.array_equal(got_bits, rb):
        # only a float64 near tie may differ
        assert abs(loss - rloss) <= 1e-12 * max(rloss, 1e-300), (loss, rloss)
    else:
        assert used == rused
    return loss


@pytest.mark.parametrize("E,r,dout", [(1, 5, 7), (3, 40, 96), (8, 256, 64)])
def test_allocation_matches_oracle(bm, E, r, dout):
    a, bet, eps = _alloc_inputs(E, r, E * r)
    full = 16 * dout * E * r
    ad, bd, ed = _cuda(a), _cuda(bet), _cuda(eps)
    for frac in (0.0, 0.01, 0.15, 0.3, 0.6, 1.0):
        budget = int(frac * full) + (dout // 3 if 0 < frac < 1 else 0)
        _say("allocate E=%d r=%d budget=%d" % (E, r, budget))
        bits, lam, used, gap = bm.fqcm_allocate(ad, bd, ed, dout, budget)
        bits = bits.cpu().numpy()
        _, rlam, _ = fqcm.lagrangian(a, bet, eps, dout, budget)
        assert lam == rlam, (lam, rlam)
        loss = _check_alloc(bm, a, bet, eps, dout, budget, bits, used, gap)
        bound = fqcm.lp_bound(a, bet, eps, dout, budget, lam)
        assert gap >= 0.0 and abs((loss - bound) - gap) <= 1e-9 * loss + 1e-300, (gap, loss, bound)


def test_allocation_full_size_against_lagrangian_and_bound(bm):
    """Qwen3-shaped gate projection (262 144 columns): too large for the
    oracle's dynamic program, so the checks are the Lagrangian multiplier
    (bit-exact), a loss never above the Lagrangian widths', the bits within
    the budget, and lp_gap = loss - the oracle's dual bound (printed)."""
    E, r, dout = 128, 2048, 768
    a, bet, eps = _alloc_inputs(E, r, E * r)
    full = 16 * dout * E * r
    ad, bd, ed = _cuda(a), _cuda(bet), _cuda(eps)
    for frac in (0.01, 0.15, 0.3, 0.6):
        budget = int(frac * full) + 101
        bits, lam, used, gap = bm.fqcm_allocate(ad, bd, ed, dout, budget)
        bits = bits.cpu().numpy()
        lb, rlam, lused = fqcm.lagrangian(a, bet, eps, dout, budget)
        assert lam == rlam
        loss = fqcm.total_loss(a, bet, eps, bits)
        lag = fqcm.total_loss(a, bet, eps, lb)
        bound = fqcm.lp_bound(a, bet, eps, dout, budget, lam)
        assert used <= budget and used == int(bits.astype(np.int64).sum()) * dout
        assert used >= lused and loss <= lag * (1 + 1e-12)
        assert gap >= 0.0 and abs((loss - bound) - gap) <= 1e-9 * loss
        _say("full size frac=%.2f: loss %.9e, Lagrangian %.9e, LP bound %.9e, gap %.3e "
             "(%.2e of the loss), units left %d" % (frac, loss, lag, bound, gap, gap / loss,
                                                   (budget - used) // dout))


def test_fqcm_chain_feeds_the_device_packer(bm):
    # eps and beta from the device, the allocation under the synthetic
    # layer's own bit total, then a device pack of the new widths
    L = synth.make_layer(synth.LAYERS["tiny"])
    spec = L.spec
    P, a = L.p["gate"], L.a["gate"]
    rng = np.random.default_rng(5)
    T = 64
    z = (rng.standard_normal((T, spec.r)) * 0.1).astype(np.float32)
    ids = np.stack([rng.choice(spec.E, spec.k, replace=False) for _ in range(T)]).astype(np.int32)
    g = np.full((T, spec.k), 1.0 / spec.k, np.float32)
    pd, ad = _cuda(P), _cuda(a)
    eps = bm.fqcm_distortion(pd)
    bet = bm.fqcm_beta(_cuda(z), _cuda(ids), _cuda(g), spec.E)
    budget = int(L.bits["gate"].astype(np.int64).sum()) * spec.dout
    bits, lam, used, gap = bm.fqcm_allocate(ad, bet, eps, spec.dout, budget)
    bits = bits.cpu().numpy()
    assert used <= budget and used == int(bits.astype(np.int64).sum()) * spec.dout
    assert set(np.unique(bits)) <= set(fqcm.WIDTHS)
    blob = bm.pack_device(pd, ad, bits).cpu().numpy()
    assert bm.blob_check(blob) == (spec.E, spec.dout, spec.r)
    # the oracle, from the same z, routing and p, gives the same widths
    rb, rused = fqcm.allocate(a, fqcm.beta(z, ids, g, spec.E),
                              fqcm.distortion(P.reshape(-1, spec.dout)).reshape(
                                  spec.E, spec.r, 8), spec.dout, budget)
    agree = np.mean(rb == bits)
    assert agree >= 0.98, agree   # float64 sums in another order may move a near tie
