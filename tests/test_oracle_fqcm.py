"""Pins of the FQCM oracle (oracle/fqcm.py).

* distortion: eps(0) against an exactly rounded sum of squares; the golden
  hand-derived quantizer cases (tests/golden/quantizer_cases.json) give eps(b)
  from their printed codes, scale and offset; columns that the quantizer
  represents exactly give 0 (two-level columns at b = 1, fp16 values at 16).
* beta: the one-hot routing matrix form G^T (z * z), a different order of
  summation; linearity in the routing weights; unrouted experts stay 0.
* allocation (the integer program's minimum within the budget): brute force
  over every allocation of tiny instances gives the same minimum loss (and
  the same widths where that minimum is unique); a hand-built instance whose
  Lagrangian result leaves a unit unused that the optimum spends; the dual
  bound D(lam) is never above it; at a budget the Lagrangian result uses up,
  both agree; the end points of the budget.
* Lagrangian: optimal for the bits it uses (brute force).
"""
import itertools
import json
import math
import os

import numpy as np
import pytest

from oracle import fqcm

GOLD = os.path.join(os.path.dirname(__file__), "golden", "quantizer_cases.json")
W = np.array(fqcm.WIDTHS)


def _unit(n, dout, seed):
    rng = np.random.default_rng(seed)
    P = rng.standard_normal((n, dout)).astype(np.float32)
    return (P / np.linalg.norm(P, axis=1, keepdims=True)).astype(np.float32)


def test_eps_zero_width_is_the_squared_norm():
    P = _unit(7, 50, 1)
    eps = fqcm.distortion(P)
    for i in range(7):
        ref = math.fsum(float(v) * float(v) for v in P[i])
        assert abs(eps[i, 0] - ref) <= 1e-15 * ref


def test_eps_from_hand_derived_cases():
    with open(GOLD) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        p = np.array(c["p"], np.float32)
        s = float(np.uint16(int(c["s_bits"], 16)).view(np.float16))
        m = float(np.uint16(int(c["m_bits"], 16)).view(np.float16))
        ref = math.fsum((float(pi) - (m + s * qi)) ** 2 for pi, qi in zip(p, c["q"]))
        got = fqcm.distortion(p[None])[0, list(fqcm.WIDTHS).index(c["b"])]
        assert abs(got - ref) <= 1e-15 * max(ref, 1e-30), c


def test_eps_exact_columns_are_zero():
    # two fp16 values whose difference is an fp16 value: exact at one bit
    col = np.array([0.25, 0.75, 0.25, 0.75, 0.25], np.float32)
    eps = fqcm.distortion(col[None])[0]
    assert eps[1] == 0.0 and eps[7] == 0.0 and eps[0] > 0
    # fp16 values: exact at 16 bits
    col = np.array([0.1, -0.3, 0.7], np.float32).astype(np.float16).astype(np.float32)
    assert fqcm.distortion(col[None])[0, 7] == 0.0


def test_beta_matches_routing_matrix_form():
    rng = np.random.default_rng(2)
    T, k, E, r = 9, 3, 5, 11
    z = rng.standard_normal((T, r)).astype(np.float32)
    ids = rng.integers(0, E - 1, size=(T, k))          # expert E-1 never routed
    g = rng.random((T, k)).astype(np.float32)
    G = np.zeros((T, E))
    for t in range(T):
        for j in range(k):
            G[t, ids[t, j]] += np.float64(g[t, j])
    ref = G.T @ (z.astype(np.float64) ** 2)
    got = fqcm.beta(z, ids, g, E)
    assert np.allclose(got, ref, rtol=1e-13, atol=0)
    assert np.all(got[E - 1] == 0)
    assert np.allclose(fqcm.beta(z, ids, 2 * g, E), 2 * got, rtol=1e-15, atol=0)


def _tiny(n, seed, dout=6):
    rng = np.random.default_rng(seed)
    P = _unit(n, dout, seed + 50)
    eps = fqcm.distortion(P)
    a = rng.lognormal(0, 0.7, n).astype(np.float32)
    bet = rng.lognormal(0, 1.0, n)
    return a, bet, eps, dout


def _brute(L, dout, budget):
    """(least loss, its allocations) over every allocation within budget;
    losses summed in column order, as float64."""
    best, arg = math.inf, []
    for combo in itertools.product(range(len(W)), repeat=L.shape[0]):
        if int(W[list(combo)].sum()) * dout > budget:
            continue
        v = 0.0
        for i, c in enumerate(combo):
            v += float(L[i, c])
        if v < best * (1 - 1e-12):
            best, arg = v, [combo]
        elif v <= best * (1 + 1e-12):
            arg.append(combo)
    return best, arg


@pytest.mark.parametrize("seed", [0, 1, 2, 3])
def test_lagrangian_is_optimal_for_the_bits_it_uses(seed):
    a, bet, eps, dout = _tiny(4, seed)
    L = fqcm.losses(a, bet, eps)
    for budget in (0, dout, 5 * dout, 11 * dout, 23 * dout, 40 * dout, 64 * dout):
        bits, lam, used = fqcm.lagrangian(a, bet, eps, dout, budget)
        assert used <= budget and used == int(bits.astype(np.int64).sum()) * dout
        got = fqcm.total_loss(a, bet, eps, bits)
        best, _ = _brute(L, dout, used)
        assert got <= best * (1 + 1e-12) + 1e-300, (seed, budget, got, best)


@pytest.mark.parametrize("seed", [0, 1, 2, 3, 6])
def test_allocation_is_the_brute_force_minimum(seed):
    a, bet, eps, dout = _tiny(4, seed)
    L = fqcm.losses(a, bet, eps)
    for units in (0, 1, 2, 3, 5, 7, 11, 13, 19, 23, 31, 40, 64):
        budget = units * dout + (seed % 3)      # a remainder below one unit
        bits, used = fqcm.allocate(a, bet, eps, dout, budget)
        assert used <= budget and used == int(bits.astype(np.int64).sum()) * dout
        got = fqcm.total_loss(a, bet, eps, bits)
        best, arg = _brute(L, dout, budget)
        assert abs(got - best) <= 1e-12 * best + 1e-300, (seed, units, got, best)
        if len(arg) == 1:
            assert np.array_equal(bits, W[list(arg[0])]), (seed, units)


def test_allocation_spends_what_the_lagrangian_leaves():
    """Three columns, 3 budget units (dout = 1, a = beta = 1, so L = eps):
    A drops 10 at width 2, B drops 9 at width 2, C drops 4 at width 1.  The
    multiplier that first fits (4.5) takes A alone (2 units, loss 13); the
    optimum adds C in the unit left over (loss 9)."""
    eps = np.array([[10, 10, 0, 0, 0, 0, 0, 0],
                    [9, 9, 0, 0, 0, 0, 0, 0],
                    [4, 0, 0, 0, 0, 0, 0, 0]], dtype=np.float64)
    a = np.ones(3, np.float32)
    bet = np.ones(3)
    bits, lam, used = fqcm.lagrangian(a, bet, eps, 1, 3)
    assert list(bits) == [2, 0, 0] and lam == 4.5 and used == 2
    assert fqcm.total_loss(a, bet, eps, bits) == 13.0
    bits, used = fqcm.allocate(a, bet, eps, 1, 3)
    assert list(bits) == [2, 0, 1] and used == 3
    assert fqcm.total_loss(a, bet, eps, bits) == 9.0
    assert fqcm.lp_bound(a, bet, eps, 1, 3, 4.5) <= 9.0


@pytest.mark.parametrize("seed", [4, 5])
def test_allocation_against_lagrangian_and_dual_bound(seed):
    a, bet, eps, dout = _tiny(12, seed)
    for units in (3, 17, 40, 77, 150):
        budget = units * dout
        bits, used = fqcm.allocate(a, bet, eps, dout, budget)
        got = fqcm.total_loss(a, bet, eps, bits)
        lb, lam, lused = fqcm.lagrangian(a, bet, eps, dout, budget)
        lag = fqcm.total_loss(a, bet, eps, lb)
        assert got <= lag * (1 + 1e-12)                 # never worse than the relaxation
        for f in (0.0, 0.5, 1.0, 2.0):                   # weak duality
            assert fqcm.lp_bound(a, bet, eps, dout, budget, f * lam) <= got * (1 + 1e-12)
        # at the bits the Lagrangian result uses, it is optimal: equal losses
        b2, u2 = fqcm.allocate(a, bet, eps, dout, lused)
        assert abs(fqcm.total_loss(a, bet, eps, b2) - lag) <= 1e-12 * lag


def test_allocation_end_points():
    a, bet, eps, dout = _tiny(6, 9)
    bits, used = fqcm.allocate(a, bet, eps, dout, 0)
    assert np.all(bits == 0) and used == 0
    bits, used = fqcm.allocate(a, bet, eps, dout, dout - 1)   # less than one unit
    assert np.all(bits == 0) and used == 0
    bits, used = fqcm.allocate(a, bet, eps, dout, 10 ** 9)
    L = fqcm.losses(a, bet, eps)
    assert np.array_equal(bits, W[np.argmin(L, axis=1)])
    bits, lam, used = fqcm.lagrangian(a, bet, eps, dout, 10 ** 9)
    assert lam == 0.0 and np.array_equal(bits, W[np.argmin(L, axis=1)])
    # an expert that calibration never routes to gets no bits
    bet0 = bet.copy()
    bet0[2] = 0.0
    bits, used = fqcm.allocate(a, bet0, eps, dout, 30 * dout)
    assert bits[2] == 0
    # more budget never raises the loss
    prev = math.inf
    for units in range(0, 60, 3):
        b, _ = fqcm.allocate(a, bet, eps, dout, units * dout)
        cur = fqcm.total_loss(a, bet, eps, b)
        assert cur <= prev * (1 + 1e-12)
        prev = cur


def test_losses_scale_with_a_squared_and_beta():
    a, bet, eps, dout = _tiny(5, 11)
    L = fqcm.losses(a, bet, eps)
    assert np.allclose(fqcm.losses(2 * a, bet, eps), 4 * L, rtol=1e-15, atol=0)
    assert np.allclose(fqcm.losses(a, 3 * bet, eps), 3 * L, rtol=1e-15, atol=0)
    assert np.all(fqcm.losses(a, bet, 0 * eps) == 0)
    # one column, one width: the product of the three factors
    i, c = 3, 2
    assert L[i, c] == pytest.approx(float(a[i]) ** 2 * bet[i] * eps[i, c], rel=1e-15)
