"""FQCM importance and budgeted width allocation (test infrastructure only).

Source: BitsMoE blog note, the FQCM part of the Methodology (the routed
activation importance beta, the loss L = a^2 beta eps and the marginal gain
of a wider code) and "Usage" (the allocation under a bit budget over the
widths {0,1,2,3,4,6,8,16}, solved by the authors as an integer linear
program).

Readings used here (the pages leave these steps open):
  * beta_{e,k} = sum over calibration pairs (t, slot) routed to e of
    g_{t,slot} (phi_k^T x_t)^2, i.e. with z_t = Phi^T x_t, the routing-weighted
    sum of z_{t,k}^2; accumulated in float64 in pair order.
  * eps_{e,k}(b) = || p_{e,k} - Q_b(p_{e,k}) ||^2 with Q_b the format's
    quantizer (oracle.quantize: fp16 scale and offset, float32 codes),
    eps(0) = ||p||^2 (the column is dropped) and eps(16) the fp16 rounding
    error; float64 sums.
  * L_{e,k}(b) = a_{e,k}^2 beta_{e,k} eps_{e,k}(b), evaluated as
    ((a * a) * beta) * eps in float64.
  * Budget: sum over columns of dout * b <= budget bits (the pages count a
    wider code by its m = dout extra bits per unit of width; metadata and
    group padding are not counted), i.e. sum of b <= floor(budget / dout)
    budget units.
  * Solver: the integer program itself, solved exactly (allocate): a plain
    dynamic program over the columns in order and the budget units used so
    far, float64 sums, ties to the narrower width at each column and, among
    equal totals, to the fewest units.  Any solver giving the same minimum
    is equivalent; this one is here because a reader can check it by eye.
  * The Lagrangian relaxation (lagrangian, lp_bound) is kept for the
    multiplier the library reports and for the dual bound: for a multiplier
    lam >= 0 each column takes the width minimising L(b) + lam * (dout * b)
    (float64, ties to the narrower width), lam is the smallest float64 whose
    total fits (bisection over the ordered bit patterns of non-negative
    doubles), and D(lam) = sum over columns of that minimum - lam * dout *
    floor(budget / dout) is a lower bound on every allocation's loss.

Pinned by tests/test_oracle_fqcm.py: closed forms of eps (dropped column,
exact two-level columns, fp16-exact columns), brute-force beta loops,
brute-force enumeration of every allocation on tiny instances (the dynamic
program's minimum is the brute-force minimum), a hand-built instance where
the Lagrangian result is not optimal, the dual bound, and planted mistakes.
"""
import numpy as np

from oracle.quantize import Q_WIDTHS, dequantize, fp16_rne, quantize_columns

WIDTHS = (0, 1, 2, 3, 4, 6, 8, 16)


def distortion(P: np.ndarray) -> np.ndarray:
    """P: n x dout float32 unit directions.  Returns n x 8 float64 eps for
    the widths (0, 1, 2, 3, 4, 6, 8, 16)."""
    P = np.asarray(P, dtype=np.float32)
    p64 = P.astype(np.float64)
    out = np.zeros((P.shape[0], len(WIDTHS)), dtype=np.float64)
    out[:, 0] = (p64 * p64).sum(axis=1)
    for i, b in enumerate(WIDTHS):
        if b == 0:
            continue
        if b == 16:
            phat = fp16_rne(P).astype(np.float64)
        else:
            q, s, m = quantize_columns(P, b)
            phat = dequantize(q, s, m)
        d = p64 - phat
        out[:, i] = (d * d).sum(axis=1)
    return out


def beta(z: np.ndarray, ids: np.ndarray, g: np.ndarray, E: int) -> np.ndarray:
    """z: T x r float32 (z_t = Phi^T x_t); ids, g: T x k routing.  Returns
    E x r float64 beta, summed in pair order (t, then slot)."""
    z = np.asarray(z, dtype=np.float32)
    T, k = ids.shape
    out = np.zeros((E, z.shape[1]), dtype=np.float64)
    for t in range(T):
        z2 = z[t].astype(np.float64) * z[t].astype(np.float64)
        for j in range(k):
            e = int(ids[t, j])
            if 0 <= e < E:
                out[e] += np.float64(g[t, j]) * z2
    return out


def losses(a: np.ndarray, bet: np.ndarray, eps: np.ndarray) -> np.ndarray:
    """L(b) = ((a * a) * beta) * eps(b) in float64; shape (..., 8)."""
    a = np.asarray(a, dtype=np.float32).astype(np.float64)
    imp = (a * a) * np.asarray(bet, dtype=np.float64)
    return imp[..., None] * np.asarray(eps, dtype=np.float64)


def choose(L: np.ndarray, dout: int, lam: float) -> np.ndarray:
    """Per-column width index minimising L(b) + lam * (dout * b); ties go to
    the narrower width (the first minimum)."""
    cost = L + np.float64(lam) * (np.float64(dout) * np.array(WIDTHS, dtype=np.float64))
    return np.argmin(cost, axis=-1)


def _bits_used(idx: np.ndarray, dout: int) -> int:
    return int(np.array(WIDTHS, dtype=np.int64)[idx].sum()) * int(dout)


def lagrangian(a: np.ndarray, bet: np.ndarray, eps: np.ndarray, dout: int, budget_bits: int):
    """Lagrangian relaxation: returns (bits uint8 like a, lam float64, bits
    used) at the smallest lam whose allocation fits."""
    L = losses(a, bet, eps)
    widths = np.array(WIDTHS, dtype=np.uint8)
    idx0 = choose(L, dout, 0.0)
    if _bits_used(idx0, dout) <= budget_bits:
        return widths[idx0], 0.0, _bits_used(idx0, dout)
    # smallest lam (as a non-negative double) whose total fits; +inf always
    # fits (every column at width 0)
    lo, hi = 0, int(np.float64(np.inf).view(np.uint64))
    while hi - lo > 1:
        mid = (lo + hi) // 2
        lam = float(np.uint64(mid).view(np.float64))
        if _bits_used(choose(L, dout, lam), dout) <= budget_bits:
            hi = mid
        else:
            lo = mid
    lam = float(np.uint64(hi).view(np.float64))
    idx = choose(L, dout, lam)
    return widths[idx], lam, _bits_used(idx, dout)


def lp_bound(a, bet, eps, dout: int, budget_bits: int, lam: float) -> float:
    """Dual bound D(lam) <= the loss of every allocation within the budget."""
    L = losses(a, bet, eps).reshape(-1, len(WIDTHS))
    cost = L + np.float64(lam) * (np.float64(dout) * np.array(WIDTHS, dtype=np.float64))
    return float(cost.min(axis=1).sum()) - float(lam) * float(dout) * float(budget_bits // dout)


def allocate(a: np.ndarray, bet: np.ndarray, eps: np.ndarray, dout: int, budget_bits: int):
    """Minimum-loss widths within the budget.  Returns (bits uint8 like a,
    bits used).

    best[u] holds the least loss of the columns so far using exactly u units
    (inf where no choice reaches u); column c moves it to min over widths w
    of best[u - w] + L_c(w).  The answer is the least best[u] over u <= the
    budget units, read back through the recorded choices."""
    L = losses(a, bet, eps).reshape(-1, len(WIDTHS))
    n = L.shape[0]
    W = np.array(WIDTHS, dtype=np.int64)
    U = int(min(budget_bits // dout, int(W[-1]) * n))
    best = np.full(U + 1, np.inf)
    best[0] = 0.0
    pick = np.zeros((n, U + 1), dtype=np.uint8)
    for c in range(n):
        new = np.full(U + 1, np.inf)
        for i, w in enumerate(W):          # narrower widths first: they keep ties
            if w > U:
                break
            cand = np.full(U + 1, np.inf)
            cand[w:] = best[:U + 1 - w] + L[c, i]
            better = cand < new
            new[better] = cand[better]
            pick[c, better] = i
        best = new
    u = int(np.argmin(best))                # first minimum: the fewest units
    idx = np.zeros(n, dtype=np.int64)
    for c in range(n - 1, -1, -1):
        idx[c] = pick[c, u]
        u -= int(W[idx[c]])
    assert u == 0
    bits = W[idx].astype(np.uint8).reshape(np.shape(a))
    return bits, int(W[idx].sum()) * int(dout)


def total_loss(a, bet, eps, bits) -> float:
    L = losses(a, bet, eps)
    idx = np.searchsorted(np.array(WIDTHS), np.asarray(bits))
    return float(np.take_along_axis(L, idx[..., None], axis=-1).sum())
