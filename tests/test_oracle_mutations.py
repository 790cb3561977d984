"""Planted mistakes in the oracle must be caught by its pins.

Each case swaps one oracle function for a copy with a plausible slip (a wrong
rounding rule, a dropped term, a transposed operand, a flipped sign, a wrong
bit order) and checks that at least one pin test then fails.  The mistakes
live only here, on the CPU.
"""
import numpy as np
import pytest

from oracle import fmt, path, quantize
import tests.test_oracle_fmt as T_fmt
import tests.test_oracle_path as T_path
import tests.test_oracle_quantize as T_q


def _q_half_up(P, b):
    P = np.asarray(P, dtype=np.float32)
    if b in (0, 16):
        return _orig_qc(P, b)
    L = np.float32(2 ** b - 1)
    lo, hi = P.min(axis=1), P.max(axis=1)
    s = quantize.fp16_rne((hi - lo) / L)
    s = np.where(s == 0, np.float16(1), s).astype(np.float16)
    m = quantize.fp16_rne(lo)
    v = (P - m.astype(np.float32)[:, None]) / s.astype(np.float32)[:, None]
    return np.clip(np.floor(v + np.float32(0.5)), 0, L).astype(np.uint16), s, m


def _q_wrong_levels(P, b):
    P = np.asarray(P, dtype=np.float32)
    if b in (0, 16):
        return _orig_qc(P, b)
    L = np.float32(2 ** b)            # 2^b instead of 2^b - 1
    lo, hi = P.min(axis=1), P.max(axis=1)
    s = quantize.fp16_rne((hi - lo) / L)
    m = quantize.fp16_rne(lo)
    v = (P - m.astype(np.float32)[:, None]) / s.astype(np.float32)[:, None]
    return np.clip(np.rint(v), 0, L - 1).astype(np.uint16), s, m


_orig_qc = quantize.quantize_columns


def _apply_shifted(z, a_e, phat_e, bits_e):
    z = np.atleast_2d(np.asarray(z, dtype=np.float64))
    y = np.zeros((z.shape[0], phat_e.shape[1]))
    r = len(a_e)
    for k in np.nonzero(np.asarray(bits_e) > 0)[0]:
        y += np.outer(a_e[k] * z[:, (k + 1) % r], phat_e[k])    # wrong index
    return y


def _apply_no_a(z, a_e, phat_e, bits_e):
    z = np.atleast_2d(np.asarray(z, dtype=np.float64))
    y = np.zeros((z.shape[0], phat_e.shape[1]))
    for k in np.nonzero(np.asarray(bits_e) > 0)[0]:
        y += np.outer(z[:, k], phat_e[k])                        # dropped a
    return y


def _proj_transposed(phi, x):
    return np.atleast_2d(np.asarray(x, dtype=np.float64)) @ np.asarray(phi, dtype=np.float64).T


def _silu_sign(v):
    v = np.asarray(v, dtype=np.float64)
    return v / (1.0 + np.exp(v))


def _fails(fn, *args):
    try:
        fn(*args)
    except AssertionError:
        return True
    return False


def test_rounding_half_up_caught(monkeypatch):
    monkeypatch.setattr(quantize, "quantize_columns", _q_half_up)
    cases = T_q._cases()["cases"]
    assert any(_fails(T_q.test_hand_derived, c) for c in cases)


def test_wrong_level_count_caught(monkeypatch):
    monkeypatch.setattr(quantize, "quantize_columns", _q_wrong_levels)
    cases = T_q._cases()["cases"]
    assert any(_fails(T_q.test_hand_derived, c) for c in cases)


@pytest.mark.parametrize("bad", [_apply_shifted, _apply_no_a])
def test_expert_apply_slips_caught(monkeypatch, bad):
    monkeypatch.setattr(path, "expert_apply", bad)
    assert _fails(T_path.test_brute_force_dense) or _fails(T_path.test_one_hot_and_linearity)


def test_transposed_projection_caught(monkeypatch):
    monkeypatch.setattr(path, "spectral_proj", _proj_transposed)
    assert _fails(T_path.test_identity_and_permutation_projection)


def test_silu_sign_caught(monkeypatch):
    monkeypatch.setattr(path, "silu", _silu_sign)
    assert _fails(T_path.test_silu_identities)


def test_plane_bit_order_caught(monkeypatch):
    # rows and slots swapped inside a plane word
    monkeypatch.setattr(fmt, "plane_bit", lambda rho, u: 4 * rho + u)
    assert _fails(T_fmt.test_hand_built_planes)


# ---- FQCM oracle ----
from oracle import fqcm  # noqa: E402
import tests.test_oracle_fqcm as T_f  # noqa: E402

_orig_losses = fqcm.losses
_orig_allocate = fqcm.allocate


def _losses_a_not_squared(a, bet, eps):
    a = np.asarray(a, dtype=np.float32).astype(np.float64)
    return (a * np.asarray(bet, dtype=np.float64))[..., None] * np.asarray(eps, dtype=np.float64)


def _beta_not_squared(z, ids, g, E):
    z = np.asarray(z, dtype=np.float32)
    out = np.zeros((E, z.shape[1]))
    for t in range(ids.shape[0]):
        for j in range(ids.shape[1]):
            out[int(ids[t, j])] += np.float64(g[t, j]) * z[t].astype(np.float64)   # z, not z^2
    return out


def _distortion_m_minus(P):
    P = np.asarray(P, dtype=np.float32)
    res = np.zeros((P.shape[0], 8))
    p64 = P.astype(np.float64)
    res[:, 0] = (p64 * p64).sum(axis=1)
    for i, b in enumerate(fqcm.WIDTHS):
        if b in (0, 16):
            continue
        q, s, m = quantize.quantize_columns(P, b)
        phat = m.astype(np.float64)[:, None] - s.astype(np.float64)[:, None] * q   # sign slip
        res[:, i] = ((p64 - phat) ** 2).sum(axis=1)
    res[:, 7] = ((p64 - P.astype(np.float16).astype(np.float64)) ** 2).sum(axis=1)
    return res


_orig_lagrangian = fqcm.lagrangian


def _allocate_over_budget(a, bet, eps, dout, budget):
    # the last multiplier that did not fit: one step of the hull too many
    bits, lam, used = _orig_lagrangian(a, bet, eps, dout, budget)
    if lam > 0:
        L = _orig_losses(a, bet, eps)
        lam2 = float(np.nextafter(lam, 0.0))
        idx = fqcm.choose(L, dout, lam2)
        bits = np.array(fqcm.WIDTHS, np.uint8)[idx]
        used = int(bits.astype(np.int64).sum()) * dout
    return bits, used


def _allocate_is_lagrangian(a, bet, eps, dout, budget):
    bits, lam, used = _orig_lagrangian(a, bet, eps, dout, budget)
    return bits, used


def _allocate_dp_off_by_one_unit(a, bet, eps, dout, budget):
    # the dynamic program run with one budget unit too few
    return _orig_allocate(a, bet, eps, dout, max(budget - dout, 0))


def test_fqcm_loss_without_a_squared_caught(monkeypatch):
    monkeypatch.setattr(fqcm, "losses", _losses_a_not_squared)
    assert _fails(T_f.test_losses_scale_with_a_squared_and_beta)


def test_fqcm_beta_slip_caught(monkeypatch):
    monkeypatch.setattr(fqcm, "beta", _beta_not_squared)
    assert _fails(T_f.test_beta_matches_routing_matrix_form)


def test_fqcm_distortion_sign_caught(monkeypatch):
    monkeypatch.setattr(fqcm, "distortion", _distortion_m_minus)
    assert _fails(T_f.test_eps_from_hand_derived_cases)


@pytest.mark.parametrize("bad", [_allocate_over_budget, _allocate_is_lagrangian,
                                 _allocate_dp_off_by_one_unit])
def test_fqcm_allocation_slips_caught(monkeypatch, bad):
    monkeypatch.setattr(fqcm, "allocate", bad)
    assert any(_fails(T_f.test_allocation_is_the_brute_force_minimum, s) for s in range(4))
    assert _fails(T_f.test_allocation_spends_what_the_lagrangian_leaves)


_orig_down = path.moe_down


def _down_no_fp16(phi_d, a_d, phat_d, bits_d, h, ids, g):
    return _orig_down(phi_d, a_d, phat_d, bits_d,
                      np.asarray(h, np.float64).astype(np.float32) * np.float32(1 + 2 ** -12),
                      ids, g)


def _down_gate_squared(phi_d, a_d, phat_d, bits_d, h, ids, g):
    return _orig_down(phi_d, a_d, phat_d, bits_d, h, ids, np.asarray(g, np.float32) ** 2)


@pytest.mark.parametrize("bad", [_down_no_fp16, _down_gate_squared])
def test_moe_down_slips_caught(monkeypatch, bad):
    monkeypatch.setattr(path, "moe_down", bad)
    assert _fails(T_path.test_moe_down_against_dense_expert_matrices)
