"""Pins of the oracle quantizer (oracle/quantize.py).

Hand-derived cases (tests/golden/quantizer_cases.json), the code range, the
half-step error bound, the two-level set at b = 1, and nearest-fp16 checks
for b = 16 that do not reuse numpy's cast.
"""
import json
import os

import numpy as np
import pytest

from oracle.quantize import (Q_WIDTHS, dequantize, quantize_column,
                             quantize_columns, quantize_expert)

GOLD = os.path.join(os.path.dirname(__file__), "golden", "quantizer_cases.json")


def _cases():
    with open(GOLD) as f:
        return json.load(f)


@pytest.mark.parametrize("case", _cases()["cases"])
def test_hand_derived(case):
    q, s, m = quantize_column(np.array(case["p"], np.float32), case["b"])
    assert q.tolist() == case["q"]
    assert int(np.float16(s).view(np.uint16)) == int(case["s_bits"], 16)
    assert int(np.float16(m).view(np.uint16)) == int(case["m_bits"], 16)
    ph = dequantize(q[None], np.array([s]), np.array([m]))[0]
    assert ph.tolist() == case["phat"]


def test_hand_derived_fp16():
    for case in _cases()["fp16_cases"]:
        h = quantize_column(np.array(case["p"], np.float32), 16)
        assert [int(v) for v in h.view(np.uint16)] == [int(b, 16) for b in case["bits"]]


def _unit_columns(n, dout, seed):
    g = np.random.default_rng(seed).standard_normal((n, dout))
    return (g / np.linalg.norm(g, axis=1, keepdims=True)).astype(np.float32)


@pytest.mark.parametrize("b", Q_WIDTHS)
def test_range_and_error_bound(b):
    P = _unit_columns(300, 96, b)
    q, s, m = quantize_columns(P, b)
    L = 2 ** b - 1
    assert q.max() <= L and q.min() >= 0
    s64 = s.astype(np.float64)[:, None]
    m64 = m.astype(np.float64)[:, None]
    ph = dequantize(q, s, m)
    inside = (P >= m64) & (P <= m64 + s64 * L)
    err = np.abs(P.astype(np.float64) - ph)
    # half a step, plus the float32 rounding of (p - m)/s near a tie
    bound = s64 / 2 * (1 + 2 ** -20) + np.spacing(np.float32(1.0)) * np.abs(P)
    assert np.all(err[inside] <= np.broadcast_to(bound, err.shape)[inside])
    # values outside [m, m + sL] (fp16 rounding of the end points) stay
    # within one step of the nearest level
    out = ~inside
    assert np.all(err[out] <= np.broadcast_to(s64, err.shape)[out])
    # the extremes are represented: codes 0 and (nearly always) L appear
    assert np.all(q.min(axis=1) == 0)


def test_one_bit_two_levels():
    P = _unit_columns(200, 64, 7)
    q, s, m = quantize_columns(P, 1)
    ph = dequantize(q, s, m)
    lo = m.astype(np.float64)[:, None]
    hi = lo + s.astype(np.float64)[:, None]
    assert np.all((ph == lo) | (ph == hi))


def _fp16_neighbours(h):
    bits = h.view(np.uint16).astype(np.int32)
    up = (bits + np.where(h >= 0, 1, -1)).astype(np.uint16).view(np.float16)
    dn = (bits - np.where(h >= 0, 1, -1)).astype(np.uint16).view(np.float16)
    return up, dn


def test_fp16_nearest_even():
    P = _unit_columns(50, 128, 3)
    H = quantize_columns(P, 16)
    p64 = P.astype(np.float64)
    d = np.abs(H.astype(np.float64) - p64)
    up, dn = _fp16_neighbours(H)
    du = np.abs(up.astype(np.float64) - p64)
    dd = np.abs(dn.astype(np.float64) - p64)
    assert np.all(d <= du) and np.all(d <= dd)
    tie = (d == du) | (d == dd)
    assert np.all(H.view(np.uint16)[tie] % 2 == 0)


def test_zero_width_absent_and_expert_layout():
    rng = np.random.default_rng(0)
    P = _unit_columns(16, 96, 1)
    bits = np.array([0, 1, 2, 3, 4, 6, 8, 16] * 2, dtype=np.uint8)
    rng.shuffle(bits)
    out = quantize_expert(P, bits)
    assert np.all(out["phat"][bits == 0] == 0)
    for k in range(16):
        b = int(bits[k])
        if b == 0:
            continue
        if b == 16:
            assert np.array_equal(out["phat"][k], P[k].astype(np.float16).astype(np.float64))
        else:
            q, s, m = quantize_column(P[k], b)
            assert np.array_equal(out["q"][k], q)
            assert out["s"][k] == s and out["m"][k] == m


def test_rejects_bad_width():
    with pytest.raises(ValueError):
        quantize_columns(np.zeros((1, 4), np.float32), 5)


def test_zero_minimum_sign_is_order_free():
    # the offset of a column whose minimum is zero: -0 when a -0 is present
    # (IEEE minimum), whatever the order of the rows; +0 otherwise
    rng = np.random.default_rng(3)
    base = np.array([0.0, -0.0, 0.5, 0.25, 0.0, 0.75], np.float32)
    for _ in range(20):
        col = rng.permutation(base)
        for b in (1, 3, 8):
            q, s, m = quantize_column(col, b)
            assert m == 0 and np.signbit(m), (col, b)
    q, s, m = quantize_column(np.array([0.0, 0.5, 0.0], np.float32), 2)
    assert m == 0 and not np.signbit(m)
    q, s, m = quantize_column(np.array([-0.0, -0.0], np.float32), 2)
    assert np.signbit(m) and s == 1 and np.all(q == 0)
