"""Per-column quantization of the unit direction vectors p_{e,k}.

Source: BitsMoE blog note, "Methodology / second split" (each unit direction
p_{e,k} is quantized at its own width; the magnitude a_{e,k} is kept apart)
and "Usage" (the width set {0,1,2,3,4,6,8,16}: 0 means the component is
dropped, 16 means it is kept as FP16).

The pages do not fix the quantizer itself.  Reading used here (uniform
asymmetric codes with an fp16 scale and an fp16 offset per column, the
offset being a value, not an integer zero point):

  for 1 <= b <= 8, with all arithmetic in IEEE float32 and no fused ops:
    lo = min_i p_i, hi = max_i p_i, L = 2^b - 1
      (lo orders -0 below +0, as the IEEE 754 minimum does: a column whose
      smallest value is zero with both signs present gets m = -0)
    s = fp16_rne((hi - lo) / L); if s == 0 then s = 1
    m = fp16_rne(lo)
    q_i = clamp(round_half_even((p_i - m) / s), 0, L)
    p_hat_i = m + s * q_i                      (exact in float64)
  b = 16: p_hat_i = fp16_rne(p_i)
  b = 0 : the column is absent; it contributes nothing.

Pinned by tests/test_oracle_quantize.py: hand-derived cases
(tests/golden/quantizer_cases.json), the code range, the half-step error
bound, the two-level set at b = 1, and numpy's own float16 rounding for
b = 16.
"""
import numpy as np

WIDTHS = (0, 1, 2, 3, 4, 6, 8, 16)
Q_WIDTHS = (1, 2, 3, 4, 6, 8)


def fp16_rne(x) -> np.ndarray:
    """float32 -> float16, round to nearest, ties to even (numpy's cast)."""
    return np.asarray(x, dtype=np.float32).astype(np.float16)


def quantize_columns(P: np.ndarray, b: int):
    """Quantize each row of P (n x dout float32, one column p per row) at b.

    Returns (q uint16 n x dout, s float16 n, m float16 n) for 1 <= b <= 8,
    the float16 values (n x dout) for b == 16, None for b == 0.
    """
    P = np.asarray(P, dtype=np.float32)
    if b == 0:
        return None
    if b == 16:
        return fp16_rne(P)
    if b not in Q_WIDTHS:
        raise ValueError("width %r not in %r" % (b, WIDTHS))
    L = np.float32(2 ** b - 1)
    lo = P.min(axis=1)
    # the sign of a zero minimum: -0 if any -0 is present (IEEE minimum)
    neg0 = np.any((P == 0) & np.signbit(P), axis=1)
    lo = np.where(lo == 0, np.where(neg0, np.float32(-0.0), np.float32(0.0)),
                  lo).astype(np.float32)
    hi = P.max(axis=1)
    s32 = (hi - lo) / L                       # float32 subtract, float32 divide
    s = fp16_rne(s32)
    s = np.where(s == np.float16(0), np.float16(1), s).astype(np.float16)
    m = fp16_rne(lo)
    v = (P - m.astype(np.float32)[:, None]) / s.astype(np.float32)[:, None]
    q = np.clip(np.rint(v), np.float32(0), L).astype(np.uint16)
    return q, s, m


def quantize_column(p: np.ndarray, b: int):
    """Single-column form of quantize_columns (p: dout float32)."""
    out = quantize_columns(np.asarray(p, dtype=np.float32)[None, :], b)
    if out is None:
        return None
    if b == 16:
        return out[0]
    q, s, m = out
    return q[0], s[0], m[0]


def dequantize(q: np.ndarray, s, m) -> np.ndarray:
    """p_hat = m + s*q in float64 (exact for fp16 s, m and q < 2^8)."""
    s = np.asarray(s, dtype=np.float64)
    m = np.asarray(m, dtype=np.float64)
    if s.ndim == 1:
        s = s[:, None]
        m = m[:, None]
    return m + s * np.asarray(q, dtype=np.float64)


def quantize_expert(p_e: np.ndarray, bits_e: np.ndarray):
    """Quantize all r columns of one expert (p_e: r x dout, bits_e: r).

    Returns dict with
      'phat'  : r x dout float64 dequantized directions (0 rows for b == 0)
      'q'     : r x dout uint16 codes (b <= 8), fp16 bit patterns (b == 16),
                0 for b == 0
      's','m' : r float16 (1 and 0 where unused)
    """
    r, dout = p_e.shape
    phat = np.zeros((r, dout), dtype=np.float64)
    q = np.zeros((r, dout), dtype=np.uint16)
    s = np.ones(r, dtype=np.float16)
    m = np.zeros(r, dtype=np.float16)
    for b in Q_WIDTHS:
        cols = np.nonzero(bits_e == b)[0]
        if cols.size == 0:
            continue
        qq, ss, mm = quantize_columns(p_e[cols], b)
        q[cols] = qq
        s[cols] = ss
        m[cols] = mm
        phat[cols] = dequantize(qq, ss, mm)
    cols = np.nonzero(bits_e == 16)[0]
    if cols.size:
        h = quantize_columns(p_e[cols], 16)
        q[cols] = h.view(np.uint16)
        phat[cols] = h.astype(np.float64)
    return {"phat": phat, "q": q, "s": s, "m": m}
