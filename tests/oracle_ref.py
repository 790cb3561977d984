"""Oracle reference values for the GPU parity tests (CPU, float64).

Thin helpers that feed the oracle the exact inputs the GPU sees (fp16 Phi
and x) and evaluate it only at the requested (token, slot) pairs, so that
full-size layers stay cheap.  Only tests, smoke() and the benchmark's CPU
baseline use this.
"""
import numpy as np

from oracle import path
from oracle.quantize import quantize_expert


def phi16(layer, proj):
    return np.asarray(layer.phi[proj], np.float16)


def z_ref(layer, x):
    return {p: path.spectral_proj(phi16(layer, p), x) for p in ("gate", "up")}


def pairs_ref(layer, x, ids, pairs=None, want_y=False):
    """h (and optionally y_gate, y_up) at the listed (t, slot) pairs."""
    T, K = ids.shape
    if pairs is None:
        pairs = [(t, s) for t in range(T) for s in range(K)]
    z = z_ref(layer, x)
    out_h, out_g, out_u = {}, {}, {}
    by_e = {}
    for t, s in pairs:
        by_e.setdefault(int(ids[t, s]), []).append((t, s))
    for e, lst in by_e.items():
        tt = [t for t, _ in lst]
        y = {}
        for p in ("gate", "up"):
            ph = quantize_expert(layer.p[p][e], layer.bits[p][e])["phat"]
            y[p] = path.expert_apply(z[p][tt], layer.a[p][e], ph, layer.bits[p][e])
        h = path.silu(y["gate"]) * y["up"]
        for i, ts in enumerate(lst):
            out_h[ts] = h[i]
            out_g[ts] = y["gate"][i]
            out_u[ts] = y["up"][i]
    if want_y:
        return out_h, out_g, out_u
    return out_h


def max_rel_err(got, ref):
    """max |got - ref| / max |ref| (ref all zero: max |got|)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.abs(ref).max()
    err = np.abs(got - ref).max()
    return err / den if den > 0 else err
