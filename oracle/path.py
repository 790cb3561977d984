"""Float64 restatement of the decode-time gate/up path.

Sources (BitsMoE blog note, "Methodology"):
* first split: with P = U Sigma, W_e x = P (Phi^T x); the bracket does not
  depend on the expert, so the experts a token selects share z = Phi^T x;
  the computation is x -> z = Phi^T x -> the expert's own P A applied to z.
* second split: W_e = sum_k a_{e,k} p_{e,k} phi_k^T with unit p_{e,k}; only
  p_{e,k} is quantized, so the expert output is
  y_e = sum_{k : b_{e,k} > 0} a_{e,k} z_k p_hat_{e,k}.
The gate/up pairing h = SiLU(y_gate) * y_up, SiLU(v) = v / (1 + e^-v), is the
usual gated MLP of the modelled MoE layers; the pages only name gate_proj and
up_proj.  Routing weights are not applied to h (they belong after the down
projection).

Pins (tests/test_oracle_path.py): Phi = I and Phi = permutation give z
exactly; Parseval for orthogonal Phi; the brute-force dense product
(sum_k a p_hat phi^T) x; one-hot a; linearity; 0-bit columns removable
bit-for-bit; SiLU against scipy's logistic function and its odd-part
identity.
"""
import numpy as np

from .quantize import quantize_expert


def spectral_proj(phi: np.ndarray, x: np.ndarray) -> np.ndarray:
    """z[t, k] = sum_i phi[i, k] x[t, i]  (phi: din x r, x: T x din)."""
    phi = np.asarray(phi, dtype=np.float64)
    x = np.atleast_2d(np.asarray(x, dtype=np.float64))
    return x @ phi


def expert_apply(z: np.ndarray, a_e: np.ndarray, phat_e: np.ndarray,
                 bits_e: np.ndarray) -> np.ndarray:
    """y[t, i] = sum over k ascending with b_k > 0 of a_k z[t,k] phat[k, i].

    z: T x r, a_e: r, phat_e: r x dout (float64), bits_e: r.
    """
    z = np.atleast_2d(np.asarray(z, dtype=np.float64))
    a_e = np.asarray(a_e, dtype=np.float64)
    y = np.zeros((z.shape[0], phat_e.shape[1]), dtype=np.float64)
    for k in np.nonzero(np.asarray(bits_e) > 0)[0]:
        y += np.outer(a_e[k] * z[:, k], phat_e[k])
    return y


def silu(v: np.ndarray) -> np.ndarray:
    v = np.asarray(v, dtype=np.float64)
    return v / (1.0 + np.exp(-v))


def moe_gateup(phi_g, phi_u, a_g, a_u, phat_g, phat_u, bits_g, bits_u,
               x: np.ndarray, ids: np.ndarray) -> np.ndarray:
    """h[t, slot, :] = SiLU(y_gate) * y_up for expert e = ids[t, slot].

    phat_*: E x r x dout float64 dequantized directions (see quantize).
    Tokens are grouped by expert only to reuse each expert's directions;
    every (t, slot) output is computed independently.
    """
    ids = np.asarray(ids)
    T, K = ids.shape
    zg = spectral_proj(phi_g, x)
    zu = spectral_proj(phi_u, x)
    dout = phat_g.shape[2]
    h = np.zeros((T, K, dout), dtype=np.float64)
    for e in np.unique(ids):
        tt, ss = np.nonzero(ids == e)
        yg = expert_apply(zg[tt], a_g[e], phat_g[e], bits_g[e])
        yu = expert_apply(zu[tt], a_u[e], phat_u[e], bits_u[e])
        h[tt, ss] = silu(yg) * yu
    return h


def dequantized_layer(p: np.ndarray, bits: np.ndarray, experts=None) -> np.ndarray:
    """phat for the listed experts (others left zero): E x r x dout float64."""
    E, r, dout = p.shape
    out = np.zeros((E, r, dout), dtype=np.float64)
    for e in (range(E) if experts is None else experts):
        out[e] = quantize_expert(p[e], bits[e])["phat"]
    return out


def moe_down(phi_d, a_d, phat_d, bits_d, h: np.ndarray, ids: np.ndarray,
             g: np.ndarray) -> np.ndarray:
    """out[t, :] = sum over slots j (ascending) of g[t, j] * y_{t,j}, with
    y_{t,j} = sum_k a_{e,k} z_k p_hat_{e,k} for e = ids[t, j] and
    z = Phi_down^T fp16(h[t, j]).

    The down projection restated with the same two splits (BitsMoE blog
    note, Methodology): its shared basis Phi_down (dout x r_d) lives in the
    input space of down_proj, so z depends on the pair's own h and is formed
    per (token, slot); the pages name only gate and up, so this is the plain
    extension.  Reading: the down projection's input is h rounded to fp16
    (the activation precision of the path); the routing weights g are
    applied once, after the expert products.  phat_d: E x r_d x din float64.
    h: T x k x dout; returns T x din float64.  Pairs whose id is outside
    [0, E) are skipped.
    """
    ids = np.asarray(ids)
    T, K = ids.shape
    E = phat_d.shape[0]
    h16 = np.asarray(h, dtype=np.float32).astype(np.float16)
    out = np.zeros((T, phat_d.shape[2]), dtype=np.float64)
    for t in range(T):
        for j in range(K):
            e = int(ids[t, j])
            if not 0 <= e < E:
                continue
            z = spectral_proj(phi_d, h16[t, j])
            y = expert_apply(z, a_d[e], phat_d[e], bits_d[e])[0]
            out[t] += np.float64(g[t, j]) * y
    return out
