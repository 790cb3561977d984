"""Seeded random tensors for the synthetic spectral MoE layers.

Recipe (all draws from numpy's PCG64, one independent stream per
(layer family, tensor, index) derived with SeedSequence):

* Phi (din x r) per linear type: Q factor of a QR decomposition of an N(0,1)
  matrix in float64, columns sign-fixed so that diag(R) > 0; rounded to fp16
  for the fp16 layers, kept as float32 for the tiny fp32 layer.
* a (E x r): k^-decay * exp(ln_sigma * N(0,1)), k = 1..r.
* p (E x r x dout): N(0,1) columns scaled to unit Euclidean length, float32.
* bits (E x r): for the tiny layer iid uniform over {0,1,2,3,4,6,8,16}; for
  the model-shaped layers, all E*r units of one linear type are ranked by
  descending a^2 (ties by ascending (e, k)) and the widths are dealt out
  highest first, the count of each width set by cumulative rounding of the
  histogram percentages.
* x (T x din): N(0,1), a fixed per-layer set of round(outlier_frac * din)
  channels multiplied by outlier_scale for every token, rounded to fp16.
* down projection (make_down): the same recipe with input dout, output din
  and rank r_d = min(r, dout), streams named "..._down".
* g (T x k, make_gates): softmax over each token's k slots of N(0,1) logits.
* ids (T x k): per token k distinct experts; "uniform" draws them uniformly
  without replacement; "zipf" gives experts popularity weights rank^-s (ranks
  from a seeded permutation) and takes, per token, the k largest
  Efraimidis-Spirakis keys log(u)/w.
"""
import zlib
from dataclasses import dataclass
from typing import Dict, Optional

import numpy as np

from .configs import LayerSpec, Workload, WIDTH_SET


def _rng(family: str, tensor: str, index: int = 0) -> np.random.Generator:
    ss = np.random.SeedSequence([zlib.crc32(family.encode()),
                                 zlib.crc32(tensor.encode()), int(index)])
    return np.random.Generator(np.random.PCG64(ss))


def _orthogonal(n: int, rng: np.random.Generator) -> np.ndarray:
    g = rng.standard_normal((n, n))
    q, r = np.linalg.qr(g)
    q = q * np.sign(np.diag(r))[None, :]
    return q


def histogram_bits(a: np.ndarray, hist: Dict[int, float]) -> np.ndarray:
    """Deal widths to units ranked by descending a^2 (a: E x r)."""
    E, r = a.shape
    n = E * r
    a2 = (a.astype(np.float64) ** 2).reshape(-1)
    # lexsort: last key primary -> descending a^2, then ascending flat index
    order = np.lexsort((np.arange(n), -a2))
    widths = sorted(hist.keys(), reverse=True)
    bits = np.zeros(n, dtype=np.uint8)
    cum = 0.0
    start = 0
    for w in widths:
        cum += hist[w]
        end = int(round(n * cum / 100.0))
        end = min(max(end, start), n)
        bits[order[start:end]] = w
        start = end
    bits[order[start:]] = widths[-1]
    return bits.reshape(E, r)


@dataclass
class Layer:
    spec: LayerSpec
    phi: Dict[str, np.ndarray]    # "gate"/"up": din x r (float32 or float16)
    a: Dict[str, np.ndarray]      # E x r float32
    p: Dict[str, np.ndarray]      # E x r x dout float32, unit columns
    bits: Dict[str, np.ndarray]   # E x r uint8
    outlier_channels: np.ndarray  # int64 indices into din


def _make_type(spec: LayerSpec, proj: str, n_in: int = 0, n_out: int = 0, r: int = 0):
    """Factors of one linear type: Phi (n_in x r), a (E x r), p (E x r x
    n_out), bits (E x r); gate and up use (din, dout, r)."""
    fam = spec.name
    n_in, n_out, r = n_in or spec.din, n_out or spec.dout, r or spec.r
    phi = _orthogonal(n_in, _rng(fam, "phi_" + proj))[:, :r]
    phi = phi.astype(np.float16) if spec.phi_fp16 else phi.astype(np.float32)
    rng_a = _rng(fam, "a_" + proj)
    kk = np.arange(1, r + 1, dtype=np.float64)
    a = (kk[None, :] ** (-spec.decay)) * np.exp(
        spec.ln_sigma * rng_a.standard_normal((spec.E, r)))
    a = a.astype(np.float32)
    p = np.empty((spec.E, r, n_out), dtype=np.float32)
    for e in range(spec.E):
        g = _rng(fam, "p_" + proj, e).standard_normal((r, n_out), dtype=np.float32)
        nrm = np.sqrt(np.einsum("kd,kd->k", g.astype(np.float64),
                                g.astype(np.float64)))
        p[e] = (g / nrm[:, None]).astype(np.float32)
    if spec.bits == "uniform":
        idx = _rng(fam, "bits_" + proj).integers(0, len(WIDTH_SET),
                                                 size=(spec.E, r))
        bits = np.asarray(WIDTH_SET, dtype=np.uint8)[idx]
    else:
        bits = histogram_bits(a, spec.bits)
    return phi, a, p, bits


_LAYER_CACHE: Dict[str, Layer] = {}


def make_layer(spec: LayerSpec, cache: bool = True) -> Layer:
    if cache and spec.name in _LAYER_CACHE:
        return _LAYER_CACHE[spec.name]
    phi, a, p, bits = {}, {}, {}, {}
    for proj in ("gate", "up"):
        phi[proj], a[proj], p[proj], bits[proj] = _make_type(spec, proj)
    n_out = int(round(spec.outlier_frac * spec.din))
    oc = np.sort(_rng(spec.name, "outliers").choice(spec.din, size=n_out,
                                                     replace=False))
    layer = Layer(spec, phi, a, p, bits, oc.astype(np.int64))
    if cache:
        _LAYER_CACHE[spec.name] = layer
    return layer


@dataclass
class DownType:
    """Factors of the down projection (input dout, output din): Phi_down
    (dout x r_d), a (E x r_d), p (E x r_d x din), bits (E x r_d), with
    r_d = min(r, dout)."""
    phi: np.ndarray
    a: np.ndarray
    p: np.ndarray
    bits: np.ndarray


_DOWN_CACHE: Dict[str, DownType] = {}


def make_down(layer: Layer) -> DownType:
    spec = layer.spec
    if spec.name not in _DOWN_CACHE:
        rd = min(spec.r, spec.dout)
        phi, a, p, bits = _make_type(spec, "down", n_in=spec.dout, n_out=spec.din, r=rd)
        _DOWN_CACHE[spec.name] = DownType(phi, a, p, bits)
    return _DOWN_CACHE[spec.name]


def make_gates(wl: Workload, layer: Layer, step: int = 0, T: Optional[int] = None):
    """Routing weights g (T x k, float32) for the routed slots: a softmax of
    N(0,1) logits over each token's k slots (they sum to 1 per token)."""
    T = wl.T if T is None else T
    lg = _rng(wl.name, "gates", step).standard_normal((T, layer.spec.k))
    w = np.exp(lg - lg.max(axis=1, keepdims=True))
    return (w / w.sum(axis=1, keepdims=True)).astype(np.float32)


def make_batch(wl: Workload, layer: Layer, step: int = 0, T: Optional[int] = None):
    """Activations x (T x din, float16) and routing ids (T x k, int32)."""
    spec = layer.spec
    T = wl.T if T is None else T
    rx = _rng(wl.name, "x", step)
    x = rx.standard_normal((T, spec.din))
    if layer.outlier_channels.size:
        x[:, layer.outlier_channels] *= spec.outlier_scale
    x = x.astype(np.float16)
    rr = _rng(wl.name, "ids", step)
    if wl.routing[0] == "uniform":
        keys = rr.random((T, spec.E))
        ids = np.argsort(keys, axis=1, kind="stable")[:, :spec.k]
    elif wl.routing[0] == "zipf":
        s = float(wl.routing[1])
        rank = np.empty(spec.E, dtype=np.float64)
        rank[_rng(wl.name, "zipf_perm").permutation(spec.E)] = np.arange(1, spec.E + 1)
        w = rank ** (-s)
        u = rr.random((T, spec.E))
        u = np.maximum(u, np.finfo(np.float64).tiny)
        keys = np.log(u) / w[None, :]
        ids = np.argsort(-keys, axis=1, kind="stable")[:, :spec.k]
    else:
        raise ValueError(wl.routing)
    return x, ids.astype(np.int32)
