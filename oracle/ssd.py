"""Shared-basis spectral decomposition (SSD) and dense reconstruction.

Source: BitsMoE blog note, "Methodology / first split": for one linear type
(gate_proj or up_proj, each W_e in R^{dout x din}) the E expert matrices are
stacked, W_cat = [W_1; ...; W_E] (read as vertical stacking, (E dout) x din,
the only orientation whose right factor lives in the shared input space), one
SVD W_cat = U Sigma Phi^T is taken, and P = U Sigma so that W_e = P_e Phi^T
with P_e the e-th block of dout rows.  "second split": the columns of P_e are
normalised, W_e = sum_k a_{e,k} p_{e,k} phi_k^T with ||p_{e,k}||_2 = 1.

Pinned by tests/test_oracle_path.py (test_ssd_reconstruction_and_structure): reconstruction of random dense W_e (which
is independent input, not built from factors) to 1e-5 relative in fp32
factors; orthonormality of Phi; unit columns; the singular values match
numpy's ``svdvals`` of the stacked matrix.
"""
import numpy as np


def ssd(W: np.ndarray, r: int = None):
    """W: E x dout x din.  Returns (phi din x r, a E x r, p E x r x dout)."""
    W = np.asarray(W, dtype=np.float64)
    E, dout, din = W.shape
    Wcat = W.reshape(E * dout, din)
    U, S, Vt = np.linalg.svd(Wcat, full_matrices=False)
    r = S.size if r is None else r
    phi = Vt[:r].T                       # din x r
    P = (U[:, :r] * S[None, :r]).reshape(E, dout, r)
    a = np.sqrt(np.einsum("edk,edk->ek", P, P))
    p = np.zeros((E, r, dout), dtype=np.float64)
    for e in range(E):
        for k in range(r):
            if a[e, k] > 0:
                p[e, k] = P[e, :, k] / a[e, k]
            else:
                p[e, k, 0] = 1.0         # any unit vector; a = 0 removes it
    return phi, a, p


def reconstruct(phi: np.ndarray, a: np.ndarray, p: np.ndarray) -> np.ndarray:
    """W_e = sum_k a_{e,k} p_{e,k} phi_k^T, summed k ascending in float64."""
    phi = np.asarray(phi, dtype=np.float64)
    a = np.asarray(a, dtype=np.float64)
    p = np.asarray(p, dtype=np.float64)
    E, r, dout = p.shape
    W = np.zeros((E, dout, phi.shape[0]), dtype=np.float64)
    for e in range(E):
        for k in range(r):
            W[e] += a[e, k] * np.outer(p[e, k], phi[:, k])
    return W
