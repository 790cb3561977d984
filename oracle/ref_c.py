"""ctypes front of the plain C oracle (oracle/ref_decode.c, built into
oracle/libbref.so by oracle/build_ref.py).  Test infrastructure only: the
tests and the benchmark's CPU baseline use it."""
import ctypes
import os

import numpy as np

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libbref.so")
_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise OSError("%s is not built (oracle/build_ref.py)" % LIB_PATH)
        L = ctypes.CDLL(LIB_PATH)
        vp, sz, i = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
        L.bref_unpack_expert.argtypes = [vp, sz, i, i, i, i, vp]
        L.bref_unpack_expert.restype = i
        L.bref_gateup.argtypes = [vp, sz, vp, sz, vp, vp, vp, i, i, i, i, i, i, i, vp]
        L.bref_gateup.restype = i
        _lib = L
    return _lib


def _ptr(a):
    return a.ctypes.data


def unpack_expert(blob, E, dout, r, e):
    """r x dout uint16 codes of expert e (0 for 0-bit columns)."""
    blob = np.ascontiguousarray(np.frombuffer(bytes(blob), np.uint8) if not
                                isinstance(blob, np.ndarray) else blob, dtype=np.uint8)
    out = np.zeros((r, dout), np.uint16)
    if lib().bref_unpack_expert(_ptr(blob), blob.nbytes, E, dout, r, e, _ptr(out)):
        raise ValueError("blob does not check")
    return out


def gateup(blob_g, blob_u, phi_t_f16, x_f16, ids, E, dout, r, threads=1):
    """h (T x k x dout float64) from the packed blobs, Phi^T (2r x din fp16:
    gate rows then up rows) and x (T x din fp16)."""
    bg = np.ascontiguousarray(blob_g, dtype=np.uint8)
    bu = np.ascontiguousarray(blob_u, dtype=np.uint8)
    phi = np.ascontiguousarray(phi_t_f16, dtype=np.float16)
    x = np.ascontiguousarray(x_f16, dtype=np.float16)
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    T, k = ids.shape
    din = x.shape[1]
    assert phi.shape == (2 * r, din)
    h = np.empty((T, k, dout), np.float64)
    if lib().bref_gateup(_ptr(bg), bg.nbytes, _ptr(bu), bu.nbytes, _ptr(phi), _ptr(x), _ptr(ids),
                         T, k, E, din, dout, r, int(threads), _ptr(h)):
        raise MemoryError("bref_gateup")
    return h
