"""ctypes binding of libbitsmoe.so (declared in include/bitsmoe.h).

Argument marshalling only: every device step runs in the library's gfx950
kernels.  Device buffers are torch tensors (torch provides memory and
streams); host buffers are numpy arrays.  There is no fallback: if the
library is missing, importing this module raises.
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libbitsmoe.so")

OK, EINVAL, ESHAPE, EBITS, ENOSPC, EFORMAT, EHIP = 0, -1, -2, -3, -4, -5, -6


class BitsMoEError(RuntimeError):
    def __init__(self, status, detail):
        super().__init__("%s (status %d): %s" % (_strerror(status), status, detail))
        self.status = status
        self.detail = detail


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError("libbitsmoe.so is not built (%s); run "
                          "`python -m spectral_expert_gemv_amd.build`" % LIB_PATH)
    # One HIP runtime per process: torch ships its own libamdhip64 under the
    # same soname as ROCm's, and the library's launches must run in the
    # runtime that owns torch's device memory and streams.  Importing torch
    # first makes the library's libamdhip64.so.7 dependency resolve to
    # torch's copy (loaded the other way round, the library's first launch
    # finds no device).
    import torch  # noqa: F401
    return ctypes.CDLL(LIB_PATH)


_lib = _load()

_vp, _sz, _i = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
_pi = ctypes.POINTER(ctypes.c_int)
_psz = ctypes.POINTER(ctypes.c_size_t)

_SIGS = {
    "bitsmoe_version": ([], _i),
    "bitsmoe_strerror": ([_i], ctypes.c_char_p),
    "bitsmoe_last_error_detail": ([], ctypes.c_char_p),
    "bitsmoe_pack_size": ([_i, _i, _i, _vp, _psz], _i),
    "bitsmoe_pack": ([_i, _i, _i, _vp, _vp, _vp, _vp, _sz], _i),
    "bitsmoe_blob_check": ([_vp, _sz, _pi, _pi, _pi], _i),
    "bitsmoe_spectral_proj": ([_vp, _vp, _vp, _i, _i, _i, _vp], _i),
    "bitsmoe_expert_apply": ([_vp, _sz, _i, _i, _i, _vp, _i, _vp, _i, _i, _vp, _vp, _sz, _vp], _i),
    "bitsmoe_moe_gateup_workspace_size": ([_i, _i, _i, _i, _i, _i, _psz], _i),
    "bitsmoe_moe_gateup": ([_vp, _sz, _vp, _sz, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i,
                            _vp, _vp, _sz, _vp], _i),
    "bitsmoe_moe_gateup_noalloc": ([_vp, _sz, _vp, _sz, _vp, _vp, _vp, _i, _i, _i, _i, _i,
                                    _i, _vp, _vp], _i),
    "bitsmoe_workspace_init": ([_vp, _sz, _vp], _i),
    "bitsmoe_dump_codes": ([_vp, _sz, _i, _i, _i, _i, _i, _vp, _vp], _i),
    "bitsmoe_debug_set_wait_limit": ([ctypes.c_uint32], ctypes.c_uint32),
    "bitsmoe_wait_timeouts": ([_vp, _sz, ctypes.POINTER(ctypes.c_uint32), _vp], _i),
    "bitsmoe_pack_device_workspace_size": ([_i, _i, _i, _vp, _psz], _i),
    "bitsmoe_pack_device": ([_i, _i, _i, _vp, _vp, _vp, _vp, _sz, _vp, _sz, _vp], _i),
    "bitsmoe_fqcm_distortion": ([_vp, _i, _i, _i, _vp, _vp], _i),
    "bitsmoe_fqcm_beta": ([_vp, _i, _vp, _vp, _i, _i, _i, _i, _vp, _vp], _i),
    "bitsmoe_fqcm_allocate": ([_vp, _vp, _vp, _i, _i, _i, ctypes.c_uint64, _vp,
                               ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_uint64),
                               ctypes.POINTER(ctypes.c_double), _vp, _sz, _vp], _i),
    "bitsmoe_moe_down_workspace_size": ([_i, _i, _i, _i, _i, _i, _psz], _i),
    "bitsmoe_moe_down": ([_vp, _sz, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _vp, _vp, _sz,
                          _vp], _i),
    "bitsmoe_ssd_workspace_size": ([_i, _i, _i, _i, _psz], _i),
    "bitsmoe_ssd": ([_vp, _i, _i, _i, _i, _vp, _vp, _vp, _vp, _pi, _i, _vp, _sz, _vp], _i),
}
FQCM_WS_BYTES = 1024 + 65536 * 24
for _name, (_args, _res) in _SIGS.items():
    _f = getattr(_lib, _name)
    _f.argtypes = _args
    _f.restype = _res

EXPORTS = tuple(_SIGS)


def _strerror(status):
    return _lib.bitsmoe_strerror(int(status)).decode()


def _check(status):
    if status != OK:
        raise BitsMoEError(status, _lib.bitsmoe_last_error_detail().decode())


def version():
    return _lib.bitsmoe_version()


def _ptr(t):
    """Device pointer of a torch tensor or host pointer of a numpy array."""
    if t is None:
        return None
    if isinstance(t, np.ndarray):
        return t.ctypes.data
    return t.data_ptr()


def _nbytes(t):
    if isinstance(t, np.ndarray):
        return t.nbytes
    return t.numel() * t.element_size()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


# ---------------------------------------------------------------- host side

def pack_size(E, dout, r, bits):
    bits = np.ascontiguousarray(bits, dtype=np.uint8)
    out = ctypes.c_size_t(0)
    _check(_lib.bitsmoe_pack_size(E, dout, r, bits.ctypes.data, ctypes.byref(out)))
    return out.value


def pack(p, a, bits):
    """Quantize and pack one linear type (p: E x r x dout, a, bits: E x r)."""
    p = np.ascontiguousarray(p, dtype=np.float32)
    a = np.ascontiguousarray(a, dtype=np.float32)
    bits = np.ascontiguousarray(bits, dtype=np.uint8)
    E, r, dout = p.shape
    if a.shape != (E, r) or bits.shape != (E, r):
        raise ValueError("a and bits must be E x r")
    n = pack_size(E, dout, r, bits)
    out = np.zeros(n, dtype=np.uint8)
    _check(_lib.bitsmoe_pack(E, dout, r, p.ctypes.data, a.ctypes.data, bits.ctypes.data,
                             out.ctypes.data, out.nbytes))
    return out


def blob_check(blob):
    blob = np.ascontiguousarray(blob, dtype=np.uint8)
    E, dout, r = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
    _check(_lib.bitsmoe_blob_check(blob.ctypes.data, blob.nbytes, ctypes.byref(E),
                                   ctypes.byref(dout), ctypes.byref(r)))
    return E.value, dout.value, r.value


# -------------------------------------------------------------- device side

def spectral_proj(phi_t, x, z, stream=None):
    """z[T, R] = x[T, din] @ phi_t[R, din]^T (phi_t, x fp16; z float32)."""
    R, din = phi_t.shape
    T = x.shape[0]
    _check(_lib.bitsmoe_spectral_proj(_ptr(phi_t), _ptr(x), _ptr(z), T, din, R,
                                      _stream(stream)))


def expert_apply(packed, E, dout, r, z, ids, y, z_stride=None, ws=None, stream=None):
    T, k = ids.shape
    zs = z.shape[1] if z_stride is None else z_stride
    _check(_lib.bitsmoe_expert_apply(_ptr(packed), _nbytes(packed), E, dout, r, _ptr(z), zs,
                                     _ptr(ids), T, k, _ptr(y), _ptr(ws),
                                     0 if ws is None else _nbytes(ws), _stream(stream)))


def moe_gateup_workspace_size(T, k, E, din, dout, r):
    out = ctypes.c_size_t(0)
    _check(_lib.bitsmoe_moe_gateup_workspace_size(T, k, E, din, dout, r, ctypes.byref(out)))
    return out.value


def moe_gateup(packed_gate, packed_up, phi_t_gateup, x, ids, E, dout, r, h, ws, stream=None):
    T, k = ids.shape
    din = x.shape[1]
    _check(_lib.bitsmoe_moe_gateup(_ptr(packed_gate), _nbytes(packed_gate), _ptr(packed_up),
                                   _nbytes(packed_up), _ptr(phi_t_gateup), _ptr(x), _ptr(ids),
                                   T, k, E, din, dout, r, _ptr(h), _ptr(ws), _nbytes(ws),
                                   _stream(stream)))


# bytes of the static workspace behind moe_gateup_noalloc
GATEUP_NOALLOC_MAX_WS = 64 << 20


def moe_gateup_noalloc(packed_gate, packed_up, phi_t_gateup, x, ids, E, dout, r, h,
                       stream=None):
    """moe_gateup on the library's static per-device workspace (no workspace
    argument; calls that overlap in time on one device race)."""
    T, k = ids.shape
    din = x.shape[1]
    _check(_lib.bitsmoe_moe_gateup_noalloc(_ptr(packed_gate), _nbytes(packed_gate),
                                           _ptr(packed_up), _nbytes(packed_up),
                                           _ptr(phi_t_gateup), _ptr(x), _ptr(ids), T, k, E,
                                           din, dout, r, _ptr(h), _stream(stream)))


def workspace_init(ws, stream=None):
    _check(_lib.bitsmoe_workspace_init(_ptr(ws), _nbytes(ws), _stream(stream)))


def debug_set_wait_limit(spins):
    """Sets the bound on the one-launch gate/up kernel's waits for z (0: give
    up at once, every row NaN); returns the previous bound.  Test hook."""
    return int(_lib.bitsmoe_debug_set_wait_limit(int(spins)))


def wait_timeouts(ws=None, stream=None):
    """Waits of the one-launch gate/up kernels that gave up (rows written as
    NaN) since the workspace was zero-filled; ws=None reads the static
    workspace of moe_gateup_noalloc.  Synchronises the stream."""
    n = ctypes.c_uint32(0)
    if ws is None:
        _check(_lib.bitsmoe_wait_timeouts(None, 0, ctypes.byref(n), _stream(stream)))
    else:
        _check(_lib.bitsmoe_wait_timeouts(_ptr(ws), _nbytes(ws), ctypes.byref(n),
                                          _stream(stream)))
    return int(n.value)


DUMP_I8, DUMP_F16, DUMP_LANE = 0, 1, 2


def dump_codes(packed, E, dout, r, e, codes, path=DUMP_LANE, stream=None):
    """Codes of expert e as decoder `path` builds them (DUMP_I8: int8 operand
    bytes of the one-launch kernel; DUMP_F16: fp16 operands of the batched
    kernel; DUMP_LANE: codes of the lane-per-row kernel)."""
    _check(_lib.bitsmoe_dump_codes(_ptr(packed), _nbytes(packed), E, dout, r, e, path,
                                   _ptr(codes), _stream(stream)))


def pack_device_workspace_size(E, dout, r, bits):
    bits = np.ascontiguousarray(bits, dtype=np.uint8)
    out = ctypes.c_size_t(0)
    _check(_lib.bitsmoe_pack_device_workspace_size(E, dout, r, bits.ctypes.data,
                                                   ctypes.byref(out)))
    return out.value


def pack_device(p, a, bits, out=None, ws=None, stream=None):
    """Quantize and pack one linear type on the GPU.  p: E x r x dout and a:
    E x r float32 device tensors; bits: E x r host widths.  Returns the blob as
    a uint8 device tensor (`out` if given); the call returns once it is
    complete."""
    import torch
    bits = np.ascontiguousarray(bits, dtype=np.uint8)
    E, r, dout = p.shape
    if tuple(a.shape) != (E, r) or bits.shape != (E, r):
        raise ValueError("a and bits must be E x r")
    if p.dtype != torch.float32 or a.dtype != torch.float32:
        raise ValueError("p and a must be float32")
    if not (p.is_contiguous() and a.is_contiguous()):
        raise ValueError("p and a must be contiguous")
    if out is None:
        out = torch.empty(pack_size(E, dout, r, bits), dtype=torch.uint8, device=p.device)
    if ws is None:
        ws = torch.empty(pack_device_workspace_size(E, dout, r, bits), dtype=torch.uint8,
                         device=p.device)
    _check(_lib.bitsmoe_pack_device(E, dout, r, _ptr(p), _ptr(a), bits.ctypes.data, _ptr(out),
                                    _nbytes(out), _ptr(ws), _nbytes(ws), _stream(stream)))
    return out


def fqcm_distortion(p, eps=None, stream=None):
    """eps (E x r x 8 float64 device tensor) of the unit directions p
    (E x r x dout float32 device tensor)."""
    import torch
    E, r, dout = p.shape
    if p.dtype != torch.float32 or not p.is_contiguous():
        raise ValueError("p must be contiguous float32")
    if eps is None:
        eps = torch.empty((E, r, 8), dtype=torch.float64, device=p.device)
    _check(_lib.bitsmoe_fqcm_distortion(_ptr(p), E, r, dout, _ptr(eps), _stream(stream)))
    return eps


def fqcm_beta(z, ids, g, E, beta=None, stream=None):
    """beta (E x r float64) from z (T x r float32, row stride z.stride(0)),
    ids (T x k int32) and routing weights g (T x k float32), device tensors."""
    import torch
    T, r = z.shape
    k = ids.shape[1]
    if z.dtype != torch.float32 or z.stride(1) != 1:
        raise ValueError("z must be float32 with unit column stride")
    if ids.dtype != torch.int32 or g.dtype != torch.float32 or tuple(g.shape) != (T, k):
        raise ValueError("ids must be int32 and g float32, both T x k")
    if beta is None:
        beta = torch.empty((E, r), dtype=torch.float64, device=z.device)
    _check(_lib.bitsmoe_fqcm_beta(_ptr(z), z.stride(0), _ptr(ids.contiguous()),
                                  _ptr(g.contiguous()), T, k, E, r, _ptr(beta), _stream(stream)))
    return beta


def fqcm_allocate(a, beta, eps, dout, budget_bits, bits=None, ws=None, stream=None):
    """Least-loss widths within the bit budget; returns (bits uint8 device
    tensor E x r, the Lagrangian multiplier lam, bits used, loss minus the
    dual bound at lam)."""
    import torch
    E, r = a.shape
    if bits is None:
        bits = torch.empty((E, r), dtype=torch.uint8, device=a.device)
    if ws is None:
        ws = torch.empty(FQCM_WS_BYTES, dtype=torch.uint8, device=a.device)
    lam = ctypes.c_double(0.0)
    used = ctypes.c_uint64(0)
    gap = ctypes.c_double(0.0)
    _check(_lib.bitsmoe_fqcm_allocate(_ptr(a), _ptr(beta), _ptr(eps), E, r, dout,
                                      int(budget_bits), _ptr(bits), ctypes.byref(lam),
                                      ctypes.byref(used), ctypes.byref(gap), _ptr(ws),
                                      _nbytes(ws), _stream(stream)))
    return bits, lam.value, used.value, gap.value


def moe_down_workspace_size(T, k, E, dout, din, r_d):
    out = ctypes.c_size_t(0)
    _check(_lib.bitsmoe_moe_down_workspace_size(T, k, E, dout, din, r_d, ctypes.byref(out)))
    return out.value


def moe_down(packed_down, phi_t_down, h, ids, g, E, din, r_d, out=None, ws=None, stream=None):
    """out (T x din float32) = sum_j g[t, j] * down_e(h[t, j]); h: T x k x
    dout float32, ids: T x k int32, g: T x k float32, phi_t_down: r_d x dout
    fp16, packed_down: the down blob; all device tensors."""
    import torch
    T, k, dout = h.shape
    if h.dtype != torch.float32 or g.dtype != torch.float32 or ids.dtype != torch.int32:
        raise ValueError("h and g must be float32, ids int32")
    h, ids, g = h.contiguous(), ids.contiguous(), g.contiguous()
    if out is None:
        out = torch.empty((T, din), dtype=torch.float32, device=h.device)
    if ws is None:
        ws = torch.empty(moe_down_workspace_size(T, k, E, dout, din, r_d), dtype=torch.uint8,
                         device=h.device)
    _check(_lib.bitsmoe_moe_down(_ptr(packed_down), _nbytes(packed_down), _ptr(phi_t_down),
                                 _ptr(h), _ptr(ids), _ptr(g), T, k, E, dout, din, r_d, _ptr(out),
                                 _ptr(ws), _nbytes(ws), _stream(stream)))
    return out


def ssd_workspace_size(E, dout, din, r):
    out = ctypes.c_size_t(0)
    _check(_lib.bitsmoe_ssd_workspace_size(E, dout, din, r, ctypes.byref(out)))
    return out.value


def ssd(W, r, max_sweeps=30, ws=None, stream=None):
    """Shared-basis decomposition of W (E x dout x din float32 device tensor).
    Returns (phi din x r, a E x r, p E x r x dout) device float32 tensors,
    sigma^2 (numpy float64, r) and the Jacobi sweeps taken."""
    import torch
    E, dout, din = W.shape
    if W.dtype != torch.float32 or not W.is_contiguous():
        raise ValueError("W must be contiguous float32")
    phi = torch.empty((din, r), dtype=torch.float32, device=W.device)
    a = torch.empty((E, r), dtype=torch.float32, device=W.device)
    p = torch.empty((E, r, dout), dtype=torch.float32, device=W.device)
    if ws is None:
        ws = torch.empty(ssd_workspace_size(E, dout, din, r), dtype=torch.uint8, device=W.device)
    s2 = np.zeros(r, dtype=np.float64)
    sw = ctypes.c_int(0)
    _check(_lib.bitsmoe_ssd(_ptr(W), E, dout, din, r, _ptr(phi), _ptr(a), _ptr(p),
                            s2.ctypes.data, ctypes.byref(sw), int(max_sweeps), _ptr(ws),
                            _nbytes(ws), _stream(stream)))
    return phi, a, p, s2, sw.value
