"""MI355X-native spectral MoE gate/up decode path (BitsMoE).

The compute lives in ``libbitsmoe.so`` (hand-written gfx950 HIP kernels
behind a C ABI, ``include/bitsmoe.h``); ``bitsmoe`` is its ctypes binding and
``layer`` keeps a packed layer resident in device memory.
"""
from . import bitsmoe  # noqa: F401  (raises ImportError if the library is not built)
from .layer import DeviceLayer  # noqa: F401

__all__ = ["bitsmoe", "DeviceLayer"]
