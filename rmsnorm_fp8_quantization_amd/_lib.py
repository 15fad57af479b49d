"""ctypes view of ``libnormfp8.so`` with the same names as the C ABI (include/normfp8.h).

Argument marshalling only: every computation happens in the HIP kernels behind these
entry points. Loading fails loudly if the library has not been built; there is no
fallback implementation.
"""
from __future__ import annotations

import contextlib
import ctypes
import os
import threading

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libnormfp8.so")

# status codes (norm_status_t)
NORM_OK, NORM_ERR_INVALID_ARG, NORM_ERR_UNSUPPORTED, NORM_ERR_MISALIGNED, \
    NORM_ERR_WORKSPACE_TOO_SMALL, NORM_ERR_HIP = range(6)
# enums
NORM_LAYERNORM, NORM_RMSNORM = 0, 1
NORM_F32, NORM_F16, NORM_BF16, NORM_FP8_E4M3, NORM_FP8_E5M2 = range(5)
NORM_SCALING_NONE, NORM_SCALING_DELAYED_TENSOR, NORM_SCALING_MXFP8_1D32, NORM_SCALING_MXFP8_1D32_CEIL = range(4)
NORM_Q_ROWWISE, NORM_Q_COLWISE, NORM_Q_ROWWISE_COLWISE, NORM_Q_COLWISE_ROWMAJOR = 1, 2, 3, 4
NORM_Q_SCALES_PADDED = 8
(NORM_ROUTE_ROW, NORM_ROUTE_ROW_TRANSPOSE, NORM_ROUTE_STATS_TILES, NORM_ROUTE_BAND, NORM_ROUTE_SPLIT,
 NORM_ROUTE_SINGLE_PASS_COLWISE, NORM_ROUTE_GENERAL) = range(7)
NORM_WS_HEADER_BYTES = 16384

EXPORTS = ("norm_fwd_workspace_size", "norm_bwd_workspace_size", "norm_fwd", "norm_bwd",
           "norm_bwd_add", "norm_bwd_noalloc", "norm_workspace_init", "norm_workspace_check", "norm_bwd_launch_shape",
           "norm_fwd_launch_shape",
           "norm_tuning_set", "norm_last_error", "norm_abi_version")
ABI_VERSION = 2
KNOB_UNSET = -2 ** 31  # INT_MIN: a tuning override that is not set

_P = ctypes.c_void_p
_I = ctypes.c_int
_I64 = ctypes.c_int64
_F = ctypes.c_float
_SZ = ctypes.c_size_t

_SIGS = {
    "norm_fwd_workspace_size": [_I64, _I64, _I, _I, _I, _I, _I, _I, _I, _F, _I, _I, ctypes.POINTER(_SZ)],
    "norm_bwd_workspace_size": [_I64, _I64, _I, _I, _I, _I, _F, _I, _I, ctypes.POINTER(_SZ)],
    "norm_fwd": [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _SZ,
                 _I64, _I64, _I, _I, _I, _I, _I, _I, _I, _F, _I],
    "norm_bwd": [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _I64, _I64, _I, _I, _I, _I, _I],
    "norm_bwd_add": [_P, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _I64, _I64, _I, _I, _I, _I],
    "norm_bwd_noalloc": [_P, _P, _P, _P, _P, _P, _P, _P, _P, _I64, _I64, _I, _I, _I, _I, _I],
    "norm_workspace_init": [_P, _P, _SZ],
    "norm_workspace_check": [_P, _P, ctypes.POINTER(ctypes.c_uint32)],
    "norm_bwd_launch_shape": [_I64, _I64, _I, _I, _I, _I, _I, _I, _I, ctypes.POINTER(_I64)],
    "norm_fwd_launch_shape": [_I64, _I64, _I, _I, _I, _I, _I, _I, _I, ctypes.POINTER(_I64)],
    "norm_tuning_set": [ctypes.c_char_p, _I, ctypes.POINTER(_I)],
    "norm_last_error": [],
    "norm_abi_version": [],
}

_lib = None
_lock = threading.Lock()


class NormError(RuntimeError):
    def __init__(self, fn, code, msg):
        super().__init__(f"{fn} failed with status {code}: {msg}")
        self.code = code


def load():
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise ImportError(
                    f"{LIB_PATH} is missing: build it with `python -m rmsnorm_fp8_quantization_amd.build` "
                    "(the HIP library is required; there is no fallback path)")
            lib = ctypes.CDLL(LIB_PATH)
            for name, args in _SIGS.items():
                fn = getattr(lib, name)
                fn.argtypes = args
                fn.restype = ctypes.c_char_p if name == "norm_last_error" else ctypes.c_int
            _lib = lib
    return _lib


def call(name, *args):
    """Call an entry point; raise NormError with norm_last_error() on a non-zero status."""
    lib = load()
    rc = getattr(lib, name)(*args)
    if rc != NORM_OK:
        raise NormError(name, rc, lib.norm_last_error().decode())
    return rc


@contextlib.contextmanager
def tuning(**knobs):
    """Set planner overrides (``NORMFP8_ROW_CFG=3``, ...) for the duration of a block, through
    ``norm_tuning_set``, and restore the previous values afterwards."""
    prev = {}
    try:
        for name, value in knobs.items():
            old = _I(0)
            call("norm_tuning_set", name.encode(), int(value), ctypes.byref(old))
            prev[name] = old.value
        yield
    finally:
        for name, value in prev.items():
            call("norm_tuning_set", name.encode(), value, None)


def status(name, *args):
    """Call an entry point and return its status code (no exception)."""
    return getattr(load(), name)(*args)
