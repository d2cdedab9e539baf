"""ctypes loader for the in-tree HIP library ``libhashenc.so``.

There is no fallback: if the library has not been built, importing the binding raises.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libhashenc.so")

HASHENC_OK = 0
HASHENC_EINVAL = -1
HASHENC_EALIGN = -2
HASHENC_ENOMEM = -3
HASHENC_EHIP = -4
HASHENC_EUNSUPPORTED = -5

HASHENC_DLINEAR = 0
HASHENC_HERMITE = 1
HASHENC_RBF = 2
HASHENC_D2_LAPLACIAN = 1
HASHENC_D2_DIAG = 2
MAX_LEVELS = 32


class HashencConfig(ctypes.Structure):
    _fields_ = [
        ("d", ctypes.c_int32),
        ("n_levels", ctypes.c_int32),
        ("n_features", ctypes.c_int32),
        ("kind", ctypes.c_int32),
        ("d2_mode", ctypes.c_int32),
        ("n_min", ctypes.c_int32),
        ("n_max", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
        ("growth", ctypes.c_double),
        ("table_size", ctypes.c_uint32 * 5),
        ("resolutions", ctypes.POINTER(ctypes.c_int32)),
        ("rbf_eps", ctypes.c_double),
        ("rbf_rings", ctypes.c_int32),
        ("reserved2", ctypes.c_int32),
    ]


class HashencMlp(ctypes.Structure):
    _fields_ = [
        ("in_", ctypes.c_int32),
        ("hidden", ctypes.c_int32),
        ("depth", ctypes.c_int32),
        ("out", ctypes.c_int32),
        ("omega", ctypes.c_float),
        ("reserved", ctypes.c_int32),
    ]


# (name, restype, argtypes) of every exported entry point.
P = ctypes.c_void_p
I32 = ctypes.c_int32
I64 = ctypes.c_int64
SIGNATURES = [
    ("hashenc_create", ctypes.c_int, [ctypes.POINTER(HashencConfig), ctypes.POINTER(P)]),
    ("hashenc_destroy", None, [P]),
    ("hashenc_info", ctypes.c_int, [P, ctypes.POINTER(I64), ctypes.POINTER(I32), P]),
    ("hashenc_derive_active", ctypes.c_int, [P, I32, ctypes.POINTER(P)]),
    ("hashenc_active_levels", ctypes.c_int, [P, ctypes.POINTER(I32)]),
    ("hashenc_c2f_active_levels", ctypes.c_int, [I32, I32, I64, I64, ctypes.POINTER(I32)]),
    ("hashenc_param_layout", ctypes.c_int,
     [P, I32, I32, ctypes.POINTER(I64), ctypes.POINTER(I64), ctypes.POINTER(I32), ctypes.POINTER(I32)]),
    ("hashenc_forward", ctypes.c_int, [P, I64, P, P, P, P, P, P]),
    ("hashenc_forward_workspace_size", ctypes.c_int, [P, I64, ctypes.POINTER(ctypes.c_size_t)]),
    ("hashenc_forward_ws", ctypes.c_int, [P, I64, P, P, P, P, P, P, ctypes.c_size_t, P]),
    ("hashenc_diag_forward_packed", ctypes.c_int, [P, I64, P, P, P, P, P, P, ctypes.c_size_t, P]),
    ("hashenc_backward", ctypes.c_int, [P, I64, P, P, P, P, P, P]),
    ("hashenc_backward_workspace_size", ctypes.c_int, [P, I64, ctypes.POINTER(ctypes.c_size_t)]),
    ("hashenc_backward_ws", ctypes.c_int, [P, I64, P, P, P, P, P, P, ctypes.c_size_t, P]),
    ("hashenc_backward_noalloc", ctypes.c_int, [P, I64, P, P, P, P, P, P]),
    ("hashenc_forward_counting", ctypes.c_int, [P, I64, P, P, P, P, P, P, ctypes.c_size_t, P, ctypes.c_size_t, P]),
    ("hashenc_backward_counted", ctypes.c_int, [P, I64, P, P, P, P, P, P, ctypes.c_size_t, P]),
    ("hashenc_residual_workspace_size", ctypes.c_int,
     [P, ctypes.POINTER(HashencMlp), I64, ctypes.POINTER(ctypes.c_size_t)]),
    ("hashenc_residual", ctypes.c_int,
     [P, ctypes.POINTER(HashencMlp), I64, P, P, P, P, P, P, P, P, ctypes.c_size_t, P]),
    ("hashenc_fd_residual_workspace_size", ctypes.c_int,
     [P, ctypes.POINTER(HashencMlp), I64, ctypes.POINTER(ctypes.c_size_t)]),
    ("hashenc_fd_residual", ctypes.c_int,
     [P, ctypes.POINTER(HashencMlp), ctypes.c_float, I64, P, P, P, P, P, P, P, P, P, ctypes.c_size_t, P]),
    ("hashenc_last_error", ctypes.c_char_p, []),
    ("hashenc_debug_indices", ctypes.c_int, [P, I64, P, I32, P, P]),
    ("hashenc_diag_binned_workspace_size", ctypes.c_int, [P, I64, ctypes.POINTER(ctypes.c_size_t)]),
    ("hashenc_diag_backward_binned", ctypes.c_int, [P, I64, P, P, P, P, P, P, ctypes.c_size_t, P]),
    ("hashenc_diag_copy", ctypes.c_int, [P, P, I64, P]),
    ("hashenc_diag_cache_read", ctypes.c_int, [P, I64, I32, P, P]),
]

_lib = None


def load() -> ctypes.CDLL:
    """Load the built library (raises if it is missing)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"HIP library not built: {LIB_PATH} is missing "
                "(run `python -m multiresolution_hash_grid_multires_amd.build`)")
        lib = ctypes.CDLL(LIB_PATH)
        for name, res, args in SIGNATURES:
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


class HashencError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"hashenc error {code}: {message}")
        self.code = code


def check(code: int) -> None:
    if code != HASHENC_OK:
        msg = load().hashenc_last_error()
        raise HashencError(code, msg.decode() if msg else "")
