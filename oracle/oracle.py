"""ctypes wrapper around the plain C oracle (``hashgrid_oracle.c``).

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py``.  It imports nothing from the HIP package and the HIP
package imports nothing from here.

Every function takes a plain configuration ``spec`` (a dict) and host NumPy arrays and
returns fp64 NumPy arrays.  The spec keys are:

    d, L, F           dimension (1..4; 4 for the space-time Hermite grid), number of levels,
                      features per slot
    kind              "dlinear" (Instant-NGP d-linear), "hermite" (Hermite-NGP) or "rbf"
                      (DInf-Grid Gaussian RBF; rbf_eps = epsilon, rbf_rings = k)
    T                 list of table sizes, one per derivative order (d-linear: [T])
    n_min, n_max      coarsest / finest resolution (geometric progression)
    growth            optional per-level growth factor b (overrides n_max)
    resolutions       optional explicit list of N_l
    d2_mode           "laplacian" or "diag" (Hermite second-order output)
    active_levels     optional number of active levels (coarse-to-fine schedule: levels
                      l >= active_levels encode to zero and receive no gradient)
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "hashgrid_oracle.c")
# HASHGRID_ORACLE_LIB points the wrapper at another build of the same source (used to check,
# on the CPU, that the pins catch mistakes planted in a copy of the oracle).
_LIB = os.environ.get("HASHGRID_ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")
# The same source built with -DORC_FP32: the per-point arithmetic after the position stage in
# fp32 (its outputs measure the fp32 rounding floor; it is not a reference).
_LIB32 = os.path.join(_HERE, "liboracle_f32.so")

MAX_LEVELS = 32
MAX_D = 4


GCC_FLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-fPIC", "-shared", "-Wall"]


def build_oracle(force: bool = True, out: str | None = None, extra_flags: list[str] | None = None,
                 src: str | None = None) -> str:
    """Compile the oracle with gcc (plain IEEE arithmetic: no fast-math, no contraction), and
    its fp32 working-precision build beside it.  `out`, `extra_flags` and `src` build one
    other variant instead (a sanitizer build, or a planted-mistake copy in a test)."""
    if out is not None:
        tmp = out + ".tmp"
        subprocess.check_call(["gcc", *GCC_FLAGS, *(extra_flags or []), "-o", tmp, src or _SRC, "-lm"])
        os.replace(tmp, out)
        return out
    for lib, flags in ((_LIB, []), (_LIB32, ["-DORC_FP32"])):
        if force or not os.path.exists(lib):
            tmp = lib + ".tmp"
            subprocess.check_call(["gcc", *GCC_FLAGS, *flags, "-o", tmp, _SRC, "-lm"])
            os.replace(tmp, lib)
    return _LIB


class _Cfg(ctypes.Structure):
    _fields_ = [
        ("d", ctypes.c_int32), ("L", ctypes.c_int32), ("F", ctypes.c_int32),
        ("kind", ctypes.c_int32), ("d2_mode", ctypes.c_int32),
        ("T", ctypes.c_uint32 * (MAX_D + 1)), ("N", ctypes.c_int32 * MAX_LEVELS),
        ("active", ctypes.c_int32), ("rings", ctypes.c_int32), ("eps", ctypes.c_double),
    ]


_libs: dict = {}


def _load(precision: str = "f64"):
    """The oracle library (precision "f64"), or its fp32 working-precision build ("f32")."""
    if precision not in ("f64", "f32"):
        raise ValueError("precision must be 'f64' or 'f32'")
    if precision not in _libs:
        path = _LIB if precision == "f64" else _LIB32
        if not os.path.exists(path):
            build_oracle(force=False)
        lib = ctypes.CDLL(path)
        P = ctypes.c_void_p
        lib.orc_levels.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_double, P]
        lib.orc_levels.restype = ctypes.c_int
        lib.orc_layout.argtypes = [P, P, P, P, P]
        lib.orc_layout.restype = ctypes.c_int64
        lib.orc_hash.argtypes = [ctypes.c_int, P]
        lib.orc_hash.restype = ctypes.c_uint32
        lib.orc_indices.argtypes = [P, ctypes.c_int64, P, ctypes.c_int, P]
        lib.orc_indices.restype = None
        lib.orc_forward.argtypes = [P, ctypes.c_int64, P, P, P, P, P]
        lib.orc_forward.restype = None
        lib.orc_backward_f64.argtypes = [P, ctypes.c_int64, P, P, P, P, P]
        lib.orc_backward_f64.restype = None
        lib.orc_residual.argtypes = [P, ctypes.c_int32, ctypes.c_int32, ctypes.c_double,
                                     ctypes.c_int64, P, P, P, P, P, P, P, P, P, P]
        lib.orc_residual.restype = ctypes.c_int
        lib.orc_fd_residual.argtypes = [P, ctypes.c_int32, ctypes.c_int32, ctypes.c_double, ctypes.c_double,
                                        ctypes.c_int64, P, P, P, P, P, P, P, P]
        lib.orc_fd_residual.restype = ctypes.c_int
        lib.orc_mlp_param_count.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32]
        lib.orc_mlp_param_count.restype = ctypes.c_int64
        lib.orc_c2f_active.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int64, ctypes.c_int64]
        lib.orc_c2f_active.restype = ctypes.c_int32
        lib.orc_max_threads.argtypes = []
        lib.orc_max_threads.restype = ctypes.c_int
        lib.orc_set_threads.argtypes = [ctypes.c_int]
        lib.orc_set_threads.restype = None
        _libs[precision] = lib
    return _libs[precision]


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def levels(L: int, n_min: int, n_max: int = 0, growth: float | None = None) -> list[int]:
    out = np.zeros(L, dtype=np.int32)
    rc = _load().orc_levels(L, n_min, n_max, float(growth or 0.0), _ptr(out))
    if rc != 0:
        raise ValueError("bad level specification")
    return [int(v) for v in out]


def resolutions(spec: dict) -> list[int]:
    if spec.get("resolutions") is not None:
        return [int(v) for v in spec["resolutions"]]
    return levels(spec["L"], spec["n_min"], spec.get("n_max", 0), spec.get("growth"))


def n_tables(spec: dict) -> int:
    return spec["d"] + 1 if spec["kind"] == "hermite" else 1


def make_cfg(spec: dict) -> _Cfg:
    c = _Cfg()
    c.d, c.L, c.F = spec["d"], spec["L"], spec["F"]
    if not (1 <= c.d <= MAX_D and 1 <= c.L <= MAX_LEVELS and 1 <= c.F <= 8):
        raise ValueError("unsupported shape")
    c.kind = {"dlinear": 0, "hermite": 1, "rbf": 2}[spec["kind"]]
    if c.kind == 2:
        c.rings, c.eps = int(spec["rbf_rings"]), float(spec["rbf_eps"])
        if not (1 <= c.rings <= 4 and c.eps > 0 and c.d <= 3):
            raise ValueError("rbf_rings must be 1..4, rbf_eps > 0 and d <= 3")
    c.d2_mode = 2 if spec.get("d2_mode", "laplacian") == "diag" else 1
    T = list(spec["T"])
    if len(T) == 1:
        T = T * n_tables(spec)
    for k in range(n_tables(spec)):
        c.T[k] = int(T[k])
    for l, v in enumerate(resolutions(spec)):
        c.N[l] = v
    a = spec.get("active_levels")
    if a is not None and not 1 <= int(a) <= c.L:
        raise ValueError("active_levels outside 1..L")
    c.active = 0 if a is None else int(a)
    return c


def layout(spec: dict) -> dict:
    c = make_cfg(spec)
    nt, L = n_tables(spec), spec["L"]
    offs = np.zeros(nt * L, np.int64)
    rows = np.zeros(nt * L, np.int64)
    width = np.zeros(nt * L, np.int32)
    dense = np.zeros(nt * L, np.int32)
    total = _load().orc_layout(ctypes.byref(c), _ptr(offs), _ptr(rows), _ptr(width), _ptr(dense))
    return {"n_params": int(total), "N": [int(v) for v in c.N[:L]],
            "offset": offs.reshape(nt, L), "rows": rows.reshape(nt, L),
            "width": width.reshape(nt, L), "dense": dense.reshape(nt, L).astype(bool)}


def hash_vertex(v) -> int:
    arr = np.asarray(v, dtype=np.uint32)
    return int(_load().orc_hash(len(arr), _ptr(arr)))


def _f32(a, shape=None):
    a = np.ascontiguousarray(a, dtype=np.float32)
    if shape is not None and a.shape != tuple(shape):
        a = a.reshape(shape)
    return a


def indices(spec: dict, x: np.ndarray, table: int = 0) -> np.ndarray:
    c = make_cfg(spec)
    x = _f32(x)
    n = x.shape[0]
    out = np.zeros((n, spec["L"], 1 << spec["d"]), np.int32)
    _load().orc_indices(ctypes.byref(c), n, _ptr(x), table, _ptr(out))
    return out


def _f64(a):
    return None if a is None else np.ascontiguousarray(a, dtype=np.float64)


def forward(spec: dict, x: np.ndarray, params: np.ndarray, precision: str = "f64"):
    """gamma [n, L*F]; Hermite and RBF add dgamma [n, d, L*F] and d2gamma (Laplacian
    [n, L*F] or diagonal [n, d, L*F]).  Returns (gamma, dgamma, d2gamma), None where not
    defined.  ``params`` may be fp32 (widened exactly) or fp64.  precision "f32": the same
    arithmetic in fp32 (the rounding floor, not a reference)."""
    c = make_cfg(spec)
    x, params = _f32(x), _f64(params)
    n, d, LF = x.shape[0], spec["d"], spec["L"] * spec["F"]
    gamma = np.zeros((n, LF))
    dg = d2 = None
    if spec["kind"] in ("hermite", "rbf"):
        dg = np.zeros((n, d, LF))
        d2 = np.zeros((n, d, LF)) if c.d2_mode == 2 else np.zeros((n, LF))
    _load(precision).orc_forward(ctypes.byref(c), n, _ptr(x), _ptr(params), _ptr(gamma), _ptr(dg), _ptr(d2))
    return gamma, dg, d2


def backward(spec: dict, x: np.ndarray, g_gamma=None, g_dgamma=None, g_d2=None, n_params=None,
             precision: str = "f64"):
    """Gradient of <G, forward(theta)> with respect to theta (fp64, params layout).
    Upstream arrays are fp32 (exactly widened) or fp64; None means zero."""
    c = make_cfg(spec)
    x = _f32(x)
    n = x.shape[0]
    if n_params is None:
        n_params = layout(spec)["n_params"]
    grad = np.zeros(n_params)
    _load(precision).orc_backward_f64(ctypes.byref(c), n, _ptr(x), _ptr(_f64(g_gamma)), _ptr(_f64(g_dgamma)),
                             _ptr(_f64(g_d2)), _ptr(grad))
    return grad


def c2f_active_levels(L: int, L0: int, t: int, tau: int) -> int:
    """Active level count of the coarse-to-fine schedule at step t."""
    a = int(_load().orc_c2f_active(L, L0, t, tau))
    if a < 0:
        raise ValueError("bad coarse-to-fine schedule")
    return a


def max_threads() -> int:
    return int(_load().orc_max_threads())


def set_threads(n: int) -> None:
    """Threads the oracle uses from now on (for timing; results do not depend on it)."""
    _load().orc_set_threads(int(n))


def mlp_param_count(n_in: int, hidden: int, depth: int) -> int:
    return int(_load().orc_mlp_param_count(n_in, hidden, depth))


def residual(spec: dict, hidden: int, depth: int, omega: float, x, params, mlp, precision: str = "f64"):
    """Fused PINN residual.  Returns a dict of fp64 results: u [n], grad_u [n, d], lap_u [n],
    r [n], loss (float), grad_params [n_params], grad_mlp [n_mlp]."""
    c = make_cfg(spec)
    x, params, mlp = _f32(x), _f64(params), _f64(mlp)
    n, d = x.shape[0], spec["d"]
    out = {"u": np.zeros(n), "grad_u": np.zeros((n, d)), "lap_u": np.zeros(n), "r": np.zeros(n),
           "grad_params": np.zeros(params.size), "grad_mlp": np.zeros(mlp.size)}
    loss = np.zeros(1)
    rc = _load(precision).orc_residual(ctypes.byref(c), hidden, depth, float(omega), n, _ptr(x), _ptr(params),
                              _ptr(mlp), _ptr(out["u"]), _ptr(out["grad_u"]), _ptr(out["lap_u"]),
                              _ptr(out["r"]), _ptr(loss), _ptr(out["grad_params"]),
                              _ptr(out["grad_mlp"]))
    if rc != 0:
        raise ValueError("bad residual configuration")
    out["loss"] = float(loss[0])
    return out


def fd_residual(spec: dict, hidden: int, depth: int, omega: float, eps: float, x, params, mlp,
                precision: str = "f64"):
    """INGP-FD comparator: the residual with the Laplacian of u taken by central differences
    over the 2d+1 stencil points (d-linear encoding).  Returns a dict of fp64 results:
    u_stencil [n, 2d+1], r [n], loss (float), grad_params [n_params], grad_mlp [n_mlp]."""
    c = make_cfg(spec)
    x, params, mlp = _f32(x), _f64(params), _f64(mlp)
    n, d = x.shape[0], spec["d"]
    out = {"u_stencil": np.zeros((n, 2 * d + 1)), "r": np.zeros(n),
           "grad_params": np.zeros(params.size), "grad_mlp": np.zeros(mlp.size)}
    loss = np.zeros(1)
    rc = _load(precision).orc_fd_residual(ctypes.byref(c), hidden, depth, float(omega), float(eps), n, _ptr(x),
                                 _ptr(params), _ptr(mlp), _ptr(out["u_stencil"]), _ptr(out["r"]), _ptr(loss),
                                 _ptr(out["grad_params"]), _ptr(out["grad_mlp"]))
    if rc != 0:
        raise ValueError("bad FD residual configuration")
    out["loss"] = float(loss[0])
    return out
