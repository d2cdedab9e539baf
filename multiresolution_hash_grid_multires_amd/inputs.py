"""Seeded synthetic workloads shared by the tests, the benchmark and the smoke check.

This module holds data only: the workload specifications and NumPy generators for
points, table entries, upstream gradients and MLP weights.  It contains none of the
encoding's arithmetic, so both the HIP path and the CPU oracle can be fed from it.

Every array is drawn from ``numpy.random.default_rng(SeedSequence([workload_id, stream]))``
with the streams below, and is float32.
"""
from __future__ import annotations

import math

import numpy as np

STREAM_POINTS, STREAM_TABLES, STREAM_UPSTREAM, STREAM_MLP, STREAM_CLUSTERS, STREAM_DELTA = range(6)

# Workload specifications.  "spec" is the encoder configuration in the plain form that
# both the library binding and the oracle accept.
WORKLOADS: dict[str, dict] = {
    # 2D Instant-NGP d-linear: every level is a dense 1:1 grid (largest level 55^2 <= 2^12).
    "dlinear2d_L4_T12": {
        "id": 1,
        "spec": {"d": 2, "L": 4, "F": 2, "kind": "dlinear", "T": [1 << 12], "n_min": 16,
                 "growth": 1.5},
        "n_points": 4096,
        "tables": ("uniform", 1.0),
        "outputs": ("gamma",),
    },
    # 2D Hermite-NGP: three order tables (f; f_x,f_y; f_xy) of 2^14 rows, N 16..512.
    "hermite2d_L8_T14": {
        "id": 2,
        "spec": {"d": 2, "L": 8, "F": 2, "kind": "hermite", "T": [1 << 14] * 3, "n_min": 16,
                 "n_max": 512, "d2_mode": "laplacian"},
        "n_points": 1 << 16,
        "tables": ("normal", 1e-2),
        "outputs": ("gamma", "dgamma", "d2gamma"),
    },
    # 2D Hermite-NGP with the order-table sizes of the Hermite-NGP ablation's best setting
    # (14-14-10: f and (f_x, f_y) in 2^14 rows, f_xy in 2^10), otherwise as workload 2.
    "hermite2d_L8_T14_14_10": {
        "id": 10,
        "spec": {"d": 2, "L": 8, "F": 2, "kind": "hermite", "T": [1 << 14, 1 << 14, 1 << 10], "n_min": 16,
                 "n_max": 512, "d2_mode": "laplacian"},
        "n_points": 1 << 16,
        "tables": ("normal", 1e-2),
        "outputs": ("gamma", "dgamma", "d2gamma"),
    },
    # 3D Instant-NGP d-linear at the standard size: L=16, F=2, T=2^19, N 16..2048.
    "dlinear3d_L16_T19": {
        "id": 3,
        "spec": {"d": 3, "L": 16, "F": 2, "kind": "dlinear", "T": [1 << 19], "n_min": 16,
                 "n_max": 2048},
        "n_points": 1 << 20,
        "tables": ("uniform", 1e-4),
        "outputs": ("gamma",),
    },
    # 3D Hermite-NGP: four order tables of 2^19 rows (widths F, 3F, 3F, F), N 16..1024,
    # diagonal second derivatives.
    "hermite3d_L16_T19": {
        "id": 4,
        "spec": {"d": 3, "L": 16, "F": 2, "kind": "hermite", "T": [1 << 19] * 4, "n_min": 16,
                 "n_max": 1024, "d2_mode": "diag"},
        "n_points": 1 << 20,
        "tables": ("normal", 1e-2),
        "outputs": ("gamma", "dgamma", "d2gamma"),
    },
    # Fused PINN residual: the 3D Hermite encoding feeding a SIREN 32->64->64->1, omega=30,
    # half the points uniform and half from 8 Gaussian clusters (sigma 0.02).
    "pinn_residual3d": {
        "id": 5,
        "spec": {"d": 3, "L": 16, "F": 2, "kind": "hermite", "T": [1 << 19] * 4, "n_min": 16,
                 "n_max": 1024, "d2_mode": "laplacian"},
        "n_points": 1 << 21,
        "tables": ("normal", 1e-2),
        "mlp": {"hidden": 64, "depth": 2, "omega": 30.0},
        "clustered_half": True,
        "outputs": ("residual", "loss"),
    },
    # INGP-FD comparator: the same residual step with the 3D d-linear encoding of the standard
    # size (N 16..2048) and the Laplacian of u by central differences over 7 stencil points,
    # step eps = 2^-11 (the finest level's cell width); same SIREN, points and table scale as
    # the fused Hermite residual.
    "fd_residual3d": {
        "id": 6,
        "spec": {"d": 3, "L": 16, "F": 2, "kind": "dlinear", "T": [1 << 19], "n_min": 16,
                 "n_max": 2048},
        "n_points": 1 << 21,
        "tables": ("normal", 1e-2),
        "mlp": {"hidden": 64, "depth": 2, "omega": 30.0},
        "fd_eps": 2.0 ** -11,
        "clustered_half": True,
        "outputs": ("residual", "loss"),
    },
    # Space-time Hermite-NGP (d = 4): 16 coefficients per vertex in five order tables of 2^16
    # rows (widths F, 4F, 6F, 4F, F), 8 levels N 4..64 (the four coarsest dense), diagonal
    # second derivatives, 2^18 points uniform in [0,1)^4.
    "hermite4d_L8_T16": {
        "id": 9,
        "spec": {"d": 4, "L": 8, "F": 2, "kind": "hermite", "T": [1 << 16] * 5, "n_min": 4, "n_max": 64,
                 "d2_mode": "diag"},
        "n_points": 1 << 18,
        "tables": ("normal", 1e-2),
        "outputs": ("gamma", "dgamma", "d2gamma"),
    },
    # DInf-Grid Gaussian RBF, 2D: four co-located dense grids N = 64..512 (the largest 512 on
    # a side, the 2D setting the summary recommends), eps = 1 with 3-ring neighbourhoods (36
    # vertices per level), one stratified point per pixel of a 512 x 512 image.
    "rbf2d_L4_N512": {
        "id": 7,
        "spec": {"d": 2, "L": 4, "F": 2, "kind": "rbf", "T": [1 << 19], "n_min": 64, "n_max": 512,
                 "rbf_eps": 1.0, "rbf_rings": 3, "d2_mode": "laplacian"},
        "n_points": 1 << 18,
        "stratified_side": 512,
        "tables": ("normal", 1e-2),
        "outputs": ("gamma", "dgamma", "d2gamma"),
    },
    # DInf-Grid Gaussian RBF, 3D: N = 7..56 (about 56 on a side, the 3D setting the summary
    # recommends), eps = 1, 3 rings (216 vertices per level), one stratified point per cell
    # of a 64^3 grid, diagonal second derivatives.
    "rbf3d_L4_N56": {
        "id": 8,
        "spec": {"d": 3, "L": 4, "F": 2, "kind": "rbf", "T": [1 << 18], "n_min": 7, "n_max": 56,
                 "rbf_eps": 1.0, "rbf_rings": 3, "d2_mode": "diag"},
        "n_points": 1 << 18,
        "stratified_side": 64,
        "tables": ("normal", 1e-2),
        "outputs": ("gamma", "dgamma", "d2gamma"),
    },
}


def rng(workload_id: int, stream: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([int(workload_id), int(stream)]))


def points(workload_id: int, n: int, d: int, clustered_half: bool = False) -> np.ndarray:
    """x in [0,1)^d, float32 [n, d].  With ``clustered_half`` the second half comes from 8
    Gaussian clusters (sigma 0.02, centres uniform in [0.15, 0.85]^d); coordinates that
    fall outside [0,1) are redrawn."""
    r = rng(workload_id, STREAM_POINTS)
    if not clustered_half:
        return r.random((n, d), dtype=np.float32)
    n_uni = n - n // 2
    x = np.empty((n, d), np.float32)
    x[:n_uni] = r.random((n_uni, d), dtype=np.float32)
    rc = rng(workload_id, STREAM_CLUSTERS)
    centres = rc.uniform(0.15, 0.85, size=(8, d))
    m = n - n_uni
    ids = rc.integers(0, 8, size=m)
    pts = centres[ids] + 0.02 * rc.standard_normal((m, d))
    bad = np.any((pts < 0.0) | (pts >= 1.0), axis=1)
    while bad.any():
        pts[bad] = centres[ids[bad]] + 0.02 * rc.standard_normal((int(bad.sum()), d))
        bad = np.any((pts < 0.0) | (pts >= 1.0), axis=1)
    x[n_uni:] = pts.astype(np.float32)
    # float32 rounding can carry a value just below 1 up to 1.0: pull it back inside.
    np.minimum(x, np.float32(1.0 - 2.0 ** -24), out=x)
    return x


def stratified_points(workload_id: int, side: int, d: int) -> np.ndarray:
    """One point uniform in each of the side^d cells of [0,1)^d (stratified sampling), cells
    in row-major order with the first axis fastest, float32 [side^d, d]."""
    r = rng(workload_id, STREAM_POINTS)
    idx = np.indices((side,) * d).reshape(d, -1)[::-1].T  # first axis fastest
    x = (idx + r.random(idx.shape)) / side
    x = x.astype(np.float32)
    np.minimum(x, np.float32(1.0 - 2.0 ** -24), out=x)
    return x


def workload_points(name: str, n: int | None = None) -> np.ndarray:
    """The points of a workload (its first n, when given)."""
    W = WORKLOADS[name]
    d = W["spec"]["d"]
    if "stratified_side" in W:
        x = stratified_points(W["id"], W["stratified_side"], d)
    else:
        x = points(W["id"], W["n_points"], d, W.get("clustered_half", False))
    return x if n is None else x[:n]


def tables(workload_id: int, n_params: int, dist: tuple) -> np.ndarray:
    """Table entries, float32 [n_params]: ("uniform", a) ~ U[-a, a]; ("normal", s) ~ N(0, s^2)."""
    r = rng(workload_id, STREAM_TABLES)
    kind, a = dist
    if kind == "uniform":
        return r.uniform(-a, a, size=n_params).astype(np.float32)
    if kind == "normal":
        return (a * r.standard_normal(n_params)).astype(np.float32)
    raise ValueError(kind)


def upstream(workload_id: int, shapes: list[tuple]) -> list[np.ndarray]:
    """Upstream gradients ~ N(0, 1), float32, one array per requested shape, drawn in order."""
    r = rng(workload_id, STREAM_UPSTREAM)
    return [r.standard_normal(s, dtype=np.float32) for s in shapes]


def delta(workload_id: int, n_params: int) -> np.ndarray:
    """A random parameter direction (for adjoint-identity checks), float32 N(0, 1)."""
    return rng(workload_id, STREAM_DELTA).standard_normal(n_params, dtype=np.float32)


def siren_mlp(workload_id: int, n_in: int, hidden: int, depth: int) -> np.ndarray:
    """SIREN-style initial weights, float32, packed W1,b1,...,Wo,bo (row-major out x in):
    first layer U(+-1/n_in), later layers U(+-sqrt(6/fan_in)/30), biases U(+-1/sqrt(fan_in))."""
    r = rng(workload_id, STREAM_MLP)
    parts = []
    for k in range(depth + 1):
        fan_in = n_in if k == 0 else hidden
        fan_out = 1 if k == depth else hidden
        lim = 1.0 / fan_in if k == 0 else math.sqrt(6.0 / fan_in) / 30.0
        parts.append(r.uniform(-lim, lim, size=fan_in * fan_out))
        parts.append(r.uniform(-1.0 / math.sqrt(fan_in), 1.0 / math.sqrt(fan_in), size=fan_out))
    return np.concatenate(parts).astype(np.float32)
