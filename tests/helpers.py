"""Test-side helpers: building table contents from known fields on dense levels.

These restate the stated layout reading (row = sum_i v_i (N+1)^i on a dense level, slots of
order k in lexicographic axis order, feature innermost) in order to construct inputs whose
interpolated values are known in closed form.
"""
from itertools import combinations

import numpy as np


def dense_vertices(N: int, d: int) -> np.ndarray:
    """Integer vertex coordinates of every row of a dense level, [rows, d], x fastest."""
    r = np.arange((N + 1) ** d)
    return np.stack([(r // (N + 1) ** i) % (N + 1) for i in range(d)], axis=1)


def slots(d: int, k: int):
    """Axis tuples of the derivative slots of order k, in row order."""
    return list(combinations(range(d), k))


def fill_dense_hermite(params, lay, spec, level, deriv_fn):
    """deriv_fn(axes_tuple, xyz [rows, d]) -> values [rows, F]: the mixed partial of the field
    over the given axes at the vertex positions.  Writes every order table of a dense level."""
    d, F = spec["d"], spec["F"]
    N = lay["N"][level]
    V = dense_vertices(N, d)
    pos = V / float(N)
    for k in range(d + 1):
        assert lay["dense"][k, level]
        off, w = lay["offset"][k, level], lay["width"][k, level]
        block = np.zeros(((N + 1) ** d, w))
        for s, axes in enumerate(slots(d, k)):
            block[:, s * F:(s + 1) * F] = deriv_fn(axes, pos)
        params[off:off + block.size] = block.ravel()
    return params


def rel_err(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    den = np.max(np.abs(b))
    return float(np.max(np.abs(a - b)) / (den if den > 0 else 1.0))
