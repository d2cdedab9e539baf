"""Oracle pins for the interpolants.

d-linear: Instant-NGP explainer (nxrte.com), step 3 (d-linear interpolation of the 2^d
vertex features); Hermite-NGP notes (m0rtzz.github.io), key design 1 (the reconstruction
sum over vertices and derivative multi-indices with the Delta x^{|alpha|} scaling, the 1D
value and derivative bases, the tensor-product basis) and key design 2 (the basis
derivatives and their factorised d-dimensional form).  Special cases are checked against
scipy's RegularGridInterpolator and CubicHermiteSpline, closed forms (affine and per-axis
cubic reproduction, partition of unity) and finite differences.
"""
import numpy as np
import pytest
from numpy.polynomial import polynomial as npoly
from scipy.interpolate import CubicHermiteSpline, RegularGridInterpolator

from tests.helpers import dense_vertices, fill_dense_hermite, rel_err


def _rand_pts(n, d, seed):
    """x = k 2^-16: x * N is exact in fp32 for N < 256, so the position the oracle evaluates
    (x rounded through fl32(x N)) is x itself and closed forms apply at x."""
    k = np.random.default_rng(seed).integers(0, 1 << 16, size=(n, d))
    return (k / 65536.0).astype(np.float32)


# ================================================================ d-linear
def test_dlinear_reproduces_affine_fields_on_dense_levels(orc):
    spec = {"d": 3, "L": 3, "F": 2, "kind": "dlinear", "T": [1 << 16], "resolutions": [4, 9, 16]}
    lay = orc.layout(spec)
    a = np.array([[0.3, -1.2, 2.0], [1.5, 0.25, -0.75]])
    c0 = np.array([0.1, -2.0])
    params = np.zeros(lay["n_params"])
    for l, N in enumerate(lay["N"]):
        assert lay["dense"][0, l]
        pos = dense_vertices(N, 3) / N
        vals = pos @ a.T + c0
        params[lay["offset"][0, l]:lay["offset"][0, l] + vals.size] = vals.ravel()
    x = _rand_pts(500, 3, 1)
    g, _, _ = orc.forward(spec, x, params)
    expect = x.astype(np.float64) @ a.T + c0
    for l in range(3):
        assert np.max(np.abs(g[:, 2 * l:2 * l + 2] - expect)) < 1e-12


def test_dlinear_partition_of_unity_on_hashed_levels(orc):
    spec = {"d": 3, "L": 4, "F": 1, "kind": "dlinear", "T": [1 << 8], "n_min": 4, "n_max": 64}
    lay = orc.layout(spec)
    assert not lay["dense"][0, -1]
    g, _, _ = orc.forward(spec, _rand_pts(300, 3, 2), np.ones(lay["n_params"]))
    assert np.max(np.abs(g - 1.0)) < 1e-13


@pytest.mark.parametrize("d", [2, 3])
def test_dlinear_matches_scipy_regular_grid(orc, d):
    N = 7
    spec = {"d": d, "L": 1, "F": 1, "kind": "dlinear", "T": [1 << 12], "resolutions": [N]}
    lay = orc.layout(spec)
    vals = np.random.default_rng(3).uniform(-1, 1, lay["n_params"])
    x = _rand_pts(400, d, 4)
    g, _, _ = orc.forward(spec, x, vals)
    # rows are x-fastest, so the C-ordered grid has axes (..., y, x)
    grid = vals.reshape([N + 1] * d)
    axes = [np.arange(N + 1) / N] * d
    rgi = RegularGridInterpolator(axes, grid, method="linear")
    ref = rgi(x.astype(np.float64)[:, ::-1])
    assert np.max(np.abs(g[:, 0] - ref)) < 1e-12


# ================================================================ Hermite
def _poly_field(d, F, seed):
    """A sum of products of per-axis cubics, per feature: returns deriv_fn(axes, pos) giving
    the mixed partial over `axes` (each axis differentiated once), and the full field
    value/gradient/second-derivative evaluators."""
    rng = np.random.default_rng(seed)
    terms = [[[rng.uniform(-1, 1, 4) for _ in range(d)] for _ in range(3)] for _ in range(F)]

    def ev(pos, orders):
        """pos [n, d]; orders[i] = derivative order along axis i -> [n, F]."""
        out = np.zeros((pos.shape[0], F))
        for f in range(F):
            for term in terms[f]:
                prod = np.ones(pos.shape[0])
                for i in range(d):
                    coef = term[i]
                    for _ in range(orders[i]):
                        coef = npoly.polyder(coef)
                    prod *= npoly.polyval(pos[:, i], coef)
                out[:, f] += prod
        return out

    def deriv_fn(axes, pos):
        return ev(pos, [1 if i in axes else 0 for i in range(d)])

    return deriv_fn, ev


@pytest.mark.parametrize("d,mode", [(2, "laplacian"), (3, "diag"), (3, "laplacian"), (4, "diag"), (4, "laplacian")])
def test_hermite_reproduces_per_axis_cubics(orc, d, mode):
    F = 2
    spec = {"d": d, "L": 2, "F": F, "kind": "hermite", "T": [1 << 16] * (d + 1),
            "resolutions": [5, 11], "d2_mode": mode}
    lay = orc.layout(spec)
    deriv_fn, ev = _poly_field(d, F, 5)
    params = np.zeros(lay["n_params"])
    for l in range(2):
        fill_dense_hermite(params, lay, spec, l, deriv_fn)
    x = _rand_pts(400, d, 6)
    xd = x.astype(np.float64)
    g, dg, d2 = orc.forward(spec, x, params)
    val = ev(xd, [0] * d)
    grads = [ev(xd, [1 if j == i else 0 for j in range(d)]) for i in range(d)]
    hess = [ev(xd, [2 if j == i else 0 for j in range(d)]) for i in range(d)]
    for l in range(2):
        sl = slice(l * F, (l + 1) * F)
        assert rel_err(g[:, sl], val) < 1e-12
        for i in range(d):
            assert rel_err(dg[:, i, sl], grads[i]) < 1e-11
            if mode == "diag":
                assert rel_err(d2[:, i, sl], hess[i]) < 1e-10
        if mode == "laplacian":
            assert rel_err(d2[:, sl], sum(hess)) < 1e-10


def test_hermite_1d_profile_matches_scipy_cubic_hermite_spline(orc):
    # data that depends on x only: value and x-slope tables random along x, constant in y;
    # the y and xy derivative tables are zero.  Every row y is then the textbook 1D spline.
    N, F = 9, 1
    spec = {"d": 2, "L": 1, "F": F, "kind": "hermite", "T": [1 << 10] * 3, "resolutions": [N],
            "d2_mode": "laplacian"}
    lay = orc.layout(spec)
    rng = np.random.default_rng(7)
    p = rng.uniform(-1, 1, N + 1)
    m = rng.uniform(-5, 5, N + 1)
    V = dense_vertices(N, 2)
    params = np.zeros(lay["n_params"])
    params[lay["offset"][0, 0]:lay["offset"][0, 0] + V.shape[0]] = p[V[:, 0]]
    blk = np.zeros((V.shape[0], 2))
    blk[:, 0] = m[V[:, 0]]                 # slot x of the order-1 table
    params[lay["offset"][1, 0]:lay["offset"][1, 0] + blk.size] = blk.ravel()
    x = _rand_pts(300, 2, 8)
    g, dg, lap = orc.forward(spec, x, params)
    spl = CubicHermiteSpline(np.arange(N + 1) / N, p, m)
    xs = x[:, 0].astype(np.float64)
    assert np.max(np.abs(g[:, 0] - spl(xs))) < 1e-12
    assert np.max(np.abs(dg[:, 0, 0] - spl.derivative(1)(xs))) < 1e-10
    assert np.max(np.abs(dg[:, 1, 0])) < 1e-12
    assert np.max(np.abs(lap[:, 0] - spl.derivative(2)(xs))) < 1e-8


def test_hermite_interpolates_vertex_data(orc):
    # at a vertex (t = 0) the field is the stored value and its gradient the stored first
    # derivatives, on hashed levels too
    spec = {"d": 3, "L": 3, "F": 2, "kind": "hermite", "T": [1 << 9] * 4,
            "resolutions": [4, 8, 16], "d2_mode": "diag"}
    lay = orc.layout(spec)
    assert not lay["dense"][0, 2]
    params = np.random.default_rng(9).normal(0, 1, lay["n_params"])
    k = np.random.default_rng(10).integers(0, 4, size=(50, 3))
    x = (k / 4.0).astype(np.float32)          # vertices of every level (4 | N)
    g, dg, _ = orc.forward(spec, x, params)
    idx0 = orc.indices(spec, x, 0)
    idx1 = orc.indices(spec, x, 1)
    for l in range(3):
        o0, o1 = lay["offset"][0, l], lay["offset"][1, l]
        for f in range(2):
            expect = params[o0 + idx0[:, l, 0] * 2 + f]
            assert np.max(np.abs(g[:, 2 * l + f] - expect)) < 1e-12
            for i in range(3):
                expect_d = params[o1 + idx1[:, l, 0] * 6 + i * 2 + f]
                assert np.max(np.abs(dg[:, i, 2 * l + f] - expect_d)) < 1e-10


def test_hermite_value_tables_equal_smoothstep_dlinear(orc):
    # with every derivative table zero, the Hermite field is the d-linear field with each
    # t replaced by 3t^2 - 2t^3
    N = 8
    sh = {"d": 2, "L": 1, "F": 1, "kind": "hermite", "T": [1 << 10] * 3, "resolutions": [N]}
    sl = {"d": 2, "L": 1, "F": 1, "kind": "dlinear", "T": [1 << 10], "resolutions": [N]}
    lh, ll = orc.layout(sh), orc.layout(sl)
    vals = np.random.default_rng(11).uniform(-1, 1, ll["n_params"])
    ph = np.zeros(lh["n_params"])
    ph[:vals.size] = vals
    # points with t in a dyadic grid so that the warped point is exact in fp32
    cell = np.random.default_rng(12).integers(0, N, size=(200, 2))
    t = np.random.default_rng(13).integers(0, 1 << 10, size=(200, 2)) / 1024.0
    x = ((cell + t) / N).astype(np.float32)
    s = 3 * t ** 2 - 2 * t ** 3
    xw = ((cell + s) / N).astype(np.float32)
    gh, _, _ = orc.forward(sh, x, ph)
    gl, _, _ = orc.forward(sl, xw, vals)
    # the warped point is rounded to fp32 once: allow that rounding
    assert np.max(np.abs(gh - gl)) < 1e-5


@pytest.mark.parametrize("d", [3, 4])
def test_hermite_finite_differences_on_hashed_levels(orc, d):
    # random (non-polynomial across cells) tables with collisions; inside a cell the field
    # is a per-axis cubic, so central differences of step h agree to O(h^2) for the
    # gradient and exactly (up to rounding) for the diagonal second derivatives
    N = 24
    spec = {"d": d, "L": 1, "F": 2, "kind": "hermite", "T": [1 << 8] * (d + 1), "resolutions": [N],
            "d2_mode": "diag"}
    lay = orc.layout(spec)
    assert not lay["dense"][0, 0]
    params = np.random.default_rng(14).normal(0, 1, lay["n_params"])
    rng = np.random.default_rng(15)
    # x = k 2^-18: x*N is exact in fp32 for N < 32, so evaluation positions are known exactly
    cell = rng.integers(0, N, size=(60, d))
    tq = rng.integers(int(0.1 * 2 ** 18 / N), int(0.9 * 2 ** 18 / N), size=(60, d))
    k = cell * (2 ** 18 // N) + tq
    k = k.astype(np.int64)
    h = 64  # step 64 * 2^-18 = 2^-12
    x0 = (k / 2.0 ** 18).astype(np.float32)
    assert np.all(np.floor(x0.astype(np.float64) * N) == np.floor((k + h) / 2.0 ** 18 * N))
    assert np.all(np.floor(x0.astype(np.float64) * N) == np.floor((k - h) / 2.0 ** 18 * N))
    g0, dg0, d20 = orc.forward(spec, x0, params)
    hs = h / 2.0 ** 18
    for i in range(d):
        e = np.zeros(d, np.int64)
        e[i] = h
        gp, _, _ = orc.forward(spec, ((k + e) / 2.0 ** 18).astype(np.float32), params)
        gm, _, _ = orc.forward(spec, ((k - e) / 2.0 ** 18).astype(np.float32), params)
        fd1 = (gp - gm) / (2 * hs)
        fd2 = (gp - 2 * g0 + gm) / hs ** 2
        assert rel_err(fd1, dg0[:, i]) < 1e-4
        assert rel_err(fd2, d20[:, i]) < 1e-6


def test_hermite_is_c1_across_cell_faces(orc):
    # approaching a face x_0 = j/N from below and sitting on it: value and gradient agree to
    # O(delta) on a hashed level, where a C0 interpolant's gradient would jump
    N = 16
    spec = {"d": 2, "L": 1, "F": 1, "kind": "hermite", "T": [1 << 6] * 3, "resolutions": [N],
            "d2_mode": "laplacian"}
    lay = orc.layout(spec)
    params = np.random.default_rng(16).normal(0, 1, lay["n_params"])
    j = np.arange(1, N)
    y = (np.random.default_rng(17).integers(0, 1 << 12, size=j.size) / 4096.0)
    on = np.stack([j / N, y], 1).astype(np.float32)
    delta = 2.0 ** -20
    below = np.stack([j / N - delta, y], 1).astype(np.float32)
    g_on, d_on, _ = orc.forward(spec, on, params)
    g_b, d_b, _ = orc.forward(spec, below, params)
    scale = np.max(np.abs(d_on))
    assert np.max(np.abs(g_on - g_b)) < 4 * scale * delta
    assert np.max(np.abs(d_on - d_b)) < 1e-3 * scale
    # contrast: the d-linear interpolant's one-sided slopes differ across the same faces
    sl = {"d": 2, "L": 1, "F": 1, "kind": "dlinear", "T": [1 << 6], "resolutions": [N]}
    pl = params[:orc.layout(sl)["n_params"]]
    h = 2.0 ** -12
    above = (on + np.float32(h) * np.array([1, 0], np.float32)).astype(np.float32)
    f_on = orc.forward(sl, on, pl)[0]
    slope_up = (orc.forward(sl, above, pl)[0] - f_on) / h
    slope_dn = (f_on - orc.forward(sl, below, pl)[0]) / delta
    assert np.max(np.abs(slope_up - slope_dn)) > 1.0
