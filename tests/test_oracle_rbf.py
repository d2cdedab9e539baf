"""Oracle pins for the Gaussian-RBF interpolant (DInf-Grid summary, shdxiang-github-io:
可微的径向基函数插值 — normalised weights phi(|x - x_i|) / sum_j phi(|x - x_j|),
phi(r) = exp(-(eps r)^2), over a precomputed k-ring neighbourhood — and 多分辨率特征网格).

Readings: distances in units of the level's grid spacing; the k-ring neighbourhood is the box
of (2k)^d vertices around the point's cell, clipped to the grid.  Pinned against:
  - partition of unity (a constant field is reproduced with zero derivatives);
  - the flat-kernel limit eps -> 0: the plain mean of the box's vertex values (pins which
    vertices form the neighbourhood, including the clipping);
  - the sharp-kernel limit eps -> infinity: the nearest vertex's value;
  - linear fields at interior cell centres: reproduced exactly, with gradient
    2 eps^2 Var(offsets) times the slope and zero Laplacian (by symmetry), the variance being
    a closed-form 2k-term 1D sum;
  - separability: a field that depends on x alone gives the same values in 2D and 3D;
  - central differences of gamma for grad gamma and the second derivatives;
  - the adjoint identity and brute-force J^T G for the backward.
"""
import numpy as np
import pytest

from tests.helpers import dense_vertices


def _spec(d, res, k, eps, F=1, T=1 << 20, mode="diag"):
    return {"d": d, "L": len(res), "F": F, "kind": "rbf", "T": [T], "resolutions": list(res),
            "rbf_eps": eps, "rbf_rings": k, "d2_mode": mode}


@pytest.mark.parametrize("d,k", [(2, 1), (2, 3), (3, 2), (3, 3)])
def test_partition_of_unity(orc, d, k):
    spec = _spec(d, [5, 11], k, 1.0, F=2, T=1 << 8)   # level 1 hashed in 3D
    lay = orc.layout(spec)
    th = np.full(lay["n_params"], 1.75)
    x = np.random.default_rng(d + k).random((300, d), dtype=np.float32)
    x[:3] = [[0.0] * d, [1.0] * d, [0.5] * d]
    g, dg, d2 = orc.forward(spec, x, th)
    assert np.max(np.abs(g - 1.75)) < 1e-13
    assert np.max(np.abs(dg)) < 1e-11
    assert np.max(np.abs(d2)) < 1e-9


@pytest.mark.parametrize("d,k", [(2, 1), (2, 2), (3, 2)])
def test_flat_kernel_is_the_box_mean(orc, d, k):
    N = 6
    spec = _spec(d, [N], k, 1e-4)
    lay = orc.layout(spec)
    th = np.random.default_rng(1).standard_normal(lay["n_params"])
    V = dense_vertices(N, d)
    rng = np.random.default_rng(2)
    x = rng.random((200, d), dtype=np.float32)
    x[:2] = [[0.0] * d, [0.999] * d]
    g, _, _ = orc.forward(spec, x, th)
    for q in range(x.shape[0]):
        p = x[q].astype(np.float32) * np.float32(N)
        base = np.minimum(np.floor(p), N - 1).astype(int)
        lo, hi = np.maximum(base - k + 1, 0), np.minimum(base + k, N)
        inbox = np.all((V >= lo) & (V <= hi), axis=1)
        assert abs(g[q, 0] - th[inbox].mean()) < 1e-6 * (1 + np.abs(th).max())


def test_sharp_kernel_picks_the_nearest_vertex(orc):
    d, N = 3, 8
    spec = _spec(d, [N], 3, 30.0)
    lay = orc.layout(spec)
    th = np.random.default_rng(3).standard_normal(lay["n_params"])
    V = dense_vertices(N, d)
    rng = np.random.default_rng(4)
    # within 0.25 grid units of a vertex
    v = rng.integers(0, N + 1, size=(100, d))
    x = ((v + rng.uniform(-0.25, 0.25, size=(100, d))) / N).clip(0, 1).astype(np.float32)
    g, _, _ = orc.forward(spec, x, th)
    near = np.rint(x.astype(np.float64) * N).astype(int)
    idx = [int(np.nonzero(np.all(V == nv, axis=1))[0][0]) for nv in near]
    assert np.max(np.abs(g[:, 0] - th[idx])) < 1e-12


@pytest.mark.parametrize("d,k,eps", [(2, 3, 1.0), (3, 2, 0.7), (3, 3, 1.3)])
def test_linear_field_at_cell_centres(orc, d, k, eps):
    N = 16  # a power of two: the cell centres are exact in fp32
    spec = _spec(d, [N], k, eps, mode="diag")
    lay = orc.layout(spec)
    rng = np.random.default_rng(5)
    a, b = rng.uniform(-1, 1, d), rng.uniform(-1, 1)
    th = dense_vertices(N, d) @ a / N + b
    # interior cell centres: the whole box lies inside the grid
    cells = rng.integers(k - 1, N - k + 1, size=(50, d))
    x = ((cells + 0.5) / N).astype(np.float32)
    g, dg, d2 = orc.forward(spec, x, th)
    assert np.max(np.abs(g[:, 0] - (x.astype(np.float64) @ a + b))) < 1e-12
    off = np.arange(-k + 1, k + 1) - 0.5          # v - p along one axis at a cell centre
    wt = np.exp(-(eps * off) ** 2)
    var = np.sum(wt * off ** 2) / np.sum(wt)
    assert np.max(np.abs(dg[:, :, 0] - 2 * eps ** 2 * var * a)) < 1e-11
    assert np.max(np.abs(d2)) < 1e-9


def test_field_of_x_alone_is_dimension_independent(orc):
    N, k, eps = 9, 3, 1.1
    f = np.random.default_rng(6).standard_normal(N + 1)
    out = []
    pts = np.random.default_rng(7).random((120, 3), dtype=np.float32)
    for d in (2, 3):
        spec = _spec(d, [N], k, eps, mode="diag")
        th = f[dense_vertices(N, d)[:, 0]]
        out.append(orc.forward(spec, pts[:, :d], th))
    (g2, dg2, h2), (g3, dg3, h3) = out
    assert np.max(np.abs(g2 - g3)) < 1e-13
    assert np.max(np.abs(dg2[:, 0] - dg3[:, 0])) < 1e-11
    assert np.max(np.abs(h2[:, 0] - h3[:, 0])) < 1e-9
    assert np.max(np.abs(dg3[:, 1:])) < 1e-11 and np.max(np.abs(h3[:, 1:])) < 1e-8


@pytest.mark.parametrize("d", [2, 3])
def test_derivatives_match_central_differences(orc, d):
    spec = _spec(d, [6, 13], 3, 0.9, F=2, T=1 << 10, mode="diag")   # level 1 hashed in 3D
    lay = orc.layout(spec)
    th = np.random.default_rng(8).standard_normal(lay["n_params"])
    h = 2.0 ** -12
    # dyadic points, away from cell faces (the k-ring box changes across a face)
    rng = np.random.default_rng(9)
    x = (rng.integers(64, 4096 - 64, size=(40, d)) / 4096.0).astype(np.float32)
    g, dg, d2 = orc.forward(spec, x, th)
    for i in range(d):
        e = np.zeros(d, np.float32)
        e[i] = h
        gp, _, _ = orc.forward(spec, x + e, th)
        gm, _, _ = orc.forward(spec, x - e, th)
        # skip points whose stencil crosses a cell face at either level (the box moves there)
        ok = np.ones(x.shape[0], bool)
        for N in (6, 13):
            for s in (x + e, x - e):
                ok &= np.floor(s[:, i].astype(np.float32) * np.float32(N)) == np.floor(
                    x[:, i].astype(np.float32) * np.float32(N))
        assert ok.sum() > 10
        fd1 = (gp - gm) / (2 * h)
        fd2 = (gp - 2 * g + gm) / h ** 2
        scale1 = np.max(np.abs(dg[ok, i]))
        scale2 = np.max(np.abs(d2[ok, i]))
        assert np.max(np.abs(fd1[ok] - dg[ok, i])) <= 1e-4 * scale1
        assert np.max(np.abs(fd2[ok] - d2[ok, i])) <= 1e-3 * scale2


@pytest.mark.parametrize("mode", ["diag", "laplacian"])
def test_rbf_adjoint_identity(orc, mode):
    spec = _spec(3, [4, 9], 2, 1.0, F=2, T=1 << 9, mode=mode)
    lay = orc.layout(spec)
    assert not lay["dense"][0, -1]
    rng = np.random.default_rng(10)
    n, LF = 150, 4
    x = rng.random((n, 3), dtype=np.float32)
    G = (rng.standard_normal((n, LF)), rng.standard_normal((n, 3, LF)),
         rng.standard_normal((n, 3, LF)) if mode == "diag" else rng.standard_normal((n, LF)))
    grad = orc.backward(spec, x, *G)
    dth = rng.standard_normal(lay["n_params"])
    outs = orc.forward(spec, x, dth)
    rhs = sum(float(np.sum(o * g)) for o, g in zip(outs, G))
    assert abs(float(grad @ dth) - rhs) <= 1e-11 * (abs(rhs) + np.sum(np.abs(grad)))


def test_rbf_backward_brute_force_tiny(orc):
    spec = _spec(2, [3], 2, 1.0, F=1, T=64, mode="laplacian")
    lay = orc.layout(spec)
    rng = np.random.default_rng(11)
    x = rng.random((6, 2), dtype=np.float32)
    G = (rng.standard_normal((6, 1)), rng.standard_normal((6, 2, 1)), rng.standard_normal((6, 1)))
    grad = orc.backward(spec, x, *G)
    brute = np.zeros(lay["n_params"])
    for j in range(lay["n_params"]):
        e = np.zeros(lay["n_params"])
        e[j] = 1.0
        brute[j] = sum(float(np.sum(o * g)) for o, g in zip(orc.forward(spec, x, e), G))
    assert np.max(np.abs(grad - brute)) < 1e-12 * max(1.0, np.max(np.abs(brute)))


def test_rbf_rejects_bad_parameters(orc):
    for k, eps in [(0, 1.0), (5, 1.0), (2, 0.0)]:
        with pytest.raises(ValueError):
            orc.make_cfg(_spec(2, [4], k, eps))
