"""Oracle pins for the INGP-FD comparator: the residual whose Laplacian is taken by central
differences over the 2d+1 stencil points of a d-linear encoding + SIREN.

Hermite-NGP notes (m0rtzz.github.io), the 现有痛点 paragraph (INGP-FD: 2d+1 forward passes
per Laplacian, O(eps^2) truncation) and key design 2's comparison.  Pinned against:
  - a closed form: on a dense level holding an affine field the encoding is affine in x, so a
    one-hidden-layer SIREN gives u = sum_o Wo_o sin(omega (a_o . x + c_o)) + bo with the
    analytic Laplacian -omega^2 sum_o Wo_o |a_o|^2 sin(...); the FD value must sit within the
    central-difference truncation bound (eps^2 / 12) sum_i max |d^4 u / dx_i^4];
  - the analytic forward-mode Laplacian of the fused Hermite residual (a separate code path)
    for a two-layer SIREN on a Hermite encoding of the same affine field: second-order
    convergence as eps halves, and the same u at the centre;
  - the stencil order (stencil point 2i+1 is the centre of the point shifted by +eps e_i);
  - finite differences of the loss in parameter space for both gradients, and the loss's
    invariance under the output bias.
"""
import numpy as np
import pytest

from tests.helpers import dense_vertices, fill_dense_hermite


def _affine_dlinear(orc, d, N, F, A, c):
    spec = {"d": d, "L": 1, "F": F, "kind": "dlinear", "T": [(N + 1) ** d], "resolutions": [N]}
    lay = orc.layout(spec)
    assert lay["dense"][0, 0]
    pos = dense_vertices(N, d) / float(N)
    params = (pos @ A.T + c).ravel()  # row-major [rows, F]
    return spec, params


def _grid_points(n, d, eps, seed):
    # multiples of 2^-10 inside [eps, 1 - eps]: x +- eps is exact in fp32
    rng = np.random.default_rng(seed)
    lo, hi = int(eps * 1024), int((1 - eps) * 1024)
    return (rng.integers(lo, hi + 1, size=(n, d)) / 1024.0).astype(np.float32)


def _mlp_depth1(F, H, rng):
    W1 = rng.uniform(-1, 1, (H, F))
    b1 = rng.uniform(-0.5, 0.5, H)
    Wo = rng.uniform(-1, 1, H)
    bo = rng.uniform(-0.5, 0.5, 1)
    return W1, b1, Wo, bo, np.concatenate([W1.ravel(), b1, Wo, bo])


@pytest.mark.parametrize("d", [2, 3])
def test_fd_laplacian_against_closed_form(orc, d):
    rng = np.random.default_rng(d)
    F, H, omega, eps = 2, 6, 2.0, 2.0 ** -5
    A = rng.uniform(-1, 1, (F, d))
    c = rng.uniform(-0.5, 0.5, F)
    spec, params = _affine_dlinear(orc, d, 4, F, A, c)
    W1, b1, Wo, bo, mlp = _mlp_depth1(F, H, rng)
    x = _grid_points(200, d, eps, d + 10)
    out = orc.fd_residual(spec, H, 1, omega, eps, x, params, mlp)
    a = W1 @ A                       # [H, d]: u = sum_o Wo_o sin(omega (a_o . x + c_o)) + bo
    co = W1 @ c + b1
    X = x.astype(np.float64)
    arg = omega * (X @ a.T + co)     # [n, H]
    u = np.sin(arg) @ Wo + bo[0]
    lap = (-omega ** 2 * np.sin(arg) * (a ** 2).sum(1)) @ Wo
    g = -d * np.pi ** 2 * np.prod(np.sin(np.pi * X), axis=1)
    bound = eps ** 2 / 12 * np.sum(np.abs(Wo) * omega ** 4 * (a ** 4).sum(1)) + 1e-9
    assert np.max(np.abs(out["u_stencil"][:, 0] - u)) < 1e-12
    lap_fd = out["r"] + g
    assert np.max(np.abs(lap_fd - lap)) <= bound
    assert np.max(np.abs(lap_fd - lap)) > 1e-3 * bound   # the truncation term is really there
    assert out["loss"] == pytest.approx(np.mean(out["r"] ** 2), rel=1e-14)


def test_fd_converges_to_the_analytic_hermite_laplacian(orc):
    d, F, N, H, depth, omega = 3, 2, 4, 8, 2, 1.5
    rng = np.random.default_rng(5)
    A = rng.uniform(-1, 1, (F, d))
    c = rng.uniform(-0.5, 0.5, F)
    dspec, dparams = _affine_dlinear(orc, d, N, F, A, c)
    hspec = {"d": d, "L": 1, "F": F, "kind": "hermite", "T": [(N + 1) ** d] * (d + 1), "resolutions": [N],
             "d2_mode": "laplacian"}
    hlay = orc.layout(hspec)

    def deriv(axes, pos):
        if len(axes) == 0:
            return pos @ A.T + c
        if len(axes) == 1:
            return np.broadcast_to(A[:, axes[0]], (pos.shape[0], F))
        return np.zeros((pos.shape[0], F))

    hparams = fill_dense_hermite(np.zeros(hlay["n_params"]), hlay, hspec, 0, deriv)
    mlp = rng.uniform(-0.6, 0.6, orc.mlp_param_count(F, H, depth))
    x = _grid_points(150, d, 2.0 ** -3, 7)
    ref = orc.residual(hspec, H, depth, omega, x, hparams, mlp)
    errs = []
    for eps in (2.0 ** -3, 2.0 ** -4, 2.0 ** -5):
        out = orc.fd_residual(dspec, H, depth, omega, eps, x, dparams, mlp)
        assert np.max(np.abs(out["u_stencil"][:, 0] - ref["u"])) < 1e-12
        errs.append(np.max(np.abs(out["r"] - ref["r"])))
    assert errs[0] > 1e-6
    assert errs[1] <= 0.3 * errs[0] and errs[2] <= 0.3 * errs[1], errs   # O(eps^2)


def test_fd_stencil_order(orc):
    d, eps = 3, 2.0 ** -4
    spec = {"d": d, "L": 3, "F": 2, "kind": "dlinear", "T": [1 << 10], "n_min": 3, "n_max": 30}
    rng = np.random.default_rng(8)
    params = rng.uniform(-1, 1, orc.layout(spec)["n_params"])
    mlp = rng.uniform(-0.5, 0.5, orc.mlp_param_count(6, 8, 2))
    x = _grid_points(40, d, eps, 9)
    out = orc.fd_residual(spec, 8, 2, 3.0, eps, x, params, mlp)
    for i in range(d):
        for sgn, s in ((1, 2 * i + 1), (-1, 2 * i + 2)):
            xs = x.copy()
            xs[:, i] += np.float32(sgn * eps)
            centre = orc.fd_residual(spec, 8, 2, 3.0, eps, xs, params, mlp)["u_stencil"][:, 0]
            assert np.array_equal(out["u_stencil"][:, s], centre)


def test_fd_gradients_match_loss_finite_differences(orc):
    d, H, depth, omega, eps = 3, 8, 2, 2.0, 2.0 ** -4
    spec = {"d": d, "L": 3, "F": 2, "kind": "dlinear", "T": [1 << 8], "n_min": 3, "n_max": 20}
    lay = orc.layout(spec)
    assert not lay["dense"][0, -1]   # a hashed level with collisions
    rng = np.random.default_rng(12)
    theta = rng.uniform(-0.5, 0.5, lay["n_params"])
    mlp = rng.uniform(-0.5, 0.5, orc.mlp_param_count(6, H, depth))
    x = rng.random((60, d), dtype=np.float32)
    base = orc.fd_residual(spec, H, depth, omega, eps, x, theta, mlp)

    def loss(t, m):
        return orc.fd_residual(spec, H, depth, omega, eps, x, t, m)["loss"]

    h = 1e-6
    for k in range(3):
        dt = rng.standard_normal(theta.size)
        fd = (loss(theta + h * dt, mlp) - loss(theta - h * dt, mlp)) / (2 * h)
        an = float(base["grad_params"] @ dt)
        assert abs(fd - an) <= 1e-6 * max(abs(an), 1.0), (k, fd, an)
        dm = rng.standard_normal(mlp.size)
        fd = (loss(theta, mlp + h * dm) - loss(theta, mlp - h * dm)) / (2 * h)
        an = float(base["grad_mlp"] @ dm)
        assert abs(fd - an) <= 1e-6 * max(abs(an), 1.0), (k, fd, an)
    # the output bias cancels in the stencil: no effect on the loss, zero gradient
    shifted = mlp.copy()
    shifted[-1] += 0.75
    assert loss(theta, shifted) == pytest.approx(base["loss"], rel=1e-9)
    assert base["grad_mlp"][-1] == 0.0


def test_fd_rejects_hermite_and_bad_eps(orc):
    spec = {"d": 2, "L": 2, "F": 2, "kind": "hermite", "T": [256] * 3, "n_min": 3, "n_max": 9}
    x = np.zeros((4, 2), np.float32)
    with pytest.raises(ValueError):
        orc.fd_residual(spec, 4, 1, 1.0, 0.01, x, np.zeros(orc.layout(spec)["n_params"]),
                        np.zeros(orc.mlp_param_count(4, 4, 1)))
    dspec = dict(spec, kind="dlinear", T=[256])
    with pytest.raises(ValueError):
        orc.fd_residual(dspec, 4, 1, 1.0, 0.0, x, np.zeros(orc.layout(dspec)["n_params"]),
                        np.zeros(orc.mlp_param_count(4, 4, 1)))
