"""Oracle pins for the backward scatter-add and the fused PINN residual.

Backward: Instant-NGP news article (antipu.com.cn), adaptivity paragraph (gradients of
colliding vertices combine).  The encoding is linear in theta, so the backward is the
transpose of the forward: pinned by the adjoint identity, by brute force (forward applied to
every unit vector of a tiny table) and by the collision sum with a one-row table.

Residual: Hermite-NGP notes (m0rtzz.github.io), key design 2 (SIREN sin(omega .) with the
second-order chain rule and the printed single-hidden-layer Laplacian), loss section (the
residual term); pinned by that printed formula, by finite differences of u in x, and by
finite differences of the loss in parameter space.
"""
import numpy as np
import pytest

from tests.helpers import rel_err


def _pts(n, d, seed):
    return np.random.default_rng(seed).random((n, d), dtype=np.float32)


SPECS = [
    {"d": 2, "L": 3, "F": 2, "kind": "dlinear", "T": [1 << 6], "n_min": 3, "n_max": 20},
    {"d": 3, "L": 3, "F": 2, "kind": "dlinear", "T": [1 << 7], "n_min": 2, "n_max": 12},
    {"d": 2, "L": 3, "F": 2, "kind": "hermite", "T": [1 << 6, 1 << 5, 1 << 6], "n_min": 3,
     "n_max": 20, "d2_mode": "laplacian"},
    {"d": 3, "L": 2, "F": 2, "kind": "hermite", "T": [1 << 7] * 4, "n_min": 2, "n_max": 9,
     "d2_mode": "diag"},
    {"d": 3, "L": 2, "F": 1, "kind": "hermite", "T": [1 << 7] * 4, "n_min": 2, "n_max": 9,
     "d2_mode": "laplacian"},
    {"d": 4, "L": 2, "F": 2, "kind": "hermite", "T": [1 << 9, 1 << 8, 1 << 9, 1 << 7, 1 << 8], "n_min": 2,
     "n_max": 7, "d2_mode": "diag"},
]


def _upstream(spec, n, rng):
    LF, d = spec["L"] * spec["F"], spec["d"]
    gg = rng.standard_normal((n, LF))
    if spec["kind"] != "hermite":
        return gg, None, None
    gd = rng.standard_normal((n, d, LF))
    g2 = rng.standard_normal((n, d, LF)) if spec.get("d2_mode") == "diag" else rng.standard_normal((n, LF))
    return gg, gd, g2


@pytest.mark.parametrize("spec", SPECS, ids=lambda s: f"{s['kind']}{s['d']}d-{s.get('d2_mode', '')}")
def test_adjoint_identity(orc, spec):
    rng = np.random.default_rng(1)
    lay = orc.layout(spec)
    assert not lay["dense"][0, -1]           # collisions are exercised
    x = _pts(200, spec["d"], 2)
    G = _upstream(spec, 200, rng)
    grad = orc.backward(spec, x, *G)
    dtheta = rng.standard_normal(lay["n_params"])
    outs = orc.forward(spec, x, dtheta)
    rhs = sum(float(np.sum(o * g)) for o, g in zip(outs, G) if g is not None)
    lhs = float(grad @ dtheta)
    assert abs(lhs - rhs) <= 1e-11 * (abs(rhs) + np.sum(np.abs(grad)))


@pytest.mark.parametrize("spec", [SPECS[0], SPECS[3]], ids=["dlinear", "hermite"])
def test_backward_brute_force_tiny(orc, spec):
    # J^T G with J built column by column from forward(e_j) over every parameter
    spec = dict(spec, L=1, T=[8] * len(spec["T"]), n_min=3, n_max=3)
    lay = orc.layout(spec)
    x = _pts(5, spec["d"], 3)
    G = _upstream(spec, 5, np.random.default_rng(4))
    grad = orc.backward(spec, x, *G)
    brute = np.zeros(lay["n_params"])
    for j in range(lay["n_params"]):
        e = np.zeros(lay["n_params"])
        e[j] = 1.0
        outs = orc.forward(spec, x, e)
        brute[j] = sum(float(np.sum(o * g)) for o, g in zip(outs, G) if g is not None)
    assert np.max(np.abs(grad - brute)) < 1e-11 * max(1.0, np.max(np.abs(brute)))


def test_collisions_sum_not_average(orc):
    # a one-row hashed table: every vertex aliases row 0; d-linear weights sum to one, so
    # row 0 receives the plain sum of the upstream over all points
    spec = {"d": 3, "L": 2, "F": 2, "kind": "dlinear", "T": [1], "n_min": 4, "n_max": 8}
    x = _pts(300, 3, 5)
    G = np.random.default_rng(6).standard_normal((300, 4))
    grad = orc.backward(spec, x, G)
    assert grad.size == 4
    assert np.allclose(grad, G.sum(0), rtol=0, atol=1e-11)


def test_backward_accumulates_deterministically(orc):
    spec = SPECS[3]
    x = _pts(100, 3, 7)
    G = _upstream(spec, 100, np.random.default_rng(8))
    a = orc.backward(spec, x, *G)
    b = orc.backward(spec, x, *G)
    assert np.array_equal(a, b)


# ---------------------------------------------------------------- residual
RES_SPEC = {"d": 3, "L": 2, "F": 2, "kind": "hermite", "T": [1 << 9] * 4, "resolutions": [4, 7],
            "d2_mode": "laplacian"}


def _mlp(n_in, hidden, depth, seed, scale=1.0):
    rng = np.random.default_rng(seed)
    parts = []
    for k in range(depth + 1):
        fi = n_in if k == 0 else hidden
        fo = 1 if k == depth else hidden
        parts.append(rng.uniform(-1, 1, fi * fo) * scale / np.sqrt(fi))
        parts.append(rng.uniform(-0.5, 0.5, fo))
    return np.concatenate(parts)


def test_residual_single_layer_matches_printed_formula(orc):
    # Lap u = W2 [ -w^2 a * sum_i (W1 gamma_{x_i})^2 + w cos(w z) * W1 Lap gamma ],
    # a = sin(w z), z = W1 gamma + b1 (single hidden layer, as printed in key design 2)
    spec, H, w = RES_SPEC, 16, 3.0
    lay = orc.layout(spec)
    params = np.random.default_rng(20).normal(0, 0.3, lay["n_params"])
    mlp = _mlp(4, H, 1, 21)
    x = _pts(64, 3, 22)
    out = orc.residual(spec, H, 1, w, x, params, mlp)
    g, dg, lap = orc.forward(spec, x, params)
    W1 = mlp[:4 * H].reshape(H, 4)
    b1 = mlp[4 * H:5 * H]
    W2 = mlp[5 * H:6 * H]
    z = g @ W1.T + b1
    a = np.sin(w * z)
    s = sum((dg[:, i] @ W1.T) ** 2 for i in range(3))
    lap_u = (-w ** 2 * a * s + w * np.cos(w * z) * (lap @ W1.T)) @ W2
    assert rel_err(out["lap_u"], lap_u) < 1e-12
    # the manufactured source and the residual
    src = -3 * np.pi ** 2 * np.prod(np.sin(np.pi * x.astype(np.float64)), axis=1)
    assert rel_err(out["r"], lap_u - src) < 1e-12
    assert abs(out["loss"] - np.mean((lap_u - src) ** 2)) < 1e-12 * out["loss"]


def test_residual_source_is_the_laplacian_of_the_sine_product():
    # g = -3 pi^2 prod sin(pi x_i) is the Laplacian of prod sin(pi x_i): check by FD
    x = np.array([0.3, 0.55, 0.71])
    f = lambda p: np.prod(np.sin(np.pi * p))
    h = 1e-4
    lap = sum((f(x + h * e) - 2 * f(x) + f(x - h * e)) / h ** 2 for e in np.eye(3))
    assert abs(lap - (-3 * np.pi ** 2 * f(x))) < 1e-5


@pytest.mark.parametrize("depth", [1, 2])
def test_residual_forward_mode_matches_finite_differences(orc, depth):
    spec, H, w = RES_SPEC, 8, 2.0
    lay = orc.layout(spec)
    params = np.random.default_rng(23).normal(0, 0.3, lay["n_params"])
    mlp = _mlp(4, H, depth, 24)
    rng = np.random.default_rng(25)
    # x = k 2^-20 with the stencil inside one cell of both levels
    n, hk = 20, 16
    k = rng.integers(int(0.05 * 2 ** 20), int(0.95 * 2 ** 20), size=(n, 3))
    x0 = (k / 2.0 ** 20).astype(np.float32)
    base = orc.residual(spec, H, depth, w, x0, params, mlp)
    hs = hk / 2.0 ** 20
    lap_fd = np.zeros(n)
    for i in range(3):
        e = np.zeros(3, np.int64)
        e[i] = hk
        up = orc.residual(spec, H, depth, w, ((k + e) / 2.0 ** 20).astype(np.float32), params, mlp)["u"]
        dn = orc.residual(spec, H, depth, w, ((k - e) / 2.0 ** 20).astype(np.float32), params, mlp)["u"]
        same_cell = np.all([(np.floor((k + e) / 2.0 ** 20 * N) == np.floor(k / 2.0 ** 20 * N)).all(1) &
                            (np.floor((k - e) / 2.0 ** 20 * N) == np.floor(k / 2.0 ** 20 * N)).all(1)
                            for N in (4, 7)], axis=0)
        fd1 = (up - dn) / (2 * hs)
        assert rel_err(fd1[same_cell], base["grad_u"][same_cell, i]) < 1e-5
        lap_fd += (up - 2 * base["u"] + dn) / hs ** 2
        keep = same_cell if i == 0 else keep & same_cell
    assert keep.sum() > 10
    assert rel_err(lap_fd[keep], base["lap_u"][keep]) < 1e-4


def test_residual_gradients_match_loss_finite_differences(orc):
    spec, H, depth, w = RES_SPEC, 8, 2, 2.0
    lay = orc.layout(spec)
    rng = np.random.default_rng(26)
    params = rng.normal(0, 0.3, lay["n_params"])
    mlp = _mlp(4, H, depth, 27)
    x = _pts(40, 3, 28)
    out = orc.residual(spec, H, depth, w, x, params, mlp)
    for trial in range(3):
        dp = rng.standard_normal(params.size)
        dm = rng.standard_normal(mlp.size)
        eps = 1e-6
        lp = orc.residual(spec, H, depth, w, x, params + eps * dp, mlp + eps * dm)["loss"]
        lm = orc.residual(spec, H, depth, w, x, params - eps * dp, mlp - eps * dm)["loss"]
        fd = (lp - lm) / (2 * eps)
        an = out["grad_params"] @ dp + out["grad_mlp"] @ dm
        assert abs(fd - an) < 1e-6 * (abs(an) + 1e-3)
    # the output bias does not enter the Laplacian
    assert out["grad_mlp"][-1] == 0.0
