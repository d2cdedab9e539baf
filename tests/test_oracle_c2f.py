"""Oracle pins for the coarse-to-fine level activation.

Hermite-NGP notes (m0rtzz.github.io), section 方法详解, key design 3: training starts on the
coarse levels only and activates finer levels one at a time, L_active(t) = min(L, L0 +
floor(t / tau)).  Reading: L_active counts the active levels (levels l < L_active); an
inactive level encodes to zero and receives no gradient, and the encoding keeps its full
L*F width so the network's input does not change shape during the schedule.

Pinned against things other than the masking code itself: the schedule by its closed form;
the masked encoder by a separately configured encoder that simply has fewer levels (explicit
resolutions, its own parameter layout); the masked backward by that truncated encoder's
backward; the masked residual by the truncated residual with the first-layer weights of the
inactive inputs removed.
"""
import numpy as np
import pytest


def _pts(n, d, seed):
    return np.random.default_rng(seed).random((n, d), dtype=np.float32)


SPECS = [
    {"d": 3, "L": 5, "F": 2, "kind": "dlinear", "T": [1 << 9], "n_min": 2, "n_max": 40},
    {"d": 2, "L": 4, "F": 4, "kind": "dlinear", "T": [1 << 7], "n_min": 3, "n_max": 50},
    {"d": 3, "L": 4, "F": 2, "kind": "hermite", "T": [1 << 9] * 4, "n_min": 2, "n_max": 30,
     "d2_mode": "diag"},
    {"d": 2, "L": 4, "F": 1, "kind": "hermite", "T": [1 << 7, 1 << 6, 1 << 8], "n_min": 3,
     "n_max": 40, "d2_mode": "laplacian"},
]


def _ids(s):
    return f"{s['kind']}{s['d']}d-F{s['F']}"


def _truncated(orc, spec, a):
    """The same encoder configured with only its first a levels (explicit resolutions)."""
    res = orc.resolutions(spec)[:a]
    t = {k: v for k, v in spec.items() if k not in ("n_min", "n_max", "growth", "active_levels")}
    t.update(L=a, resolutions=res)
    return t


def _param_map(orc, spec, a):
    """Index array: truncated parameter j lives at full parameter idx[j]."""
    full, trunc = orc.layout(spec), orc.layout(_truncated(orc, spec, a))
    idx = np.zeros(trunc["n_params"], np.int64)
    for k in range(full["offset"].shape[0]):
        for l in range(a):
            size = full["rows"][k, l] * full["width"][k, l]
            assert size == trunc["rows"][k, l] * trunc["width"][k, l]
            t0, f0 = trunc["offset"][k, l], full["offset"][k, l]
            idx[t0:t0 + size] = np.arange(f0, f0 + size)
    return idx


def _upstream(spec, n, rng):
    LF, d = spec["L"] * spec["F"], spec["d"]
    gg = rng.standard_normal((n, LF))
    if spec["kind"] != "hermite":
        return gg, None, None
    gd = rng.standard_normal((n, d, LF))
    g2 = rng.standard_normal((n, d, LF)) if spec.get("d2_mode") == "diag" else rng.standard_normal((n, LF))
    return gg, gd, g2


def test_schedule_closed_form(orc):
    L, L0, tau = 16, 4, 250
    assert orc.c2f_active_levels(L, L0, 0, tau) == L0
    assert orc.c2f_active_levels(L, L0, tau - 1, tau) == L0
    assert orc.c2f_active_levels(L, L0, tau, tau) == L0 + 1
    assert orc.c2f_active_levels(L, L0, 5 * tau + 3, tau) == L0 + 5
    assert orc.c2f_active_levels(L, L0, (L - L0) * tau, tau) == L
    assert orc.c2f_active_levels(L, L0, 10 ** 12, tau) == L
    assert orc.c2f_active_levels(L, L, 0, 1) == L
    # monotone, one level per interval
    seq = [orc.c2f_active_levels(L, 1, t, 3) for t in range(60)]
    assert seq == [min(L, 1 + t // 3) for t in range(60)]
    for bad in [(0, 1, 0, 1), (4, 0, 0, 1), (4, 1, -1, 1), (4, 1, 0, 0)]:
        with pytest.raises(ValueError):
            orc.c2f_active_levels(*bad)


@pytest.mark.parametrize("spec", SPECS, ids=_ids)
@pytest.mark.parametrize("which", ["one", "all_but_one"])
def test_masked_forward_equals_truncated_encoder(orc, spec, which):
    L, F = spec["L"], spec["F"]
    a = 1 if which == "one" else L - 1
    lay = orc.layout(spec)
    theta = np.random.default_rng(3).standard_normal(lay["n_params"])
    x = _pts(300, spec["d"], 4)
    masked = orc.forward(dict(spec, active_levels=a), x, theta)
    trunc = orc.forward(_truncated(orc, spec, a), x, theta[_param_map(orc, spec, a)])
    for m, t in zip(masked, trunc):
        if m is None:
            continue
        assert np.array_equal(m[..., :a * F], t)            # same arithmetic, same order
        assert not np.any(m[..., a * F:])                     # inactive columns are zero
    # and the active columns differ from nothing: the unmasked encoder agrees on them
    full = orc.forward(spec, x, theta)
    for m, f in zip(masked, full):
        if m is not None:
            assert np.array_equal(m[..., :a * F], f[..., :a * F])
            assert np.any(f[..., a * F:])


@pytest.mark.parametrize("spec", SPECS, ids=_ids)
def test_masked_backward_equals_truncated_encoder(orc, spec):
    L, F = spec["L"], spec["F"]
    a = L // 2
    lay = orc.layout(spec)
    x = _pts(300, spec["d"], 5)
    G = _upstream(spec, 300, np.random.default_rng(6))   # nonzero in the inactive columns too
    grad = orc.backward(dict(spec, active_levels=a), x, *G)
    idx = _param_map(orc, spec, a)
    Gt = [None if g is None else np.ascontiguousarray(g[..., :a * F]) for g in G]
    gt = orc.backward(_truncated(orc, spec, a), x, *Gt)
    assert np.array_equal(grad[idx], gt)
    inactive = np.ones(lay["n_params"], bool)
    inactive[idx] = False
    assert inactive.any() and not np.any(grad[inactive])


@pytest.mark.parametrize("spec", [SPECS[0], SPECS[2]], ids=["dlinear", "hermite"])
def test_masked_adjoint_identity(orc, spec):
    a = 2
    ms = dict(spec, active_levels=a)
    rng = np.random.default_rng(7)
    n_params = orc.layout(spec)["n_params"]
    x = _pts(200, spec["d"], 8)
    G = _upstream(spec, 200, rng)
    grad = orc.backward(ms, x, *G)
    dtheta = rng.standard_normal(n_params)
    outs = orc.forward(ms, x, dtheta)
    rhs = sum(float(np.sum(o * g)) for o, g in zip(outs, G) if g is not None)
    assert abs(float(grad @ dtheta) - rhs) <= 1e-11 * (abs(rhs) + np.sum(np.abs(grad)))


def test_masked_residual_equals_truncated_network(orc):
    # inactive inputs are zero, so the masked network equals the truncated encoder feeding a
    # first layer without those input columns; their first-layer gradients are zero
    spec = {"d": 3, "L": 3, "F": 2, "kind": "hermite", "T": [1 << 9] * 4, "resolutions": [3, 5, 8],
            "d2_mode": "laplacian"}
    a, H, depth, omega = 2, 8, 2, 1.5
    LF, aF = spec["L"] * spec["F"], a * spec["F"]
    rng = np.random.default_rng(9)
    theta = rng.uniform(-0.3, 0.3, orc.layout(spec)["n_params"])
    n_mlp = orc.mlp_param_count(LF, H, depth)
    mlp = rng.uniform(-0.5, 0.5, n_mlp)
    W1 = mlp[:H * LF].reshape(H, LF)
    mlp_t = np.concatenate([W1[:, :aF].ravel(), mlp[H * LF:]])
    x = _pts(64, 3, 10)
    m = orc.residual(dict(spec, active_levels=a), H, depth, omega, x, theta, mlp)
    t = orc.residual(_truncated(orc, spec, a), H, depth, omega, x, theta[_param_map(orc, spec, a)], mlp_t)
    for key in ("u", "grad_u", "lap_u", "r"):
        assert np.allclose(m[key], t[key], rtol=1e-12, atol=1e-12)
    assert m["loss"] == pytest.approx(t["loss"], rel=1e-12)
    idx = _param_map(orc, spec, a)
    assert np.allclose(m["grad_params"][idx], t["grad_params"], rtol=1e-10, atol=1e-14)
    rest = np.ones(theta.size, bool)
    rest[idx] = False
    assert not np.any(m["grad_params"][rest])
    gW1 = m["grad_mlp"][:H * LF].reshape(H, LF)
    assert not np.any(gW1[:, aF:])
    assert np.allclose(gW1[:, :aF].ravel(), t["grad_mlp"][:H * aF], rtol=1e-10, atol=1e-14)
    assert np.allclose(m["grad_mlp"][H * LF:], t["grad_mlp"][H * aF:], rtol=1e-10, atol=1e-14)
