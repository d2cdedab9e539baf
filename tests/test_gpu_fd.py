"""GPU parity of the INGP-FD comparator (hashenc_fd_residual) against the oracle.

Bars, derived from the arithmetic: the stencil values u within 1e-5 normwise (the forward
bar).  The FD Laplacian multiplies the error of every u by up to 1/eps^2, so r is held to
    |r_gpu - r_ref| <= 1e-5 max|r_ref| + (4d / eps^2) (max|u_gpu - u_ref| + 2^-22 max|u|),
that is, to the propagation of the measured u error plus the fp32 rounding of the stencil
sum.  The gradients inherit the seeds' relative error, and are themselves second
differences over the stencil (sum_s c_s du_s/dtheta): the fp32 rounding of each stencil
point's term, at most about 2 gamma_64 = 2^-17 relative (two chained 64-term fp32 products),
is amplified by the stencil's cancellation
    kappa = max_p sum_s |c_s| |u_ps - bo| / max_p |Lap u_p|     (oracle values),
so the gradients are held normwise per block to 1e-4 + 2 max|r_gpu - r_ref| / max|r_ref|
+ kappa 2^-17.
"""
import numpy as np
import pytest
import torch

from multiresolution_hash_grid_multires_amd import api
from multiresolution_hash_grid_multires_amd import inputs as I
from tests.test_gpu_residual import _close, _mlp_blocks

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV, torch.float32)


def _run_gpu(spec, mlp, eps, x, params, mlp_params, with_grads=True):
    enc = api.HashGridEncoding(spec)
    n, d = x.shape
    ws = torch.empty(api.hashenc_fd_residual_workspace_size(enc.handle, mlp, n), dtype=torch.uint8, device=DEV)
    us = torch.full((n, 2 * d + 1), float("nan"), device=DEV)
    r = torch.empty(n, device=DEV)
    loss = torch.empty(1, device=DEV)
    gp = torch.zeros(enc.n_params, device=DEV) if with_grads else None
    gm = torch.zeros(mlp_params.size, device=DEV) if with_grads else None
    api.hashenc_fd_residual(enc.handle, mlp, eps, _dev(x), _dev(params), _dev(mlp_params), us, r, loss, gp, gm, ws)
    torch.cuda.synchronize()
    return {"u_stencil": us.cpu().numpy(), "r": r.cpu().numpy(), "loss": float(loss.item()),
            "grad_params": None if gp is None else gp.cpu().numpy(),
            "grad_mlp": None if gm is None else gm.cpu().numpy()}


def _r_bound(got, ref, d, eps):
    du = np.max(np.abs(got["u_stencil"] - ref["u_stencil"]))
    umax = np.max(np.abs(ref["u_stencil"]))
    return 1e-5 * np.max(np.abs(ref["r"])) + (4 * d / eps ** 2) * (du + 2.0 ** -22 * umax)


def _kappa(ref, x, d, eps, bo):
    c = np.array([-2.0 * d] + [1.0] * (2 * d)) / eps ** 2
    g = -d * np.pi ** 2 * np.prod(np.sin(np.pi * x.astype(np.float64)), axis=1)
    lap = ref["r"] + g
    return float(np.max(np.abs(ref["u_stencil"] - bo) @ np.abs(c)) / np.max(np.abs(lap)))


def _assembly_close(got, x, d, eps):
    """The residual the GPU returns against the central-difference formula evaluated in fp64
    on the GPU's own stencil values: r = sum_i (u_{2i+1} - 2 u_0 + u_{2i+2}) / eps^2 - g(x).
    The returned u are fp32 roundings (each within 2^-24 |u| of the value the kernel
    differenced), which the stencil weights sum_s |c_s| = 4d / eps^2 carry into r; beyond that
    the assembly is held to 1e-5 of max|r|, whatever the error of u itself."""
    u = got["u_stencil"].astype(np.float64)
    lap = sum(u[:, 2 * i + 1] - 2.0 * u[:, 0] + u[:, 2 * i + 2] for i in range(d)) / eps ** 2
    g = -d * np.pi ** 2 * np.prod(np.sin(np.pi * x.astype(np.float64)), axis=1)
    r64 = lap - g
    err = float(np.max(np.abs(got["r"] - r64)))
    bar = 1e-5 * float(np.max(np.abs(r64))) + (4 * d / eps ** 2) * 2.0 ** -24 * float(np.max(np.abs(u)))
    assert err <= bar, f"FD assembly: {err:.3e} vs bar {bar:.3e}"


def _compare(orc, spec, hidden, depth, omega, eps, x, params, mlp_params):
    d = spec["d"]
    mlp = api.Mlp(spec["L"] * spec["F"], hidden, depth, omega)
    got = _run_gpu(spec, mlp, eps, x, params, mlp_params)
    _assembly_close(got, x, d, eps)
    ref = orc.fd_residual(spec, hidden, depth, omega, eps, x, params, mlp_params)
    _close(got["u_stencil"], ref["u_stencil"], 1e-5, "u at the stencil points")
    dr = np.max(np.abs(got["r"] - ref["r"]))
    assert dr <= _r_bound(got, ref, d, eps), f"r: {dr:.3e} vs bound {_r_bound(got, ref, d, eps):.3e}"
    rel_r = dr / np.max(np.abs(ref["r"]))
    assert abs(got["loss"] - float(np.mean(got["r"].astype(np.float64) ** 2))) <= 1e-5 * got["loss"]
    assert abs(got["loss"] - ref["loss"]) <= (1e-5 + 2 * rel_r) * ref["loss"]
    gtol = 1e-4 + 2 * rel_r + _kappa(ref, x, d, eps, mlp_params[-1]) * 2.0 ** -17
    # Deeper networks: the second differences over the stencil copies act on every hidden
    # layer's activations, whose own cancellation can exceed the output's (kappa above).  The
    # oracle's fp32 evaluation of the same arithmetic measures that floor per block; the GPU
    # is held to three times it where it exceeds gtol.
    ref32 = orc.fd_residual(spec, hidden, depth, omega, eps, x, params, mlp_params, precision="f32") \
        if depth > 2 else None
    for name, off, size in _mlp_blocks(spec["L"] * spec["F"], hidden, depth):
        if name == f"b{depth}":
            assert got["grad_mlp"][off] == 0.0  # the output bias cancels in the stencil
            continue
        tol = gtol
        if ref32 is not None:
            b64, b32 = ref["grad_mlp"][off:off + size], ref32["grad_mlp"][off:off + size]
            tol = max(tol, 3.0 * float(np.max(np.abs(b32 - b64))) / max(float(np.max(np.abs(b64))), 1e-30))
        _close(got["grad_mlp"][off:off + size], ref["grad_mlp"][off:off + size], tol, f"grad {name}")
    lay = orc.layout(spec)
    nt, L = lay["offset"].shape
    for k in range(nt):
        for l in range(L):
            o, m = lay["offset"][k, l], lay["rows"][k, l] * lay["width"][k, l]
            tol = gtol
            if ref32 is not None:
                b64, b32 = ref["grad_params"][o:o + m], ref32["grad_params"][o:o + m]
                tol = max(tol, 3.0 * float(np.max(np.abs(b32 - b64))) / max(float(np.max(np.abs(b64))), 1e-30))
            _close(got["grad_params"][o:o + m], ref["grad_params"][o:o + m], tol, f"grad level {l}")
    return got, ref


@pytest.mark.parametrize("d,depth,hidden,omega,L", [(3, 2, 64, 3.0, 4), (3, 1, 32, 5.0, 8), (2, 2, 16, 2.0, 4),
                                                    # depth 3 and 4: the vector-ALU network kernel, as in
                                                    # the pages' depth ablation (depth 2 against 4)
                                                    (3, 3, 64, 3.0, 4), (3, 4, 32, 3.0, 8), (2, 4, 64, 2.0, 4)])
def test_fd_parity_shapes(orc, d, depth, hidden, omega, L):
    spec = {"d": d, "L": L, "F": 2, "kind": "dlinear", "T": [1 << 12], "n_min": 4, "n_max": 60 if d == 3 else 150}
    lay = orc.layout(spec)
    assert not lay["dense"][0, -1]  # hashed levels with collisions
    rng = np.random.default_rng(depth * 10 + d)
    params = (0.3 * rng.standard_normal(lay["n_params"])).astype(np.float32)
    mlp_params = I.siren_mlp(11, L * 2, hidden, depth)
    x = rng.random((1000 + 37, d), dtype=np.float32)  # several 16-point tiles, ragged tail
    e = np.array([[0.0] * d, [1.0 - 2 ** -24] * d, [2.0 ** -6] * d], np.float32)
    x[: e.shape[0]] = e                               # stencils clamped at the faces
    _compare(orc, spec, hidden, depth, omega, 2.0 ** -5, x, params, mlp_params)


def test_fd_parity_workload_settings(orc):
    # the comparator workload's encoder, network, omega and step, on 1536 of its points
    W = I.WORKLOADS["fd_residual3d"]
    spec, m = W["spec"], W["mlp"]
    lay = orc.layout(spec)
    params = I.tables(W["id"], lay["n_params"], W["tables"])
    mlp_params = I.siren_mlp(W["id"], 32, m["hidden"], m["depth"])
    xf = I.points(W["id"], W["n_points"], 3, clustered_half=True)
    x = np.concatenate([xf[:768], xf[-768:]])
    _compare(orc, spec, m["hidden"], m["depth"], m["omega"], W["fd_eps"], x, params, mlp_params)


def test_fd_with_active_levels(orc):
    spec = {"d": 3, "L": 4, "F": 2, "kind": "dlinear", "T": [1 << 12], "n_min": 4, "n_max": 60, "active_levels": 2}
    lay = orc.layout(spec)
    rng = np.random.default_rng(31)
    params = (0.3 * rng.standard_normal(lay["n_params"])).astype(np.float32)
    mlp_params = I.siren_mlp(12, 8, 32, 2)
    x = rng.random((700, 3), dtype=np.float32)
    got, _ = _compare(orc, spec, 32, 2, 3.0, 2.0 ** -5, x, params, mlp_params)
    for l in (2, 3):  # inactive levels: no gradient
        o, m = lay["offset"][0, l], lay["rows"][0, l] * lay["width"][0, l]
        assert not np.any(got["grad_params"][o:o + m])


def test_fd_atomic_backward_path(orc):
    # a table too large for the binned backward's LDS counters: the fp32-atomic backward reads
    # the SIREN kernel's level-major upstream
    # (eight hashed levels of 1024 bins each: the scatter's per-bin LDS arrays exceed the budget)
    spec = {"d": 3, "L": 8, "F": 8, "kind": "dlinear", "T": [1 << 21], "n_min": 128, "n_max": 4096}
    h = api.hashenc_create(spec)
    assert api.hashenc_backward_workspace_size(h, 1000) == 0
    lay = orc.layout(spec)
    rng = np.random.default_rng(41)
    params = (0.3 * rng.standard_normal(lay["n_params"])).astype(np.float32)
    mlp_params = I.siren_mlp(13, 64, 32, 1)
    x = rng.random((600, 3), dtype=np.float32)
    _compare(orc, spec, 32, 1, 3.0, 2.0 ** -5, x, params, mlp_params)


def test_fd_full_workload(orc):
    """2^21 points (eight internal chunks of 2d+1 stencil sets, the last 64 points): sampled stencil values and
    residuals against the oracle, the loss as the mean square of the returned residuals, and
    the gradients as the size-weighted sum of the two halves' gradients."""
    W = I.WORKLOADS["fd_residual3d"]
    spec, m = W["spec"], W["mlp"]
    eps = W["fd_eps"]
    enc = api.HashGridEncoding(spec)
    mlp = api.Mlp(32, m["hidden"], m["depth"], m["omega"])
    params = I.tables(W["id"], enc.n_params, W["tables"])
    mlp_params = I.siren_mlp(W["id"], 32, m["hidden"], m["depth"])
    x = I.points(W["id"], W["n_points"], 3, clustered_half=True)
    n = x.shape[0]
    full = _run_gpu(spec, mlp, eps, x, params, mlp_params)
    idx = np.sort(np.random.default_rng(4).choice(n, 1024, replace=False))
    idx[-1] = n - 1
    ref = orc.fd_residual(spec, m["hidden"], m["depth"], m["omega"], eps, x[idx], params, mlp_params)
    sub = {"u_stencil": full["u_stencil"][idx], "r": full["r"][idx]}
    _close(sub["u_stencil"], ref["u_stencil"], 1e-5, "sampled u")
    assert np.max(np.abs(sub["r"] - ref["r"])) <= _r_bound(sub, ref, 3, eps)
    assert abs(full["loss"] - float(np.mean(full["r"].astype(np.float64) ** 2))) <= 1e-5 * full["loss"]
    h = n // 2
    a = _run_gpu(spec, mlp, eps, x[:h], params, mlp_params)
    b = _run_gpu(spec, mlp, eps, x[h:], params, mlp_params)
    np.testing.assert_array_equal(np.concatenate([a["r"], b["r"]]), full["r"])
    _close(full["grad_mlp"], 0.5 * (a["grad_mlp"].astype(np.float64) + b["grad_mlp"]), 1e-4, "grad_mlp halves")
    _close(full["grad_params"], 0.5 * (a["grad_params"].astype(np.float64) + b["grad_params"]), 1e-4,
           "grad_params halves")


def test_fd_argument_errors():
    from multiresolution_hash_grid_multires_amd._lib import HASHENC_EINVAL, HASHENC_EUNSUPPORTED, HashencError
    spec = {"d": 3, "L": 2, "F": 2, "kind": "dlinear", "T": [1 << 10], "n_min": 4, "n_max": 16}
    enc = api.HashGridEncoding(spec)
    x = torch.rand(64, 3, device=DEV)
    p = torch.zeros(enc.n_params, device=DEV)
    loss = torch.empty(1, device=DEV)
    ok = api.Mlp(4, 16, 2, 30.0)
    mp = torch.zeros(api.mlp_param_count(4, 16, 2), device=DEV)
    wsz = api.hashenc_fd_residual_workspace_size(enc.handle, ok, 64)
    ws = torch.empty(wsz, dtype=torch.uint8, device=DEV)
    for mlp, eps, code in [(api.Mlp(4, 16, 5, 30.0), 0.01, HASHENC_EUNSUPPORTED),
                           (api.Mlp(6, 16, 2, 30.0), 0.01, HASHENC_EINVAL),
                           (ok, 0.0, HASHENC_EINVAL), (ok, float("inf"), HASHENC_EINVAL)]:
        mpm = torch.zeros(api.mlp_param_count(mlp.n_in, mlp.hidden, mlp.depth), device=DEV)
        with pytest.raises(HashencError) as e:
            api.hashenc_fd_residual(enc.handle, mlp, eps, x, p, mpm, None, None, loss, None, None, ws)
        assert e.value.code == code
    with pytest.raises(HashencError) as e:  # workspace too small
        api.hashenc_fd_residual(enc.handle, ok, 0.01, x, p, mp, None, None, loss, None, None, ws[: wsz // 2])
    assert e.value.code == HASHENC_EINVAL
    herm = api.HashGridEncoding({"d": 3, "L": 2, "F": 2, "kind": "hermite", "T": [1 << 10] * 4, "n_min": 4,
                                 "n_max": 16, "d2_mode": "laplacian"})
    with pytest.raises(HashencError) as e:
        api.hashenc_fd_residual_workspace_size(herm.handle, ok, 64)
    assert e.value.code == HASHENC_EUNSUPPORTED
