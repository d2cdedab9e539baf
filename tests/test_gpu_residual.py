"""GPU parity of the fused PINN residual step against the oracle.

Bars: residual r and loss within 1e-5 (normwise over r), gradients within 1e-4 normwise per
table-level block and per MLP parameter block.
"""
import numpy as np
import pytest
import torch

from multiresolution_hash_grid_multires_amd import api
from multiresolution_hash_grid_multires_amd import inputs as I

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
NAME = "pinn_residual3d"


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV, torch.float32)


def _mlp_blocks(n_in, hidden, depth):
    out, off = [], 0
    for k in range(depth + 1):
        fi = n_in if k == 0 else hidden
        fo = 1 if k == depth else hidden
        out.append((f"W{k}", off, fi * fo)); off += fi * fo
        out.append((f"b{k}", off, fo)); off += fo
    return out


def _close(a, b, tol, what):
    err = float(np.max(np.abs(a - b))) if a.size else 0.0
    scale = float(np.max(np.abs(b))) if b.size else 0.0
    assert err <= tol * max(scale, 1e-30), f"{what}: {err:.3e} vs scale {scale:.3e}"


def _run_gpu(spec, mlp, x, params, mlp_params, want_grads=True):
    enc = api.HashGridEncoding(spec)
    n = x.shape[0]
    ws = torch.empty(api.hashenc_residual_workspace_size(enc.handle, mlp, n), dtype=torch.uint8, device=DEV)
    r = torch.empty(n, device=DEV)
    loss = torch.empty(1, device=DEV)
    gp = torch.zeros(enc.n_params, device=DEV) if want_grads else None
    gm = torch.zeros(mlp_params.size, device=DEV) if want_grads else None
    api.hashenc_residual(enc.handle, mlp, _dev(x), _dev(params), _dev(mlp_params), r, loss, gp, gm, ws)
    torch.cuda.synchronize()
    return (r.cpu().numpy(), float(loss.item()),
            None if gp is None else gp.cpu().numpy(), None if gm is None else gm.cpu().numpy())


def _compare(orc, spec, hidden, depth, omega, x, params, mlp_params):
    lay = orc.layout(spec)
    mlp = api.Mlp(spec["L"] * spec["F"], hidden, depth, omega)
    r, loss, gp, gm = _run_gpu(spec, mlp, x, params, mlp_params)
    ref = orc.residual(spec, hidden, depth, omega, x, params, mlp_params)
    _close(r, ref["r"], 1e-5, "residual")
    assert abs(loss - ref["loss"]) <= 1e-5 * ref["loss"]
    for name, off, size in _mlp_blocks(spec["L"] * spec["F"], hidden, depth):
        _close(gm[off:off + size], ref["grad_mlp"][off:off + size], 1e-4, f"grad {name}")
    nt, L = lay["offset"].shape
    for k in range(nt):
        for l in range(L):
            o, m = lay["offset"][k, l], lay["rows"][k, l] * lay["width"][k, l]
            _close(gp[o:o + m], ref["grad_params"][o:o + m], 1e-4, f"grad table {k} level {l}")


def test_residual_parity_pinn_workload(orc):
    W = I.WORKLOADS[NAME]
    spec, m = W["spec"], W["mlp"]
    lay = orc.layout(spec)
    params = I.tables(W["id"], lay["n_params"], W["tables"])
    mlp_params = I.siren_mlp(W["id"], spec["L"] * spec["F"], m["hidden"], m["depth"])
    # the first and last 1.5k points of the workload: uniform and clustered halves
    x_full = I.points(W["id"], W["n_points"], spec["d"], clustered_half=True)
    x = np.concatenate([x_full[:1536], x_full[-1536:]])
    _compare(orc, spec, m["hidden"], m["depth"], m["omega"], x, params, mlp_params)


@pytest.mark.parametrize("depth", [3, 4])
def test_residual_parity_pinn_deeper(orc, depth):
    """The PINN workload's encoder and network width at depth 3 and 4 (the pages' depth
    ablation): 3 072 of its points, uniform and clustered, on the matrix-core kernel."""
    W = I.WORKLOADS[NAME]
    spec, m = W["spec"], W["mlp"]
    lay = orc.layout(spec)
    params = I.tables(W["id"], lay["n_params"], W["tables"])
    mlp_params = I.siren_mlp(W["id"] + depth, spec["L"] * spec["F"], m["hidden"], depth)
    x_full = I.points(W["id"], W["n_points"], spec["d"], clustered_half=True)
    x = np.concatenate([x_full[:1536], x_full[-1536:]])
    _compare(orc, spec, m["hidden"], depth, m["omega"], x, params, mlp_params)


@pytest.mark.parametrize("d,depth,hidden,omega", [(3, 1, 16, 3.0), (2, 2, 32, 30.0), (3, 3, 64, 10.0),
                                                  (3, 4, 64, 10.0), (2, 4, 48, 30.0)])
def test_residual_parity_shapes(orc, d, depth, hidden, omega):
    spec = {"d": d, "L": 4, "F": 2, "kind": "hermite", "T": [1 << 12] * (d + 1), "n_min": 4,
            "n_max": 40, "d2_mode": "diag"}
    lay = orc.layout(spec)
    rng = np.random.default_rng(depth)
    params = (0.05 * rng.standard_normal(lay["n_params"])).astype(np.float32)
    mlp_params = I.siren_mlp(7, 8, hidden, depth)
    x = rng.random((1000, d), dtype=np.float32)
    _compare(orc, spec, hidden, depth, omega, x, params, mlp_params)


def test_residual_full_size(orc):
    """2^21 + 777 points (one full 2^21-point internal chunk and a ragged one): sampled
    residuals against the oracle; the loss is the mean square of the returned residuals; and
    the gradients equal the size-weighted sum of the gradients of the two halves computed by
    separate calls (each half fits one chunk)."""
    W = I.WORKLOADS[NAME]
    spec, m = W["spec"], W["mlp"]
    enc = api.HashGridEncoding(spec)
    mlp = api.Mlp(32, m["hidden"], m["depth"], m["omega"])
    params = I.tables(W["id"], enc.n_params, W["tables"])
    mlp_params = I.siren_mlp(W["id"], 32, m["hidden"], m["depth"])
    x = I.points(W["id"], W["n_points"] + 777, 3, clustered_half=True)
    n = x.shape[0]
    r, loss, gp, gm = _run_gpu(spec, mlp, x, params, mlp_params)
    idx = np.sort(np.random.default_rng(2).choice(n, 1024, replace=False))
    idx[-1] = n - 1
    ref = orc.residual(spec, m["hidden"], m["depth"], m["omega"], x[idx], params, mlp_params)
    _close(r[idx], ref["r"], 1e-5, "sampled residual")
    assert abs(loss - float(np.mean(r.astype(np.float64) ** 2))) <= 1e-5 * loss
    h = n // 2
    ra, la, gpa, gma = _run_gpu(spec, mlp, x[:h], params, mlp_params)
    rb, lb, gpb, gmb = _run_gpu(spec, mlp, x[h:], params, mlp_params)
    np.testing.assert_array_equal(np.concatenate([ra, rb]), r)
    wa, wb = h / n, (n - h) / n
    assert abs(wa * la + wb * lb - loss) <= 1e-5 * loss
    _close(gm, wa * gma.astype(np.float64) + wb * gmb, 1e-4, "grad_mlp halves")
    _close(gp, wa * gpa.astype(np.float64) + wb * gpb, 1e-4, "grad_params halves")


def test_residual_full_size_against_oracle(orc):
    """The PINN workload as the benchmark runs it: all 2^21 points (the uniform half and the
    clustered half) in one call, every residual, the loss and every gradient block -- per
    table-level block and per MLP parameter block -- against the oracle on the same points."""
    W = I.WORKLOADS[NAME]
    spec, m = W["spec"], W["mlp"]
    lay = orc.layout(spec)
    params = I.tables(W["id"], lay["n_params"], W["tables"])
    mlp_params = I.siren_mlp(W["id"], spec["L"] * spec["F"], m["hidden"], m["depth"])
    x = I.points(W["id"], W["n_points"], spec["d"], clustered_half=True)
    assert x.shape[0] == 1 << 21
    _compare(orc, spec, m["hidden"], m["depth"], m["omega"], x, params, mlp_params)


def test_residual_argument_errors():
    from multiresolution_hash_grid_multires_amd._lib import HashencError
    W = I.WORKLOADS[NAME]
    enc = api.HashGridEncoding(W["spec"])
    mlp = api.Mlp(32, 64, 2, 30.0)
    x = torch.zeros((8, 3), device=DEV)
    p = torch.zeros(enc.n_params, device=DEV)
    mp = torch.zeros(6337, device=DEV)
    loss = torch.zeros(1, device=DEV)
    small = torch.empty(16, dtype=torch.uint8, device=DEV)
    with pytest.raises(HashencError):
        api.hashenc_residual(enc.handle, mlp, x, p, mp, None, loss, None, None, small)
    with pytest.raises(HashencError):
        api.hashenc_residual(enc.handle, api.Mlp(16, 64, 2, 30.0), x, p, torch.zeros(api.mlp_param_count(16, 64, 2),
                             device=DEV), None, loss, None, None, small)
    lin = api.HashGridEncoding(I.WORKLOADS["dlinear3d_L16_T19"]["spec"])
    with pytest.raises(HashencError):
        api.hashenc_residual_workspace_size(lin.handle, mlp, 8)
