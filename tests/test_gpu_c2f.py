"""GPU parity of coarse-to-fine level activation (derived handles computing the first
n_active levels) against the oracle with the same active level count.

Bars as for the full encoder: forward within 1e-5 and gradients within 1e-4 normwise per
level block; the columns of inactive levels exactly zero (outputs are pre-filled with a
sentinel, so they must be written), and the gradient blocks of inactive levels untouched
bit for bit (gradients accumulate into a pre-filled buffer).
"""
import numpy as np
import pytest
import torch

from multiresolution_hash_grid_multires_amd import api
from multiresolution_hash_grid_multires_amd import inputs as I
from tests.test_gpu_parity import (BWD_TOL, DEV, FWD_TOL, PATHS, _blocks_close, _dev, _points, _tables,
                                   _upstream_shapes)
from tests.test_gpu_residual import _compare

pytestmark = pytest.mark.gpu

CONFIGS = ["dlinear2d_L4_T12", "hermite2d_L8_T14", "dlinear3d_L16_T19", "hermite3d_L16_T19"]


def _active_counts(L):
    return sorted({1, L // 2, L - 1})


def _outputs(enc, n, fill):
    return {k: torch.full(v, fill, device=DEV) for k, v in enc.output_shapes(n).items()}


def _check_forward(orc, spec, a, x, params, got, what):
    L, F = spec["L"], spec["F"]
    ref = orc.forward(dict(spec, active_levels=a), x, params)
    for k, r in zip(("gamma", "dgamma", "d2gamma"), ref):
        if k not in got:
            continue
        g = got[k].cpu().numpy()
        assert not np.any(g[..., a * F:]), f"{what} {k}: inactive columns not zero"
        _blocks_close(g, r, spec, FWD_TOL, f"{what} {k} active={a}")
    return ref


@pytest.mark.parametrize("name", CONFIGS)
def test_masked_forward_parity(orc, name):
    spec = I.WORKLOADS[name]["spec"]
    lay = orc.layout(spec)
    params = _tables(name, lay["n_params"])
    x = _points(name, 3 * 1024 + 37)
    xt, pt = _dev(x), _dev(params)
    base = api.HashGridEncoding(spec)
    for a in _active_counts(spec["L"]):
        enc = api.HashGridEncoding(spec)
        enc.set_active_levels(a)
        assert enc.active_levels == a
        direct = _outputs(enc, x.shape[0], float("nan"))
        api.hashenc_forward(enc.handle, xt, pt, direct["gamma"], direct.get("dgamma"), direct.get("d2gamma"))
        ws = _outputs(enc, x.shape[0], 7.0)
        api.hashenc_forward_ws(enc.handle, xt, pt, ws["gamma"], ws.get("dgamma"), ws.get("d2gamma"),
                               enc.workspace(x.shape[0]))
        full = base.forward(xt, pt)
        torch.cuda.synchronize()
        _check_forward(orc, spec, a, x, params, direct, "forward")
        for k in direct:
            assert torch.equal(direct[k], ws[k]), f"forward_ws {k} differs from forward"
            # active columns: the same bits as the full encoder's
            assert torch.equal(direct[k][..., : a * spec["F"]], full[k][..., : a * spec["F"]]), k


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("name", CONFIGS)
def test_masked_backward_parity(orc, name, path):
    W = I.WORKLOADS[name]
    spec = W["spec"]
    lay = orc.layout(spec)
    n = 3 * 1024 + 37
    x = _points(name, n)
    ups = I.upstream(W["id"], _upstream_shapes(spec, n))   # nonzero on inactive columns too
    init = np.random.default_rng(11).standard_normal(lay["n_params"]).astype(np.float32)
    xt = _dev(x)
    U = [_dev(u) for u in ups] + [None] * (3 - len(ups))
    for a in _active_counts(spec["L"]):
        enc = api.HashGridEncoding(dict(spec, active_levels=a))
        grad = _dev(init)
        if path == "binned":
            enc.backward_binned(xt, grad, *U)
        else:
            enc.backward(xt, grad, *U)
        torch.cuda.synchronize()
        got = grad.cpu().numpy()
        ref = orc.backward(dict(spec, active_levels=a), x, *ups, n_params=lay["n_params"])
        nt = lay["offset"].shape[0]
        for k in range(nt):
            for l in range(spec["L"]):
                o, m = lay["offset"][k, l], lay["rows"][k, l] * lay["width"][k, l]
                if l >= a:
                    assert np.array_equal(got[o:o + m], init[o:o + m]), f"table {k} level {l} touched"
                    continue
                delta = got[o:o + m].astype(np.float64) - init[o:o + m]
                err = np.max(np.abs(delta - ref[o:o + m]))
                # the fp32 accumulate into the pre-filled values rounds at |init| scale
                scale = np.max(np.abs(ref[o:o + m]))
                slack = 2 * np.finfo(np.float32).eps * np.max(np.abs(init[o:o + m]))
                assert err <= BWD_TOL * scale + slack, f"table {k} level {l} active={a}: {err:.3e}"


def test_masked_full_size_forward_sampled(orc):
    # the headline-sized batch through the workspace path, sampled against the oracle
    name = "dlinear3d_L16_T19"
    W = I.WORKLOADS[name]
    spec = W["spec"]
    lay = orc.layout(spec)
    params = _tables(name, lay["n_params"])
    n = W["n_points"]
    x = I.points(W["id"], n, spec["d"], W.get("clustered_half", False))
    enc = api.HashGridEncoding(dict(spec, active_levels=9))
    out = _outputs(enc, n, float("nan"))
    api.hashenc_forward_ws(enc.handle, _dev(x), _dev(params), out["gamma"], None, None, enc.workspace(n))
    torch.cuda.synchronize()
    g = out["gamma"]
    assert not bool(g[:, 9 * spec["F"]:].abs().sum().item())
    idx = np.sort(np.random.default_rng(3).choice(n, 2048, replace=False))
    idx[-1] = n - 1
    ref = orc.forward(dict(spec, active_levels=9), x[idx], params)[0]
    _blocks_close(g.cpu().numpy()[idx], ref, spec, FWD_TOL, "sampled gamma")


@pytest.mark.parametrize("a", [1, 3])
def test_masked_residual_parity(orc, a):
    spec = {"d": 3, "L": 4, "F": 2, "kind": "hermite", "T": [1 << 12] * 4, "n_min": 4, "n_max": 40,
            "d2_mode": "laplacian", "active_levels": a}
    lay = orc.layout(spec)
    rng = np.random.default_rng(20 + a)
    params = (0.05 * rng.standard_normal(lay["n_params"])).astype(np.float32)
    x = rng.random((1500, 3), dtype=np.float32)
    for depth, hidden, omega in [(2, 32, 10.0), (3, 16, 3.0)]:  # matrix-core and vector kernels
        mlp_params = I.siren_mlp(5, 8, hidden, depth)
        _compare(orc, spec, hidden, depth, omega, x, params, mlp_params)


def test_masked_indices_cover_every_level(orc):
    # the lookup-stage export ignores the activation: every level's rows, bit-exact
    name = "hermite2d_L8_T14"
    spec = I.WORKLOADS[name]["spec"]
    x = _points(name, 1000)
    h = api.hashenc_derive_active(api.hashenc_create(spec), 2)
    out = torch.empty((x.shape[0], spec["L"], 4), dtype=torch.int32, device=DEV)
    api.hashenc_debug_indices(h, _dev(x), 1, out)
    assert np.array_equal(out.cpu().numpy(), orc.indices(spec, x, 1))
