"""GPU parity of the 4D (space-time) Hermite grid against the oracle: lookup rows bit-exact,
gamma / grad gamma / second derivatives within 1e-5 and gradients within 1e-4, normwise per
level and component (table and level for gradients)."""
import numpy as np
import pytest
import torch

from multiresolution_hash_grid_multires_amd import api
from multiresolution_hash_grid_multires_amd import inputs as I
from tests.test_gpu_parity import BWD_TOL, DEV, FWD_TOL, _blocks_close, _dev, _edge_points, _grad_close

pytestmark = pytest.mark.gpu
NAME = "hermite4d_L8_T16"


def _shapes(spec, n):
    LF, d = spec["L"] * spec["F"], spec["d"]
    return [(n, LF), (n, d, LF), (n, d, LF) if spec.get("d2_mode") == "diag" else (n, LF)]


def _forward(spec, x, params):
    enc = api.HashGridEncoding(spec)
    out = {k: torch.full(v, float("nan"), device=DEV) for k, v in enc.output_shapes(x.shape[0]).items()}
    api.hashenc_forward(enc.handle, _dev(x), _dev(params), out["gamma"], out["dgamma"], out["d2gamma"])
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in out.items()}


def _forward_ws(spec, x, params):
    """The workspace forward: the packed copy of the five tables when F <= 2 and the sizes
    allow it, else the plain forward."""
    enc = api.HashGridEncoding(spec)
    out = {k: torch.full(v, float("nan"), device=DEV) for k, v in enc.output_shapes(x.shape[0]).items()}
    api.hashenc_forward_ws(enc.handle, _dev(x), _dev(params), out["gamma"], out["dgamma"], out["d2gamma"],
                           enc.workspace(x.shape[0]))
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in out.items()}


def _backward(spec, x, ups, n_params, ws=False):
    enc = api.HashGridEncoding(spec)
    grad = torch.zeros(n_params, device=DEV)
    U = [_dev(u) for u in ups]
    (enc.backward_ws if ws else enc.backward)(_dev(x), grad, *U)
    torch.cuda.synchronize()
    return grad.cpu().numpy()


def _points(n, seed):
    x = np.random.default_rng(seed).random((n, 4), dtype=np.float32)
    e = _edge_points(4)
    x[: e.shape[0]] = e
    return x


def _check(orc, spec, x, params, ups_seed):
    got, got_ws = _forward(spec, x, params), _forward_ws(spec, x, params)
    for k, r in zip(("gamma", "dgamma", "d2gamma"), orc.forward(spec, x, params)):
        _blocks_close(got[k], r, spec, FWD_TOL, k)
        _blocks_close(got_ws[k], r, spec, FWD_TOL, f"{k} (workspace forward)")
    lay = orc.layout(spec)
    rng = np.random.default_rng(ups_seed)
    ups = [rng.standard_normal(s).astype(np.float32) for s in _shapes(spec, x.shape[0])]
    ref = orc.backward(spec, x, *ups, n_params=lay["n_params"])
    for ws in (False, True):
        _grad_close(_backward(spec, x, ups, lay["n_params"], ws), ref, lay, BWD_TOL)


def test_hermite4_indices_bit_exact(orc):
    spec = I.WORKLOADS[NAME]["spec"]
    x = _points(4099, 1)
    h = api.hashenc_create(spec)
    for k in range(5):
        out = torch.empty((x.shape[0], spec["L"], 16), dtype=torch.int32, device=DEV)
        api.hashenc_debug_indices(h, _dev(x), k, out)
        got, ref = out.cpu().numpy(), orc.indices(spec, x, k)
        assert np.array_equal(got, ref), f"table {k}: {np.sum(got != ref)} rows differ"


def test_hermite4_parity_workload(orc):
    W = I.WORKLOADS[NAME]
    spec = W["spec"]
    params = I.tables(W["id"], orc.layout(spec)["n_params"], W["tables"])
    _check(orc, spec, _points(3 * 1024 + 37, 2), params, 3)


@pytest.mark.parametrize("F,T,mode", [(1, [1 << 12] * 5, "laplacian"), (4, [1000, 3001, 777, 5000, 64], "diag"),
                                      (8, [1 << 10, 1 << 12, 1 << 11, 1 << 12, 1 << 10], "laplacian"),
                                      # packed copy with smaller power-of-two tables: level 1 is dense
                                      # in tables 0 and 1 and hashed in the others
                                      (2, [1 << 12, 1 << 12, 1 << 10, 1 << 11, 1 << 9], "diag")])
def test_hermite4_shapes(orc, F, T, mode):
    spec = {"d": 4, "L": 3, "F": F, "kind": "hermite", "T": T, "n_min": 3, "n_max": 20, "d2_mode": mode}
    lay = orc.layout(spec)
    rng = np.random.default_rng(F)
    params = rng.standard_normal(lay["n_params"]).astype(np.float32)
    _check(orc, spec, _points(1200, 4 + F), params, 5 + F)


def test_hermite4_full_size(orc):
    W = I.WORKLOADS[NAME]
    spec = W["spec"]
    lay = orc.layout(spec)
    params = I.tables(W["id"], lay["n_params"], W["tables"])
    x = I.points(W["id"], W["n_points"], 4)
    got = _forward(spec, x, params)
    idx = np.sort(np.random.default_rng(6).choice(x.shape[0], 2048, replace=False))
    idx[-1] = x.shape[0] - 1
    for k, r in zip(("gamma", "dgamma", "d2gamma"), orc.forward(spec, x[idx], params)):
        _blocks_close(got[k][idx], r, spec, FWD_TOL, f"sampled {k}")
    m = 1 << 15
    ups = I.upstream(W["id"], _shapes(spec, m))
    ref = orc.backward(spec, x[:m], *ups, n_params=lay["n_params"])
    _grad_close(_backward(spec, x[:m], ups, lay["n_params"]), ref, lay, BWD_TOL)


def test_hermite4_binned_full_size(orc):
    """The binned backward (workspace entry point) on all 2^18 points of the workload, the
    configuration the benchmark times, every gradient block against the oracle."""
    W = I.WORKLOADS[NAME]
    spec = W["spec"]
    lay = orc.layout(spec)
    x = I.points(W["id"], W["n_points"], 4)
    n = x.shape[0]
    assert api.hashenc_backward_workspace_size(api.hashenc_create(spec), n) > 0  # the binned path
    ups = I.upstream(W["id"], _shapes(spec, n))
    ref = orc.backward(spec, x, *ups, n_params=lay["n_params"])
    _grad_close(_backward(spec, x, ups, lay["n_params"], ws=True), ref, lay, BWD_TOL)


@pytest.mark.parametrize("n", [1, 63, 65, 1000])
def test_hermite4_binned_ragged(orc, n):
    """Tiles of 64 points: a single point, one short tile, one full tile and a ragged one, and
    a batch whose levels are split over several workgroups per tile."""
    W = I.WORKLOADS[NAME]
    spec = W["spec"]
    lay = orc.layout(spec)
    x = _points(max(n, 128), 20 + n)[:n]
    ups = I.upstream(W["id"] + n, _shapes(spec, n))
    ref = orc.backward(spec, x, *ups, n_params=lay["n_params"])
    _grad_close(_backward(spec, x, ups, lay["n_params"], ws=True), ref, lay, BWD_TOL)


def test_hermite4_active_levels(orc):
    W = I.WORKLOADS[NAME]
    spec = dict(W["spec"], active_levels=5)
    params = I.tables(W["id"], orc.layout(spec)["n_params"], W["tables"])
    x = _points(1500, 7)
    got = _forward(spec, x, params)
    for k in got:
        assert not np.any(got[k][..., 5 * spec["F"]:])
    _check(orc, spec, x, params, 8)


def test_hermite4_unsupported_paths():
    from multiresolution_hash_grid_multires_amd._lib import HASHENC_EUNSUPPORTED, HashencError
    spec = I.WORKLOADS[NAME]["spec"]
    h = api.hashenc_create(spec)
    assert api.hashenc_forward_workspace_size(h, 1000) > 0  # the packed copy of the tables
    assert api.hashenc_backward_workspace_size(h, 1000) > 0  # binned
    # F = 8: rows of 48 floats in the order-2 table, wider than the binned reduce takes; no
    # packed copy either
    wide = api.hashenc_create(dict(spec, F=8))
    assert api.hashenc_backward_workspace_size(wide, 1000) == 0
    assert api.hashenc_forward_workspace_size(wide, 1000) == 0
    with pytest.raises(HashencError) as e:
        api.hashenc_residual_workspace_size(h, api.Mlp(16, 32, 2, 30.0), 100)
    assert e.value.code == HASHENC_EUNSUPPORTED
