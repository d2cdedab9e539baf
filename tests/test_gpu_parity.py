"""GPU parity: the HIP library against the CPU oracle on the same seeded inputs.

Bars: lookup rows bit-exact; forward gamma / grad gamma / second derivatives within 1e-5
and gradients within 1e-4, both normwise per level and component (max|a-b| <= tol *
max|b| over that block), the oracle being fp64 after the fp32 position stage.
"""
import functools

import numpy as np
import pytest
import torch

from multiresolution_hash_grid_multires_amd import api
from multiresolution_hash_grid_multires_amd import inputs as I

pytestmark = pytest.mark.gpu

FWD_TOL = 1e-5
BWD_TOL = 1e-4
DEV = "cuda:0"


def _dev(a, dtype=torch.float32):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV, dtype)


def _upstream_shapes(spec, n):
    LF, d = spec["L"] * spec["F"], spec["d"]
    if spec["kind"] != "hermite":
        return [(n, LF)]
    return [(n, LF), (n, d, LF), (n, d, LF) if spec.get("d2_mode") == "diag" else (n, LF)]


@functools.lru_cache(maxsize=2)
def _tables(name, n_params):
    W = I.WORKLOADS[name]
    return I.tables(W["id"], n_params, W["tables"])


def _edge_points(d):
    """Points on faces, vertices and corners of the unit cube, plus out-of-range values."""
    vals = np.array([0.0, 1.0, 0.5, 0.25, 1.0 - 2 ** -24, 2 ** -24, 1 / 3, 0.999], np.float32)
    rng = np.random.default_rng(99)
    pts = rng.choice(vals, size=(64, d)).astype(np.float32)
    extra = np.array([[-0.25] * d, [1.5] * d, [np.nan] * d, [np.inf] * d, [-np.inf] * d], np.float32)
    return np.concatenate([pts, extra])


def _points(name, n, with_edges=True):
    W = I.WORKLOADS[name]
    d = W["spec"]["d"]
    x = I.points(W["id"], n, d, W.get("clustered_half", False))
    if with_edges:
        e = _edge_points(d)
        x[: e.shape[0]] = e
    return x


def _blocks_close(a, b, spec, tol, what):
    """Normwise per level and component: a, b [..., L*F] arrays."""
    L, F = spec["L"], spec["F"]
    a = a.reshape(a.shape[0], -1, L, F)
    b = b.reshape(b.shape[0], -1, L, F)
    for comp in range(a.shape[1]):
        for l in range(L):
            ref = b[:, comp, l]
            err = np.max(np.abs(a[:, comp, l] - ref))
            scale = np.max(np.abs(ref))
            assert err <= tol * max(scale, 1e-30), f"{what} comp {comp} level {l}: {err:.3e} vs {scale:.3e}"


def _grad_close(a, b, lay, tol):
    nt, L = lay["offset"].shape
    for k in range(nt):
        for l in range(L):
            o = lay["offset"][k, l]
            m = lay["rows"][k, l] * lay["width"][k, l]
            ref = b[o:o + m]
            err = np.max(np.abs(a[o:o + m] - ref))
            scale = np.max(np.abs(ref))
            assert err <= tol * max(scale, 1e-30), f"grad table {k} level {l}: {err:.3e} vs {scale:.3e}"


def _gpu_forward(spec, x, params):
    enc = api.HashGridEncoding(spec)
    xt, pt = _dev(x), _dev(params)
    out = enc.forward(xt, pt)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in out.items()}


def _gpu_backward(spec, x, ups, n_params, path="binned"):
    enc = api.HashGridEncoding(spec)
    grad = torch.zeros(n_params, device=DEV)
    U = [_dev(u) for u in ups] + [None] * (3 - len(ups))
    if path == "binned":
        enc.backward_binned(_dev(x), grad, *U)
    else:
        enc.backward(_dev(x), grad, *U)
    torch.cuda.synchronize()
    return grad.cpu().numpy()


PATHS = ["atomic", "binned"]


CONFIGS = ["dlinear2d_L4_T12", "hermite2d_L8_T14", "dlinear3d_L16_T19", "hermite3d_L16_T19"]


# ------------------------------------------------------------------ lookup stage
@pytest.mark.parametrize("name", CONFIGS)
def test_indices_bit_exact(orc, name):
    spec = I.WORKLOADS[name]["spec"]
    x = _points(name, 4099)
    h = api.hashenc_create(spec)
    n_tab = spec["d"] + 1 if spec["kind"] == "hermite" else 1
    for k in range(n_tab):
        out = torch.empty((x.shape[0], spec["L"], 1 << spec["d"]), dtype=torch.int32, device=DEV)
        api.hashenc_debug_indices(h, _dev(x), k, out)
        got = out.cpu().numpy()
        ref = orc.indices(spec, x, k)
        assert np.array_equal(got, ref), f"table {k}: {np.sum(got != ref)} rows differ"


def test_indices_general_modulo(orc):
    # table sizes that are not powers of two take the general "mod T" path
    spec = {"d": 3, "L": 4, "F": 2, "kind": "hermite", "T": [1000, 3001, 777, 5], "n_min": 8,
            "n_max": 64, "d2_mode": "diag"}
    x = np.random.default_rng(5).random((2000, 3), dtype=np.float32)
    h = api.hashenc_create(spec)
    for k in range(4):
        out = torch.empty((2000, 4, 8), dtype=torch.int32, device=DEV)
        api.hashenc_debug_indices(h, _dev(x), k, out)
        assert np.array_equal(out.cpu().numpy(), orc.indices(spec, x, k))


# ------------------------------------------------------------------ small-n parity
@pytest.mark.parametrize("name", CONFIGS)
def test_forward_parity(orc, name):
    spec = I.WORKLOADS[name]["spec"]
    lay = orc.layout(spec)
    params = _tables(name, lay["n_params"])
    x = _points(name, 3 * 1024 + 37)  # several 256-point blocks and a ragged tail
    got = _gpu_forward(spec, x, params)
    g, dg, d2 = orc.forward(spec, x, params)
    _blocks_close(got["gamma"], g, spec, FWD_TOL, "gamma")
    if spec["kind"] == "hermite":
        _blocks_close(got["dgamma"], dg, spec, FWD_TOL, "dgamma")
        _blocks_close(got["d2gamma"], d2, spec, FWD_TOL, "d2gamma")


@pytest.mark.parametrize("name", ["dlinear2d_L4_T12", "dlinear3d_L16_T19", "hermite2d_L8_T14", "hermite3d_L16_T19"])
def test_forward_ws_matches_forward(orc, name):
    spec = I.WORKLOADS[name]["spec"]
    lay = orc.layout(spec)
    params = _dev(_tables(name, lay["n_params"]))
    xh = _points(name, 5000 + 3)
    x = _dev(xh)
    enc = api.HashGridEncoding(spec)
    a = enc.forward(x, params)
    ws = enc.workspace(5003)
    for _ in range(2):  # workspace reused
        b = enc.forward_ws(x, params, workspace=ws)
        c = enc.forward_packed(x, params, workspace=ws)  # Hermite: packed tables at this size too
    torch.cuda.synchronize()
    # same arithmetic per level on every path: identical values, within the bar vs the oracle
    ref = orc.forward(spec, xh, _tables(name, lay["n_params"]))
    for k, r in zip(("gamma", "dgamma", "d2gamma"), ref):
        if k in a:
            assert torch.equal(a[k], b[k]), k
            assert torch.equal(a[k], c[k]), k
            _blocks_close(b[k].cpu().numpy(), r, spec, FWD_TOL, k)


@pytest.mark.parametrize("n", [(1 << 15) - 1, 1 << 15])
def test_forward_ws_pack_threshold(orc, n):
    # 2D and 3D Hermite workspace forwards pack the tables from 32768 points on and run the
    # direct forward below: the same bits on both sides of the switch, against the oracle
    name = "hermite2d_L8_T14"
    spec = I.WORKLOADS[name]["spec"]
    lay = orc.layout(spec)
    tab = _tables(name, lay["n_params"])
    xh = _points(name, n)
    x, params = _dev(xh), _dev(tab)
    enc = api.HashGridEncoding(spec)
    a = enc.forward(x, params)
    b = enc.forward_ws(x, params)
    c = enc.forward_packed(x, params)
    torch.cuda.synchronize()
    ref = orc.forward(spec, xh, tab)
    for k, r in zip(("gamma", "dgamma", "d2gamma"), ref):
        assert torch.equal(a[k], b[k]), k
        assert torch.equal(a[k], c[k]), k
        _blocks_close(b[k].cpu().numpy(), r, spec, FWD_TOL, k)


@pytest.mark.parametrize("L,F", [(5, 1), (3, 2), (32, 8), (7, 4)])
def test_forward_ws_row_widths(orc, L, F):
    # output rows of L*F floats that are not a multiple of 4 (scalar stores) and the widest
    # rows (smaller transpose tiles), against the oracle
    spec = {"d": 3, "L": L, "F": F, "kind": "dlinear", "T": [1 << 14], "n_min": 4, "n_max": 300}
    lay = orc.layout(spec)
    rng = np.random.default_rng(L * 10 + F)
    params = rng.standard_normal(lay["n_params"]).astype(np.float32)
    x = rng.random((3000 + 17, 3), dtype=np.float32)
    enc = api.HashGridEncoding(spec)
    out = enc.forward_ws(_dev(x), _dev(params), workspace=enc.workspace(x.shape[0]))
    torch.cuda.synchronize()
    g, _, _ = orc.forward(spec, x, params)
    _blocks_close(out["gamma"].cpu().numpy(), g, spec, FWD_TOL, "gamma")


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("name", CONFIGS)
def test_backward_parity(orc, name, path):
    W = I.WORKLOADS[name]
    spec = W["spec"]
    lay = orc.layout(spec)
    n = 3 * 1024 + 37
    x = _points(name, n)
    ups = I.upstream(W["id"], _upstream_shapes(spec, n))
    got = _gpu_backward(spec, x, ups, lay["n_params"], path)
    ref = orc.backward(spec, x, *ups, n_params=lay["n_params"])
    _grad_close(got, ref, lay, BWD_TOL)


@pytest.mark.parametrize("F", [1, 4, 8])
@pytest.mark.parametrize("kind", ["dlinear", "hermite"])
def test_feature_widths(orc, kind, F):  # both backward paths
    spec = {"d": 3, "L": 5, "F": F, "kind": kind, "T": [1 << 12] * 4, "n_min": 6, "n_max": 90,
            "d2_mode": "laplacian"}
    if kind == "dlinear":
        spec["T"] = [1 << 12]
    lay = orc.layout(spec)
    rng = np.random.default_rng(F)
    params = rng.standard_normal(lay["n_params"]).astype(np.float32)
    x = rng.random((777, 3), dtype=np.float32)
    got = _gpu_forward(spec, x, params)
    g, dg, d2 = orc.forward(spec, x, params)
    _blocks_close(got["gamma"], g, spec, FWD_TOL, "gamma")
    if kind == "hermite":
        _blocks_close(got["dgamma"], dg, spec, FWD_TOL, "dgamma")
        _blocks_close(got["d2gamma"], d2, spec, FWD_TOL, "d2gamma")
    # the workspace forward (packed order tables for Hermite) gives the same bits
    enc = api.HashGridEncoding(spec)
    ws_out = enc.forward_ws(_dev(x), _dev(params), workspace=enc.workspace(x.shape[0]))
    pk_out = enc.forward_packed(_dev(x), _dev(params), workspace=enc.workspace(x.shape[0]))
    torch.cuda.synchronize()
    for k in got:
        assert np.array_equal(ws_out[k].cpu().numpy(), got[k]), k
        assert np.array_equal(pk_out[k].cpu().numpy(), got[k]), k
    ups = [u.astype(np.float32) for u in
           (rng.standard_normal(s) for s in _upstream_shapes(spec, 777))]
    ref = orc.backward(spec, x, *ups, n_params=lay["n_params"])
    for path in PATHS:
        _grad_close(_gpu_backward(spec, x, ups, lay["n_params"], path), ref, lay, BWD_TOL)


@pytest.mark.parametrize("T", [[1000, 3001, 777, 5], [1 << 12, 1 << 13, 1 << 11, 1 << 12],
                               [1 << 12, 1 << 12, 1 << 10, 1 << 8], [1 << 14, 1 << 14, 1 << 10]])
def test_hermite_unequal_tables(orc, T):
    # order tables of different sizes (dense on different levels, modulo and mask hashing):
    # the count pass histograms every table separately.  Power-of-two tables no larger than
    # the order-0 one are packed (their rows repeated across the order-0 rows that share
    # them), including levels dense in the order-0 table and hashed in a smaller one; the
    # last case is the 2D 14-14-10 sizing
    d = len(T) - 1
    spec = {"d": d, "L": 4, "F": 2, "kind": "hermite", "T": T, "n_min": 8, "n_max": 64 if d == 3 else 512,
            "d2_mode": "diag"}
    lay = orc.layout(spec)
    rng = np.random.default_rng(sum(T))
    params = rng.standard_normal(lay["n_params"]).astype(np.float32)
    n = 3000
    x = rng.random((n, d), dtype=np.float32)
    got = _gpu_forward(spec, x, params)
    for name, r in zip(("gamma", "dgamma", "d2gamma"), orc.forward(spec, x, params)):
        _blocks_close(got[name], r, spec, FWD_TOL, name)
    enc = api.HashGridEncoding(spec)
    pow2 = lambda t: t > 1 and t & (t - 1) == 0
    packable = all(t == T[0] or (pow2(t) and pow2(T[0]) and t < T[0]) for t in T)
    stage = 4 * n * spec["L"] * (1 + 2 * d) * spec["F"]  # level-major staging [L][n][1 + 2d][F]
    packed = 4 * int(sum(lay["rows"][0])) * (1 << d) * spec["F"] if packable else 0
    assert api.hashenc_forward_workspace_size(enc.handle, n) == (packed + 255) // 256 * 256 + stage
    ws_out = enc.forward_ws(_dev(x), _dev(params))
    pk_out = enc.forward_packed(_dev(x), _dev(params))  # packed copy at this size as well
    torch.cuda.synchronize()
    for k in got:
        assert np.array_equal(ws_out[k].cpu().numpy(), got[k]), k
        assert np.array_equal(pk_out[k].cpu().numpy(), got[k]), k
    ups = [u.astype(np.float32) for u in (rng.standard_normal(s) for s in _upstream_shapes(spec, n))]
    ref = orc.backward(spec, x, *ups, n_params=lay["n_params"])
    for path in PATHS:
        _grad_close(_gpu_backward(spec, x, ups, lay["n_params"], path), ref, lay, BWD_TOL)


# The binned d-linear backward writes one record per x-corner pair where both corners fall
# in one reduction chunk, and one record per corner elsewhere.  With F = 8 a chunk holds
# 1024 rows, so these grids take every branch:
PAIR_MODE_SPECS = {
    # dense levels N = 300, 501, 837 (chunks of whole x-lines, not powers of two) and 1400
    # (x-lines longer than a chunk: single records)
    "dense2d": {"d": 2, "L": 4, "F": 8, "kind": "dlinear", "T": [1 << 21], "n_min": 300, "n_max": 1400},
    # dense N = 16, 36; hashed N = 83, 191, 437 (2N within a chunk) and 1000 (single records)
    "hashed3d": {"d": 3, "L": 6, "F": 8, "kind": "dlinear", "T": [1 << 16], "n_min": 16, "n_max": 1000},
    # T not a power of two: hashed rows taken modulo T, single records
    "modulo3d": {"d": 3, "L": 4, "F": 2, "kind": "dlinear", "T": [50000], "n_min": 16, "n_max": 300},
}


@pytest.mark.parametrize("case", sorted(PAIR_MODE_SPECS))
def test_dlinear_record_modes(orc, case):
    spec = PAIR_MODE_SPECS[case]
    lay = orc.layout(spec)
    n = 5000
    rng = np.random.default_rng(len(case))
    x = rng.random((n, spec["d"]), dtype=np.float32)
    e = _edge_points(spec["d"])
    x[: e.shape[0]] = e
    (G,) = [u.astype(np.float32) for u in (rng.standard_normal(s) for s in _upstream_shapes(spec, n))]
    ref = orc.backward(spec, x, G, n_params=lay["n_params"])
    for path in PATHS:
        _grad_close(_gpu_backward(spec, x, [G], lay["n_params"], path), ref, lay, BWD_TOL)


def test_laplacian_is_trace_of_diagonal():
    base = {"d": 3, "L": 6, "F": 2, "kind": "hermite", "T": [1 << 14] * 4, "n_min": 8, "n_max": 200}
    x = np.random.default_rng(3).random((1000, 3), dtype=np.float32)
    enc_d = api.HashGridEncoding(dict(base, d2_mode="diag"))
    enc_l = api.HashGridEncoding(dict(base, d2_mode="laplacian"))
    params = _dev(np.random.default_rng(4).normal(0, 0.01, enc_d.n_params).astype(np.float32))
    od = enc_d.forward(_dev(x), params)
    ol = enc_l.forward(_dev(x), params)
    torch.testing.assert_close(od["gamma"], ol["gamma"], rtol=0, atol=0)
    s = od["d2gamma"].sum(1)
    assert float((s - ol["d2gamma"]).abs().max()) <= 1e-5 * float(s.abs().max())


def test_optional_outputs_and_upstreams(orc):
    spec = I.WORKLOADS["hermite2d_L8_T14"]["spec"]
    lay = orc.layout(spec)
    params = _tables("hermite2d_L8_T14", lay["n_params"])
    x = _points("hermite2d_L8_T14", 600)
    h = api.hashenc_create(spec)
    dg = torch.full((600, 2, 16), 7.0, device=DEV)
    api.hashenc_forward(h, _dev(x), _dev(params), None, dg, None)
    _, dref, _ = orc.forward(spec, x, params)
    _blocks_close(dg.cpu().numpy(), dref, spec, FWD_TOL, "dgamma only")
    # only the Laplacian upstream
    G = np.random.default_rng(8).standard_normal((600, 16)).astype(np.float32)
    grad = torch.zeros(lay["n_params"], device=DEV)
    api.hashenc_backward(h, _dev(x), None, None, _dev(G), grad)
    _grad_close(grad.cpu().numpy(), orc.backward(spec, x, None, None, G, n_params=lay["n_params"]), lay, BWD_TOL)


def test_tiny_and_empty_batches(orc):
    spec = I.WORKLOADS["dlinear3d_L16_T19"]["spec"]
    lay = orc.layout(spec)
    params = _tables("dlinear3d_L16_T19", lay["n_params"])
    enc = api.HashGridEncoding(spec)
    pt = _dev(params)
    for n in (1, 63, 65, 257):
        x = _points("dlinear3d_L16_T19", n, with_edges=False)
        got = enc.forward(_dev(x), pt)["gamma"].cpu().numpy()
        _blocks_close(got, orc.forward(spec, x, params)[0], spec, FWD_TOL, f"n={n}")
    empty = torch.empty((0, 3), device=DEV)
    out = torch.empty((0, 32), device=DEV)
    api.hashenc_forward(enc.handle, empty, pt, out)
    grad = torch.zeros(lay["n_params"], device=DEV)
    api.hashenc_backward(enc.handle, empty, out, None, None, grad)
    torch.cuda.synchronize()
    assert float(grad.abs().max()) == 0.0


# ------------------------------------------------------------------ full-size checks
@pytest.mark.parametrize("name", ["dlinear3d_L16_T19", "hermite3d_L16_T19", "hermite2d_L8_T14"])
def test_full_size_forward_sampled(orc, name):
    W = I.WORKLOADS[name]
    spec = W["spec"]
    lay = orc.layout(spec)
    params = _tables(name, lay["n_params"])
    x = I.points(W["id"], W["n_points"], spec["d"])
    got = _gpu_forward(spec, x, params)
    idx = np.sort(np.random.default_rng(1).choice(x.shape[0], 4096, replace=False))
    idx[-1] = x.shape[0] - 1
    g, dg, d2 = orc.forward(spec, x[idx], params)
    _blocks_close(got["gamma"][idx], g, spec, FWD_TOL, "gamma")
    if spec["kind"] == "hermite":
        _blocks_close(got["dgamma"][idx], dg, spec, FWD_TOL, "dgamma")
        _blocks_close(got["d2gamma"][idx], d2, spec, FWD_TOL, "d2gamma")


@pytest.mark.parametrize("name", ["dlinear3d_L16_T19", "hermite3d_L16_T19", "hermite2d_L8_T14",
                                  "hermite2d_L8_T14_14_10", "hermite4d_L8_T16"])
def test_full_size_forward_ws_sampled(orc, name):
    """The workspace forward in the launch configuration the benchmark times: every level
    active, all of the workload's points, the workspace shared with the backward (d-linear:
    LDS levels, L2 passes and the level-major transpose; Hermite: packed tables, level-major
    staging and the rearrangement into rows; 4D Hermite: the packed copy of the five tables).
    4096 sampled points and the last one against the oracle, per level and component."""
    W = I.WORKLOADS[name]
    spec = W["spec"]
    lay = orc.layout(spec)
    params = _tables(name, lay["n_params"])
    n = W["n_points"]
    x = I.points(W["id"], n, spec["d"])
    enc = api.HashGridEncoding(spec)
    ws = enc.workspace(n)
    shapes = enc.output_shapes(n)
    outs = {k: torch.full(s, float("nan"), device=DEV) for k, s in shapes.items()}
    api.hashenc_forward_ws(enc.handle, _dev(x), _dev(params), outs["gamma"], outs.get("dgamma"),
                           outs.get("d2gamma"), ws)
    torch.cuda.synchronize()
    got = {k: v.cpu().numpy() for k, v in outs.items()}
    for k, v in got.items():
        assert np.isfinite(v).all(), f"{k}: unwritten entries"
    idx = np.sort(np.random.default_rng(11).choice(n, 4096, replace=False))
    idx[-1] = n - 1
    g, dg, d2 = orc.forward(spec, x[idx], params)
    _blocks_close(got["gamma"][idx], g, spec, FWD_TOL, "gamma")
    if spec["kind"] == "hermite":
        _blocks_close(got["dgamma"][idx], dg, spec, FWD_TOL, "dgamma")
        _blocks_close(got["d2gamma"][idx], d2, spec, FWD_TOL, "d2gamma")


@pytest.mark.parametrize("name", ["dlinear3d_L16_T19", "hermite3d_L16_T19"])
def test_full_size_backward(orc, name):
    W = I.WORKLOADS[name]
    spec = W["spec"]
    lay = orc.layout(spec)
    n = W["n_points"]
    x = I.points(W["id"], n, spec["d"])
    ups = I.upstream(W["id"], _upstream_shapes(spec, n))
    ref = orc.backward(spec, x, *ups, n_params=lay["n_params"])
    for path in PATHS:
        _grad_close(_gpu_backward(spec, x, ups, lay["n_params"], path), ref, lay, BWD_TOL)


@pytest.mark.parametrize("n", [256 * 512, 256 * 512 + 1])
def test_binned_scan_tile_limit(orc, n):
    # 2D Hermite scatter tiles hold 512 points at F = 2: 256 tiles is the largest count matrix
    # scanned in one pass (16 tiles per wavefront), 257 tiles the smallest scanned in two
    W = I.WORKLOADS["hermite2d_L8_T14"]
    spec = W["spec"]
    lay = orc.layout(spec)
    x = _points("hermite2d_L8_T14", n)
    ups = I.upstream(W["id"], _upstream_shapes(spec, n))
    ref = orc.backward(spec, x, *ups, n_params=lay["n_params"])
    _grad_close(_gpu_backward(spec, x, ups, lay["n_params"], "binned"), ref, lay, BWD_TOL)


def test_binned_backward_chunks_and_clusters(orc):
    # more points than one 2^21 chunk, half of them clustered (hot bins split across work
    # items), a workspace reused across calls and accumulation into a non-zero gradient
    W = I.WORKLOADS["dlinear3d_L16_T19"]
    spec = dict(W["spec"], L=6, n_max=600)
    lay = orc.layout(spec)
    n = (1 << 21) + 777
    x = I.points(5, n, 3, clustered_half=True)
    (G,) = I.upstream(3, [(n, 12)])
    enc = api.HashGridEncoding(spec)
    ws = enc.workspace(n)
    grad = torch.full((lay["n_params"],), 0.5, device=DEV)
    for _ in range(2):
        enc.backward_ws(_dev(x), grad, _dev(G), workspace=ws)
    torch.cuda.synchronize()
    ref = orc.backward(spec, x, G, n_params=lay["n_params"])
    _grad_close(grad.cpu().numpy() - 0.5, 2 * ref, lay, BWD_TOL)


@pytest.mark.parametrize("name", CONFIGS)
def test_adjoint_identity_on_gpu(name):
    # <backward(G), dtheta> = <G, forward(dtheta)>, both sides from the HIP path, in fp64 sums
    W = I.WORKLOADS[name]
    spec = W["spec"]
    enc = api.HashGridEncoding(spec)
    n = W["n_points"]
    x = _dev(I.points(W["id"], n, spec["d"]))
    dtheta = _dev(I.delta(W["id"], enc.n_params))
    ups = [_dev(u) for u in I.upstream(W["id"], _upstream_shapes(spec, n))]
    out = enc.forward(x, dtheta)
    grad = torch.zeros(enc.n_params, device=DEV)
    enc.backward(x, grad, *(ups + [None] * (3 - len(ups))))
    keys = ["gamma", "dgamma", "d2gamma"][: len(ups)]
    rhs = sum(float((out[k].double() * u.double()).sum()) for k, u in zip(keys, ups))
    lhs = float((grad.double() * dtheta.double()).sum())
    scale = float((grad.double().abs() * dtheta.double().abs()).sum())
    assert abs(lhs - rhs) <= 1e-5 * scale


@pytest.mark.parametrize("name,n", [("dlinear3d_L16_T19", 3 * 8192 + 37), ("dlinear2d_L4_T12", 65536 + 5)])
def test_counting_pair(orc, name, n):
    """The counting forward (bin counts taken while gathering) and the counted backward: gamma
    bit-identical to forward_ws, gradient against the oracle and against backward_ws.  The
    2D grid keeps all four levels in LDS, so its counts all come from the count kernel."""
    W = I.WORKLOADS[name]
    spec = W["spec"]
    lay = orc.layout(spec)
    enc = api.HashGridEncoding(spec)
    x = _points(name, n)
    params = _tables(name, lay["n_params"])
    (G,) = I.upstream(W["id"], _upstream_shapes(spec, n))
    xt, pt, Gt = _dev(x), _dev(params), _dev(G)
    fws, bws = enc.forward_workspace(n), enc.backward_workspace(n)
    assert bws is not None
    bws.fill_(0x7b)   # stale contents must not matter
    out = enc.forward_counting(xt, pt, fws, bws)
    ref_out = enc.forward_ws(xt, pt, enc.workspace(n))
    assert torch.equal(out["gamma"], ref_out["gamma"])
    got = enc.backward_counted(xt, torch.zeros(enc.n_params, device=DEV), Gt, bwd_workspace=bws)
    want = enc.backward_ws(xt, torch.zeros(enc.n_params, device=DEV), Gt, workspace=enc.workspace(n))
    torch.cuda.synchronize()
    got, want = got.cpu().numpy(), want.cpu().numpy()
    _grad_close(got, orc.backward(spec, x, G, n_params=lay["n_params"]), lay, BWD_TOL)
    _grad_close(got, want.astype(np.float64), lay, 1e-5)
    # a second pair on the same workspaces (counters re-zeroed by the forward)
    enc.forward_counting(xt, pt, fws, bws)
    again = enc.backward_counted(xt, torch.zeros(enc.n_params, device=DEV), Gt, bwd_workspace=bws)
    torch.cuda.synchronize()
    _grad_close(again.cpu().numpy(), got.astype(np.float64), lay, 1e-5)


def test_counting_pair_full_size_and_fallbacks():
    """The headline batch through the counting pair matches forward_ws / backward_ws; where the
    counts do not apply (a small d-linear batch, the Hermite kind) the pair is forward_ws and
    backward_ws."""
    for name, n in (("dlinear3d_L16_T19", None), ("dlinear3d_L16_T19", 1000), ("hermite3d_L16_T19", 40000)):
        W = I.WORKLOADS[name]
        spec = W["spec"]
        n = n or W["n_points"]
        enc = api.HashGridEncoding(spec)
        x = _dev(I.points(W["id"], n, spec["d"]))
        p = _dev(_tables(name, enc.n_params))
        ups = [_dev(u) for u in I.upstream(W["id"], _upstream_shapes(spec, n))]
        ups += [None] * (3 - len(ups))
        fws = enc.forward_workspace(n)
        bws = enc.backward_workspace(n)
        out = enc.forward_counting(x, p, fws, bws)
        ref = enc.forward_ws(x, p, enc.workspace(n))
        for k in ref:
            assert torch.equal(out[k], ref[k]), (name, n, k)
        a = enc.backward_counted(x, torch.zeros(enc.n_params, device=DEV), *ups, bwd_workspace=bws)
        b = enc.backward_ws(x, torch.zeros(enc.n_params, device=DEV), *ups, workspace=enc.workspace(n))
        torch.cuda.synchronize()
        assert float((a - b).abs().max()) <= 1e-5 * float(b.abs().max()), (name, n)


@pytest.mark.parametrize("name", ["dlinear3d_L16_T19", "hermite3d_L16_T19"])
def test_binned_nonfinite_upstream(orc, name):
    """A NaN and an inf upstream value: the levels they reach take the binned reduce's fp64
    path, the others its fixed-point path.  Non-finite gradient entries sit where the atomic
    path (plain fp32 adds) puts them; every other entry matches the oracle."""
    W = I.WORKLOADS[name]
    spec = W["spec"]
    lay = orc.layout(spec)
    n = 3 * 1024 + 37
    x = _points(name, n, with_edges=False)
    ups = I.upstream(W["id"], _upstream_shapes(spec, n))
    F = spec["F"]
    ups[0][5, 0] = np.nan                # level 0, feature 0 of point 5
    ups[0][9, 3 * F + 1] = np.inf        # level 3, feature 1 of point 9
    got = _gpu_backward(spec, x, ups, lay["n_params"], "binned")
    atom = _gpu_backward(spec, x, ups, lay["n_params"], "atomic")
    bad = ~np.isfinite(got)
    assert bad.any()
    assert np.array_equal(bad, ~np.isfinite(atom))
    clean = [u.copy() for u in ups]
    clean[0][5, 0] = 0.0
    clean[0][9, 3 * F + 1] = 0.0
    ref = orc.backward(spec, x, *clean, n_params=lay["n_params"])
    nt, L = lay["offset"].shape
    for k in range(nt):
        for l in range(L):
            o, m = lay["offset"][k, l], lay["rows"][k, l] * lay["width"][k, l]
            ok = np.isfinite(got[o:o + m])
            err = np.max(np.abs(got[o:o + m][ok] - ref[o:o + m][ok]), initial=0.0)
            assert err <= BWD_TOL * np.max(np.abs(ref[o:o + m])), f"table {k} level {l}: {err:.3e}"


def test_backward_run_to_run_spread():
    W = I.WORKLOADS["dlinear3d_L16_T19"]
    spec = W["spec"]
    enc = api.HashGridEncoding(spec)
    n = W["n_points"]
    x = _dev(I.points(W["id"], n, 3))
    (G,) = I.upstream(W["id"], _upstream_shapes(spec, n))
    G = _dev(G)
    a = torch.zeros(enc.n_params, device=DEV)
    b = torch.zeros(enc.n_params, device=DEV)
    c = torch.zeros(enc.n_params, device=DEV)
    enc.backward(x, a, G)
    enc.backward(x, b, G)
    enc.backward_ws(x, c, G)
    assert float((a - b).abs().max()) <= 1e-5 * float(a.abs().max())
    assert float((a - c).abs().max()) <= 1e-5 * float(a.abs().max())
    # accumulation: a second call adds
    enc.backward(x, a, G)
    assert float((a - 2 * b).abs().max()) <= 1e-5 * float(b.abs().max())
    # The binned reduce sums each bin's values as exact fixed-point integers, so a bin that one
    # work item covers gets the same bits whatever order its records arrive in.  Here the
    # hashed levels' bins hold about 2^20 * 4 / 64 = 65536 pair records, below the work-item
    # size (2^18 entries), so the finest eight levels are bit-identical from run to run.
    d = torch.zeros(enc.n_params, device=DEV)
    enc.backward_ws(x, d, G)
    off = api.hashenc_param_layout(enc.handle, 0, 8)["offset"]
    assert torch.equal(c[off:], d[off:])
