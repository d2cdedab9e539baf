"""The allocation-free backward (hashenc_backward_noalloc, static device scratch) against the
workspace backward it varies (hashenc_backward_ws), through the C ABI: two calls in a row on
one GPU, the second with a smaller input, each compared block by block at the gradient bar
(1e-4 normwise per table and level).  The first call at the benchmark's full size runs several
chunks of the scratch; the second reuses the scratch the first left behind."""
import ctypes

import numpy as np
import pytest
import torch

from multiresolution_hash_grid_multires_amd import _lib, api
from multiresolution_hash_grid_multires_amd import inputs as I

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
BWD_TOL = 1e-4


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV, torch.float32)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _blocks_close(a, b, h, spec):
    nt = spec["d"] + 1 if spec["kind"] == "hermite" else 1
    for k in range(nt):
        for l in range(spec["L"]):
            lay = api.hashenc_param_layout(h, k, l)
            o, m = lay["offset"], lay["rows"] * lay["width"]
            ref = b[o:o + m]
            err = float(np.max(np.abs(a[o:o + m] - ref)))
            scale = float(np.max(np.abs(ref)))
            assert err <= BWD_TOL * max(scale, 1e-30), f"table {k} level {l}: {err:.3e} vs {scale:.3e}"


def _ups(spec, W, n, seed):
    LF, d = spec["L"] * spec["F"], spec["d"]
    if spec["kind"] == "dlinear":
        shapes = [(n, LF)]
    else:
        shapes = [(n, LF), (n, d, LF), (n, d, LF) if spec.get("d2_mode") == "diag" else (n, LF)]
    return I.upstream(W["id"] + seed, shapes)


def _check(name, sizes):
    W = I.WORKLOADS[name]
    spec = W["spec"]
    enc = api.HashGridEncoding(spec)
    lib = _lib.load()
    for call, n in enumerate(sizes):
        x = _dev(I.points(W["id"] + 17 * call, n, spec["d"]))
        ups = [_dev(u) for u in _ups(spec, W, n, 31 * call)] + [None] * 2
        U = ups[:3]
        got = torch.zeros(enc.n_params, device=DEV)
        want = torch.zeros(enc.n_params, device=DEV)
        stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        print(f"noalloc {name} call {call} n={n}", flush=True)
        _lib.check(lib.hashenc_backward_noalloc(enc.handle, n, _ptr(x), _ptr(U[0]), _ptr(U[1]), _ptr(U[2]),
                                                _ptr(got), stream))
        enc.backward_ws(x, want, *U)
        torch.cuda.synchronize()
        _blocks_close(got.cpu().numpy().astype(np.float64), want.cpu().numpy().astype(np.float64), enc.handle, spec)


def test_noalloc_dlinear_full_size_then_smaller():
    _check("dlinear3d_L16_T19", [I.WORKLOADS["dlinear3d_L16_T19"]["n_points"], 5003])


def test_noalloc_hermite_then_smaller():
    _check("hermite3d_L16_T19", [100_003, 3001])


def test_noalloc_hermite2d_and_atomic_fallback():
    _check("hermite2d_L8_T14", [I.WORKLOADS["hermite2d_L8_T14"]["n_points"], 777])
    _check("rbf3d_L4_N56", [4096, 1000])  # no binned plan: the atomic scatter-add, no scratch


def test_noalloc_hermite4d_chunked_then_smaller():
    # about 19 KB of records per 4D point: 50k points take several chunks of the scratch
    _check("hermite4d_L8_T16", [50_001, 999])
