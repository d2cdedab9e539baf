"""Host-side checks of the C ABI (no GPU needed): the library loads and exports every
declared entry point; configuration validation, level progression and parameter layout
agree with the oracle's; every argument error is reported before any launch."""
import ctypes
import os
import re

import numpy as np
import pytest

from multiresolution_hash_grid_multires_amd import _lib, api
from multiresolution_hash_grid_multires_amd.inputs import WORKLOADS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_symbols():
    names = set()
    for h in ("hashenc.h", "hashenc_diag.h"):
        text = open(os.path.join(ROOT, "include", h)).read()
        names |= set(re.findall(r"HASHENC_API\s+[\w\s\*]+?\b(hashenc_\w+)\s*\(", text))
    return names


def test_library_exports_every_declared_symbol():
    lib = _lib.load()
    names = _declared_symbols()
    assert {"hashenc_create", "hashenc_forward", "hashenc_backward", "hashenc_residual"} <= names
    for n in names:
        assert hasattr(lib, n), n
    assert {s[0] for s in _lib.SIGNATURES} == names


@pytest.mark.parametrize("name", list(WORKLOADS))
def test_layout_matches_oracle(orc, name):
    spec = WORKLOADS[name]["spec"]
    h = api.hashenc_create(spec)
    n_params, width, res = api.hashenc_info(h)
    lay = orc.layout(spec)
    assert n_params == lay["n_params"]
    assert width == spec["L"] * spec["F"]
    assert res == lay["N"]
    nt = lay["offset"].shape[0]
    for k in range(nt):
        for l in range(spec["L"]):
            pl = api.hashenc_param_layout(h, k, l)
            assert pl["offset"] == lay["offset"][k, l]
            assert pl["rows"] == lay["rows"][k, l]
            assert pl["width"] == lay["width"][k, l]
            assert pl["dense"] == bool(lay["dense"][k, l])


def test_explicit_resolutions_and_growth(orc):
    spec = {"d": 3, "L": 3, "F": 2, "kind": "hermite", "T": [1 << 10, 1 << 12, 1 << 8, 1 << 9],
            "resolutions": [5, 9, 30], "d2_mode": "diag"}
    h = api.hashenc_create(spec)
    assert api.hashenc_info(h)[2] == [5, 9, 30]
    assert api.hashenc_info(h)[0] == orc.layout(spec)["n_params"]
    h2 = api.hashenc_create({"d": 2, "L": 4, "F": 1, "kind": "dlinear", "T": [4096], "n_min": 16, "growth": 1.5})
    assert api.hashenc_info(h2)[2] == [16, 24, 36, 54]


def _create_code(**over):
    spec = {"d": 3, "L": 4, "F": 2, "kind": "dlinear", "T": [1 << 12], "n_min": 4, "n_max": 32}
    spec.update(over)
    return api._spec_to_config(spec)


@pytest.mark.parametrize("field,value", [
    ("d", 1), ("d", 4), ("n_levels", 0), ("n_levels", 33), ("n_features", 3), ("n_features", 16),
    ("kind", 7), ("reserved", 1), ("n_min", 0), ("n_max", 2),
])
def test_create_rejects_bad_config(field, value):
    cfg, keep = _create_code()
    setattr(cfg, field, value)
    out = ctypes.c_void_p()
    rc = _lib.load().hashenc_create(ctypes.byref(cfg), ctypes.byref(out))
    assert rc == _lib.HASHENC_EINVAL
    assert out.value is None
    assert _lib.load().hashenc_last_error()


def test_create_rejects_bad_hermite_mode_and_table():
    cfg, keep = _create_code(kind="hermite")
    cfg.d2_mode = 0
    out = ctypes.c_void_p()
    assert _lib.load().hashenc_create(ctypes.byref(cfg), ctypes.byref(out)) == _lib.HASHENC_EINVAL
    cfg.d2_mode = 2
    cfg.table_size[2] = 0
    assert _lib.load().hashenc_create(ctypes.byref(cfg), ctypes.byref(out)) == _lib.HASHENC_EINVAL
    assert b"table_size[2]" in _lib.load().hashenc_last_error()


def test_create_rejects_resolution_out_of_range():
    with pytest.raises(_lib.HashencError) as e:
        api.hashenc_create({"d": 2, "L": 2, "F": 2, "kind": "dlinear", "T": [64], "resolutions": [4, 0]})
    assert e.value.code == _lib.HASHENC_EINVAL
    with pytest.raises(_lib.HashencError):
        api.hashenc_create({"d": 2, "L": 2, "F": 2, "kind": "dlinear", "T": [64], "n_min": 4,
                            "growth": 1e7})


def test_null_arguments_and_destroy_null():
    lib = _lib.load()
    assert lib.hashenc_create(None, None) == _lib.HASHENC_EINVAL
    lib.hashenc_destroy(None)
    assert lib.hashenc_info(None, None, None, None) == _lib.HASHENC_EINVAL
    assert lib.hashenc_forward(None, 1, None, None, None, None, None, None) == _lib.HASHENC_EINVAL


def test_forward_backward_validation_before_launch():
    lib = _lib.load()
    h = api.hashenc_create({"d": 3, "L": 2, "F": 2, "kind": "dlinear", "T": [1 << 10], "n_min": 4, "n_max": 8})
    P = ctypes.c_void_p
    a, b, c = P(0x10000), P(0x20000), P(0x30000)   # aligned, never dereferenced
    mis = P(0x20004)
    # n == 0 and "no outputs" are successful no-ops
    assert lib.hashenc_forward(h, 0, None, None, None, None, None, None) == 0
    assert lib.hashenc_forward(h, 5, a, b, None, None, None, None) == 0
    assert lib.hashenc_backward(h, 5, a, None, None, None, c, None) == 0
    # errors
    assert lib.hashenc_forward(h, -1, a, b, c, None, None, None) == _lib.HASHENC_EINVAL
    assert lib.hashenc_forward(h, 5, None, b, c, None, None, None) == _lib.HASHENC_EINVAL
    assert lib.hashenc_forward(h, 5, a, None, c, None, None, None) == _lib.HASHENC_EINVAL
    assert lib.hashenc_forward(h, 5, a, mis, c, None, None, None) == _lib.HASHENC_EALIGN
    assert lib.hashenc_forward(h, 5, a, b, c, c, None, None) == _lib.HASHENC_EUNSUPPORTED
    assert lib.hashenc_backward(h, 5, a, b, None, None, None, None) == _lib.HASHENC_EINVAL
    assert lib.hashenc_backward(h, 5, a, b, None, None, mis, None) == _lib.HASHENC_EALIGN
    assert lib.hashenc_backward(h, 5, a, b, c, None, c, None) == _lib.HASHENC_EUNSUPPORTED
    assert lib.hashenc_backward(h, 1 << 62, a, b, None, None, c, None) == _lib.HASHENC_EINVAL
    assert lib.hashenc_debug_indices(h, 5, a, 1, c, None) == _lib.HASHENC_EINVAL
    assert lib.hashenc_debug_indices(h, 5, a, 0, mis, None) == _lib.HASHENC_EALIGN
    assert lib.hashenc_diag_copy(a, mis, 8, None) == _lib.HASHENC_EALIGN
    assert lib.hashenc_diag_copy(a, b, -1, None) == _lib.HASHENC_EINVAL
    assert lib.hashenc_diag_cache_read(a, 33, 1, b, None) == _lib.HASHENC_EINVAL
    assert lib.hashenc_diag_cache_read(a, 0, 1, b, None) == _lib.HASHENC_EINVAL
    assert lib.hashenc_diag_cache_read(a, 64, 0, b, None) == _lib.HASHENC_EINVAL
    assert lib.hashenc_diag_cache_read(a, 64, 1, None, None) == _lib.HASHENC_EINVAL
    assert lib.hashenc_diag_cache_read(mis, 64, 1, b, None) == _lib.HASHENC_EALIGN
    assert lib.hashenc_param_layout(h, 1, 0, None, None, None, None) == _lib.HASHENC_EINVAL
    assert lib.hashenc_param_layout(h, 0, 2, None, None, None, None) == _lib.HASHENC_EINVAL


def test_binding_rejects_host_tensors():
    import torch
    h = api.hashenc_create({"d": 2, "L": 1, "F": 2, "kind": "dlinear", "T": [64], "n_min": 4, "n_max": 4})
    with pytest.raises(ValueError):
        api.hashenc_forward(h, torch.zeros(4, 2), torch.zeros(50), torch.zeros(4, 2))


def test_residual_validation_on_host():
    lib = _lib.load()
    herm = api.hashenc_create({"d": 3, "L": 16, "F": 2, "kind": "hermite", "T": [1 << 19] * 4,
                               "n_min": 16, "n_max": 1024, "d2_mode": "laplacian"})
    lin = api.hashenc_create({"d": 3, "L": 2, "F": 2, "kind": "dlinear", "T": [1 << 10], "n_min": 4, "n_max": 8})
    assert api.hashenc_residual_workspace_size(herm, api.Mlp(32, 64, 2, 30.0), 1 << 21) > 0
    b = ctypes.c_size_t()
    for mlp, code in [(api.Mlp(32, 64, 2, 30.0), _lib.HASHENC_EUNSUPPORTED)]:
        m = mlp.as_c()
        assert lib.hashenc_residual_workspace_size(lin, ctypes.byref(m), 8, ctypes.byref(b)) == code
    for mlp, code in [(api.Mlp(16, 64, 2, 30.0), _lib.HASHENC_EINVAL),
                      (api.Mlp(32, 65, 2, 30.0), _lib.HASHENC_EUNSUPPORTED),
                      (api.Mlp(32, 64, 5, 30.0), _lib.HASHENC_EUNSUPPORTED),
                      (api.Mlp(32, 64, 0, 30.0), _lib.HASHENC_EUNSUPPORTED),
                      (api.Mlp(32, 64, 2, float("nan")), _lib.HASHENC_EINVAL)]:
        m = mlp.as_c()
        assert lib.hashenc_residual_workspace_size(herm, ctypes.byref(m), 8, ctypes.byref(b)) == code
    m = api.Mlp(32, 64, 2, 30.0).as_c()
    P = ctypes.c_void_p
    a = P(0x10000)
    need = api.hashenc_residual_workspace_size(herm, api.Mlp(32, 64, 2, 30.0), 8)
    # too small a workspace, n = 0, a misaligned workspace: all rejected before any launch
    assert lib.hashenc_residual(herm, ctypes.byref(m), 8, a, a, a, None, a, None, None, a, need - 1, None) == _lib.HASHENC_EINVAL
    assert lib.hashenc_residual(herm, ctypes.byref(m), 0, a, a, a, None, a, None, None, a, need, None) == _lib.HASHENC_EINVAL
    assert lib.hashenc_residual(herm, ctypes.byref(m), 8, a, a, a, None, a, None, None, P(0x10010), need, None) == _lib.HASHENC_EALIGN
    assert lib.hashenc_residual(herm, ctypes.byref(m), 8, a, a, a, None, None, None, None, a, need, None) == _lib.HASHENC_EINVAL


# ---------------------------------------------------------------- coarse-to-fine activation
def test_c2f_schedule_matches_oracle(orc):
    for L in (1, 8, 16):
        for L0 in (1, 3, 16):
            for tau in (1, 7, 500):
                for t in (0, 1, tau - 1, tau, 2 * tau + 1, 40 * tau, 10 ** 15):
                    assert api.hashenc_c2f_active_levels(L, L0, t, tau) == orc.c2f_active_levels(L, L0, t, tau)


@pytest.mark.parametrize("args", [(0, 1, 0, 1), (16, 0, 0, 1), (16, 1, -1, 1), (16, 1, 0, 0)])
def test_c2f_schedule_rejects_bad_arguments(args):
    out = ctypes.c_int32()
    assert _lib.load().hashenc_c2f_active_levels(*args, ctypes.byref(out)) == _lib.HASHENC_EINVAL
    assert _lib.load().hashenc_c2f_active_levels(16, 1, 0, 1, None) == _lib.HASHENC_EINVAL


def test_derive_active_keeps_layout_and_width(orc):
    spec = {"d": 3, "L": 6, "F": 2, "kind": "hermite", "T": [1 << 10] * 4, "n_min": 4, "n_max": 64,
            "d2_mode": "laplacian"}
    h = api.hashenc_create(spec)
    assert api.hashenc_active_levels(h) == 6
    for a in (1, 3, 6):
        ha = api.hashenc_derive_active(h, a)
        assert api.hashenc_active_levels(ha) == a
        assert api.hashenc_info(ha) == api.hashenc_info(h)
        for l in range(6):
            assert api.hashenc_param_layout(ha, 2, l) == api.hashenc_param_layout(h, 2, l)
        # counted against the configuration, also from a derived handle
        hb = api.hashenc_derive_active(ha, 5)
        assert api.hashenc_active_levels(hb) == 5
    enc = api.HashGridEncoding(dict(spec, active_levels=2))
    assert enc.active_levels == 2 and enc.out_width == 12
    enc.set_active_levels(6)
    assert enc.active_levels == 6


@pytest.mark.parametrize("n_active", [0, -1, 7])
def test_derive_active_rejects_bad_count(n_active):
    spec = {"d": 2, "L": 6, "F": 2, "kind": "dlinear", "T": [1 << 10], "n_min": 4, "n_max": 64}
    h = api.hashenc_create(spec)
    out = ctypes.c_void_p()
    assert _lib.load().hashenc_derive_active(h, n_active, ctypes.byref(out)) == _lib.HASHENC_EINVAL
    assert out.value is None
    assert _lib.load().hashenc_derive_active(None, 1, ctypes.byref(out)) == _lib.HASHENC_EINVAL
    assert _lib.load().hashenc_derive_active(h, 1, None) == _lib.HASHENC_EINVAL


# ---------------------------------------------------------------- binding size checks
def test_binding_rejects_mismatched_sizes_before_launch():
    """Every tensor's element count is checked against the layout before a pointer reaches
    the library (host tensors: the size check comes before the device check)."""
    import torch
    h = api.hashenc_create({"d": 3, "L": 2, "F": 2, "kind": "hermite", "T": [1 << 10] * 4,
                            "n_min": 4, "n_max": 8, "d2_mode": "diag"})
    n_params, width, _ = api.hashenc_info(h)
    n = 5
    x = torch.zeros(n, 3)
    good = dict(params=torch.zeros(n_params), gamma=torch.zeros(n, width),
                dgamma=torch.zeros(n, 3, width), d2gamma=torch.zeros(n, 3, width))
    # the right sizes pass the size check and stop at the device check
    with pytest.raises(ValueError, match="device"):
        api.hashenc_forward(h, x, **good)
    for key in good:
        bad = dict(good)
        bad[key] = torch.zeros(good[key].numel() - 1)
        with pytest.raises(ValueError, match=key):
            api.hashenc_forward(h, x, **bad)
        with pytest.raises(ValueError, match=key):
            api.hashenc_forward_ws(h, x, **bad, workspace=None)
    with pytest.raises(ValueError, match="x must be"):
        api.hashenc_forward(h, torch.zeros(n, 2), **good)
    ups = dict(g_gamma=torch.zeros(n, width), g_dgamma=torch.zeros(n, 3, width),
               g_d2gamma=torch.zeros(n, 3, width), grad_params=torch.zeros(n_params))
    for key in ups:
        bad = dict(ups)
        bad[key] = torch.zeros(ups[key].numel() + 3)
        with pytest.raises(ValueError, match=key.replace("g_", "") if key != "grad_params" else key):
            api.hashenc_backward(h, x, **bad)
        with pytest.raises(ValueError, match=key.replace("g_", "") if key != "grad_params" else key):
            api.hashenc_backward_ws(h, x, **bad)
    mlp = api.Mlp(4, 16, 2, 30.0)
    n_mlp = api.mlp_param_count(4, 16, 2)
    assert n_mlp == 4 * 16 + 16 + 16 * 16 + 16 + 16 + 1
    with pytest.raises(ValueError, match="mlp_params"):
        api.hashenc_residual(h, mlp, x, good["params"], torch.zeros(n_mlp + 1), None, torch.zeros(1),
                             None, None, torch.zeros(8, dtype=torch.uint8))
    with pytest.raises(ValueError, match="residual"):
        api.hashenc_residual(h, mlp, x, good["params"], torch.zeros(n_mlp), torch.zeros(n - 1), torch.zeros(1),
                             None, None, torch.zeros(8, dtype=torch.uint8))
    with pytest.raises(ValueError, match="out_rows"):
        api.hashenc_debug_indices(h, x, 0, torch.zeros(n * 2 * 8 - 1, dtype=torch.int32))


# ---------------------------------------------------------------- binned chunk bound
def test_binned_chunk_keeps_entries_in_int32():
    """The binned backward indexes a chunk's entries with int32.  A 32-level 3D Hermite grid
    has 32 * 8 * 4 = 1024 entries per point, so a 2^21-point chunk would hold 2^31; the chunk
    is cut to the largest multiple of 1024 points with at most 2^31 - 2^20 entries, and the
    workspace stops growing there."""
    h = api.hashenc_create({"d": 3, "L": 32, "F": 1, "kind": "hermite", "T": [1 << 19] * 4,
                            "n_min": 16, "n_max": 2048, "d2_mode": "laplacian"})
    epp = 32 * 8 * 4
    cap = ((2 ** 31 - 2 ** 20) // epp) // 1024 * 1024
    assert cap * epp < 2 ** 31 - 2 ** 18 and cap < 1 << 21
    ws = lambda n: api.hashenc_backward_workspace_size(h, n)
    assert ws(cap) > 0  # the binned path takes this configuration
    assert ws(1 << 21) == ws(cap) == ws(3 * cap)
    assert ws(cap - 1024) < ws(cap)
    # the fused residual runs one binned chunk per pass: its workspace stops growing there too
    mlp = api.Mlp(32, 64, 2, 30.0)
    rs = lambda n: api.hashenc_residual_workspace_size(h, mlp, n)
    assert rs(1 << 21) == rs(cap) > rs(cap - 1024)
    # 16 levels (the PINN workload) keep the full 2^21-point chunk
    h16 = api.hashenc_create({"d": 3, "L": 16, "F": 2, "kind": "hermite", "T": [1 << 19] * 4,
                              "n_min": 16, "n_max": 1024, "d2_mode": "laplacian"})
    assert api.hashenc_backward_workspace_size(h16, 1 << 21) > api.hashenc_backward_workspace_size(h16, cap)


def test_small_dlinear_batches_take_the_atomic_path():
    """Below n * L = 2^18 a d-linear backward_ws scatters with atomics (no workspace); the
    Hermite kind keeps the binned path at every size; the diagnostic binned entry point sizes
    a workspace at any n."""
    lin = api.hashenc_create({"d": 3, "L": 16, "F": 2, "kind": "dlinear", "T": [1 << 19], "n_min": 16,
                              "n_max": 2048})
    assert api.hashenc_backward_workspace_size(lin, (1 << 14) - 1) == 0
    assert api.hashenc_backward_workspace_size(lin, 1 << 14) > 0
    assert api.hashenc_diag_binned_workspace_size(lin, 100) > 0
    herm = api.hashenc_create({"d": 2, "L": 8, "F": 2, "kind": "hermite", "T": [1 << 14] * 3, "n_min": 16,
                               "n_max": 512, "d2_mode": "laplacian"})
    assert api.hashenc_backward_workspace_size(herm, 1) > 0
    rbf = api.hashenc_create({"d": 2, "L": 2, "F": 2, "kind": "rbf", "T": [1 << 12], "n_min": 8, "n_max": 16,
                              "rbf_eps": 1.0, "rbf_rings": 2})
    with pytest.raises(_lib.HashencError):
        api.hashenc_diag_binned_workspace_size(rbf, 100)


def test_counting_pair_validation_before_launch():
    """hashenc_forward_counting / hashenc_backward_counted: argument errors (NULL, alignment,
    sizes, overlapping workspaces) are reported before any launch."""
    lib = _lib.load()
    h = api.hashenc_create({"d": 3, "L": 16, "F": 2, "kind": "dlinear", "T": [1 << 19], "n_min": 16,
                            "n_max": 2048})
    n = 1 << 15  # binned, one chunk: the counting path
    fneed = api.hashenc_forward_workspace_size(h, n)
    bneed = api.hashenc_backward_workspace_size(h, n)
    assert fneed > 0 and bneed > 0
    P = ctypes.c_void_p
    x, p, g = P(0x10000), P(0x20000), P(0x30000)   # aligned, never dereferenced
    fws, bws = P(1 << 40), P(1 << 41)
    call = lambda *a: lib.hashenc_forward_counting(h, n, *a, None)   # noqa: E731
    assert call(x, p, g, None, None, fws, fneed, None, bneed) == _lib.HASHENC_EINVAL
    assert call(x, p, g, None, None, fws, fneed - 1, bws, bneed) == _lib.HASHENC_EINVAL
    assert call(x, p, g, None, None, fws, fneed, bws, bneed - 1) == _lib.HASHENC_EINVAL
    assert call(x, p, g, None, None, fws, fneed, P((1 << 41) + 4), bneed) == _lib.HASHENC_EALIGN
    assert call(x, p, g, g, None, fws, fneed, bws, bneed) == _lib.HASHENC_EUNSUPPORTED
    # the backward workspace starting inside the forward's
    assert call(x, p, g, None, None, fws, fneed, P((1 << 40) + 256), bneed) == _lib.HASHENC_EINVAL
    back = lambda *a: lib.hashenc_backward_counted(h, n, *a, None)   # noqa: E731
    assert back(x, g, None, None, p, bws, bneed - 1) == _lib.HASHENC_EINVAL
    assert back(x, g, None, None, p, None, bneed) == _lib.HASHENC_EINVAL
    assert back(x, g, g, None, p, bws, bneed) == _lib.HASHENC_EUNSUPPORTED
    assert back(x, g, None, None, P(0x20004), bws, bneed) == _lib.HASHENC_EALIGN
    assert back(x, None, None, None, p, bws, bneed) == 0   # no upstream: nothing to add
