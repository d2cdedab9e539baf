"""Thin Python binding over the C ABI in ``include/hashenc.h``.

Functions keep the C names and only marshal arguments: torch tensors are checked (device,
dtype, contiguity) and passed as raw device pointers with the current HIP stream.  Every
step of the computation runs in the HIP library.  PyTorch supplies device memory and
streams only.
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass

import torch

from . import _lib
from ._lib import check, load


def _spec_to_config(spec: dict) -> tuple[_lib.HashencConfig, object]:
    cfg = _lib.HashencConfig()
    cfg.d = int(spec["d"])
    cfg.n_levels = int(spec["L"])
    cfg.n_features = int(spec["F"])
    cfg.kind = {"dlinear": _lib.HASHENC_DLINEAR, "hermite": _lib.HASHENC_HERMITE, "rbf": _lib.HASHENC_RBF}[spec["kind"]]
    cfg.d2_mode = (_lib.HASHENC_D2_DIAG if spec.get("d2_mode") == "diag" else _lib.HASHENC_D2_LAPLACIAN)
    cfg.n_min = int(spec.get("n_min", 0))
    cfg.n_max = int(spec.get("n_max", 0))
    cfg.reserved = 0
    cfg.growth = float(spec.get("growth") or 0.0)
    cfg.rbf_eps = float(spec.get("rbf_eps") or 0.0)
    cfg.rbf_rings = int(spec.get("rbf_rings") or 0)
    cfg.reserved2 = 0
    T = list(spec["T"])
    n_tab = cfg.d + 1 if cfg.kind == _lib.HASHENC_HERMITE else 1
    if len(T) == 1:
        T = T * n_tab
    for k in range(min(len(T), 5)):
        cfg.table_size[k] = int(T[k])
    keep = None
    if spec.get("resolutions") is not None:
        keep = (ctypes.c_int32 * cfg.n_levels)(*[int(v) for v in spec["resolutions"]])
        cfg.resolutions = ctypes.cast(keep, ctypes.POINTER(ctypes.c_int32))
    return cfg, keep


class Handle:
    """Owns one ``hashenc*``; destroyed with the object."""

    def __init__(self, ptr: int, spec: dict):
        self.ptr = ctypes.c_void_p(ptr)
        self.spec = dict(spec)
        self._sizes = None  # (n_params, L*F), read from the library on first use

    def __del__(self):
        # at interpreter shutdown the module globals may already be gone
        lib = getattr(_lib, "_lib", None) if _lib is not None else None
        if getattr(self, "ptr", None) is not None and self.ptr.value and lib is not None:
            lib.hashenc_destroy(self.ptr)
            self.ptr = None

    @property
    def _as_parameter_(self):
        return self.ptr


def _dev_ptr(t: torch.Tensor | None, name: str, dtype=torch.float32):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device (cuda/HIP) tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _sizes(h: Handle) -> tuple[int, int]:
    if h._sizes is None:
        n_params, width = ctypes.c_int64(), ctypes.c_int32()
        check(load().hashenc_info(h, ctypes.byref(n_params), ctypes.byref(width), None))
        h._sizes = (int(n_params.value), int(width.value))
    return h._sizes


def _expect(t, numel: int, name: str) -> None:
    """Size check of an optional tensor argument, before any pointer reaches the library:
    the kernels trust the sizes the layout implies, so a short buffer would be overrun on
    the device."""
    if t is None:
        return
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.numel() != numel:
        raise ValueError(f"{name} holds {t.numel()} elements; this call needs {numel}")


def _points(h: Handle, x) -> int:
    """n from x [n, d] (checked)."""
    if not isinstance(x, torch.Tensor):
        raise TypeError("x must be a torch.Tensor")
    d = int(h.spec["d"])
    if x.dim() != 2 or x.shape[1] != d:
        raise ValueError(f"x must be [n, {d}] (got {list(x.shape)})")
    return int(x.shape[0])


def _check_encoder_io(h: Handle, n: int, params=None, gamma=None, dgamma=None, d2gamma=None,
                      grad_params=None) -> None:
    n_params, width = _sizes(h)
    d = int(h.spec["d"])
    d2 = d if h.spec.get("d2_mode") == "diag" else 1
    _expect(params, n_params, "params")
    _expect(grad_params, n_params, "grad_params")
    _expect(gamma, n * width, "gamma")
    _expect(dgamma, n * d * width, "dgamma")
    _expect(d2gamma, n * d2 * width, "d2gamma")


def mlp_param_count(n_in: int, hidden: int, depth: int) -> int:
    """Floats of the packed SIREN parameters W1, b1, ..., Wo, bo (output width 1)."""
    n = 0
    for k in range(depth + 1):
        fi = n_in if k == 0 else hidden
        fo = 1 if k == depth else hidden
        n += fi * fo + fo
    return n


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def hashenc_create(spec: dict) -> Handle:
    cfg, keep = _spec_to_config(spec)
    out = ctypes.c_void_p()
    check(load().hashenc_create(ctypes.byref(cfg), ctypes.byref(out)))
    del keep
    return Handle(out.value, spec)


def hashenc_destroy(h: Handle) -> None:
    if h.ptr is not None and h.ptr.value:
        load().hashenc_destroy(h.ptr)
        h.ptr = None


def hashenc_info(h: Handle) -> tuple[int, int, list[int]]:
    n_params = ctypes.c_int64()
    width = ctypes.c_int32()
    res = (ctypes.c_int32 * _lib.MAX_LEVELS)()
    check(load().hashenc_info(h, ctypes.byref(n_params), ctypes.byref(width), res))
    return n_params.value, width.value, [int(v) for v in res[: int(h.spec["L"])]]


def hashenc_derive_active(h: Handle, n_active: int) -> Handle:
    """Handle computing only the first n_active levels (coarse-to-fine activation)."""
    out = ctypes.c_void_p()
    check(load().hashenc_derive_active(h, int(n_active), ctypes.byref(out)))
    return Handle(out.value, dict(h.spec, active_levels=int(n_active)))


def hashenc_active_levels(h: Handle) -> int:
    a = ctypes.c_int32()
    check(load().hashenc_active_levels(h, ctypes.byref(a)))
    return int(a.value)


def hashenc_c2f_active_levels(n_levels: int, l0: int, step: int, tau: int) -> int:
    a = ctypes.c_int32()
    check(load().hashenc_c2f_active_levels(int(n_levels), int(l0), int(step), int(tau), ctypes.byref(a)))
    return int(a.value)


def hashenc_param_layout(h: Handle, order: int, level: int) -> dict:
    off, rows = ctypes.c_int64(), ctypes.c_int64()
    width, dense = ctypes.c_int32(), ctypes.c_int32()
    check(load().hashenc_param_layout(h, order, level, ctypes.byref(off), ctypes.byref(rows),
                                      ctypes.byref(width), ctypes.byref(dense)))
    return {"offset": off.value, "rows": rows.value, "width": width.value, "dense": bool(dense.value)}


def hashenc_forward(h: Handle, x: torch.Tensor, params: torch.Tensor, gamma=None, dgamma=None,
                    d2gamma=None, stream=None) -> None:
    n = _points(h, x)
    _check_encoder_io(h, n, params, gamma, dgamma, d2gamma)
    check(load().hashenc_forward(h, n, _dev_ptr(x, "x"), _dev_ptr(params, "params"),
                                 _dev_ptr(gamma, "gamma"), _dev_ptr(dgamma, "dgamma"),
                                 _dev_ptr(d2gamma, "d2gamma"), _stream(stream)))


def hashenc_backward(h: Handle, x: torch.Tensor, g_gamma=None, g_dgamma=None, g_d2gamma=None,
                     grad_params=None, stream=None) -> None:
    n = _points(h, x)
    _check_encoder_io(h, n, None, g_gamma, g_dgamma, g_d2gamma, grad_params)
    check(load().hashenc_backward(h, n, _dev_ptr(x, "x"), _dev_ptr(g_gamma, "g_gamma"),
                                  _dev_ptr(g_dgamma, "g_dgamma"), _dev_ptr(g_d2gamma, "g_d2gamma"),
                                  _dev_ptr(grad_params, "grad_params"), _stream(stream)))


def hashenc_forward_workspace_size(h: Handle, n: int) -> int:
    b = ctypes.c_size_t()
    check(load().hashenc_forward_workspace_size(h, n, ctypes.byref(b)))
    return int(b.value)


def _ws(workspace):
    if workspace is None:
        return None, 0
    if workspace.device.type != "cuda":
        raise ValueError("workspace must be a device tensor")
    return ctypes.c_void_p(workspace.data_ptr()), workspace.numel() * workspace.element_size()


def hashenc_forward_ws(h: Handle, x: torch.Tensor, params: torch.Tensor, gamma=None, dgamma=None,
                       d2gamma=None, workspace: torch.Tensor | None = None, stream=None) -> None:
    n = _points(h, x)
    _check_encoder_io(h, n, params, gamma, dgamma, d2gamma)
    ws_ptr, ws_bytes = _ws(workspace)
    check(load().hashenc_forward_ws(h, n, _dev_ptr(x, "x"), _dev_ptr(params, "params"),
                                    _dev_ptr(gamma, "gamma"), _dev_ptr(dgamma, "dgamma"),
                                    _dev_ptr(d2gamma, "d2gamma"), ws_ptr, ws_bytes, _stream(stream)))


def hashenc_diag_forward_packed(h: Handle, x: torch.Tensor, params: torch.Tensor, gamma=None, dgamma=None,
                                d2gamma=None, workspace: torch.Tensor | None = None, stream=None) -> None:
    """The workspace forward with the packed tables at any batch size (diagnostics)."""
    n = _points(h, x)
    _check_encoder_io(h, n, params, gamma, dgamma, d2gamma)
    ws_ptr, ws_bytes = _ws(workspace)
    check(load().hashenc_diag_forward_packed(h, n, _dev_ptr(x, "x"), _dev_ptr(params, "params"),
                                             _dev_ptr(gamma, "gamma"), _dev_ptr(dgamma, "dgamma"),
                                             _dev_ptr(d2gamma, "d2gamma"), ws_ptr, ws_bytes, _stream(stream)))


def hashenc_backward_workspace_size(h: Handle, n: int) -> int:
    b = ctypes.c_size_t()
    check(load().hashenc_backward_workspace_size(h, n, ctypes.byref(b)))
    return int(b.value)


def hashenc_backward_ws(h: Handle, x: torch.Tensor, g_gamma=None, g_dgamma=None, g_d2gamma=None,
                        grad_params=None, workspace: torch.Tensor | None = None, stream=None) -> None:
    n = _points(h, x)
    _check_encoder_io(h, n, None, g_gamma, g_dgamma, g_d2gamma, grad_params)
    ws_ptr, ws_bytes = _ws(workspace)
    check(load().hashenc_backward_ws(h, n, _dev_ptr(x, "x"), _dev_ptr(g_gamma, "g_gamma"),
                                     _dev_ptr(g_dgamma, "g_dgamma"), _dev_ptr(g_d2gamma, "g_d2gamma"),
                                     _dev_ptr(grad_params, "grad_params"), ws_ptr, ws_bytes, _stream(stream)))


def hashenc_forward_counting(h: Handle, x: torch.Tensor, params: torch.Tensor, gamma=None, dgamma=None,
                             d2gamma=None, workspace: torch.Tensor | None = None,
                             bwd_workspace: torch.Tensor | None = None, stream=None) -> None:
    """hashenc_forward_ws that also leaves the binned backward's counts of x in bwd_workspace."""
    n = _points(h, x)
    _check_encoder_io(h, n, params, gamma, dgamma, d2gamma)
    ws_ptr, ws_bytes = _ws(workspace)
    bws_ptr, bws_bytes = _ws(bwd_workspace)
    check(load().hashenc_forward_counting(h, n, _dev_ptr(x, "x"), _dev_ptr(params, "params"),
                                          _dev_ptr(gamma, "gamma"), _dev_ptr(dgamma, "dgamma"),
                                          _dev_ptr(d2gamma, "d2gamma"), ws_ptr, ws_bytes, bws_ptr, bws_bytes,
                                          _stream(stream)))


def hashenc_backward_counted(h: Handle, x: torch.Tensor, g_gamma=None, g_dgamma=None, g_d2gamma=None,
                             grad_params=None, bwd_workspace: torch.Tensor | None = None, stream=None) -> None:
    """hashenc_backward_ws starting from the counts hashenc_forward_counting left for the same x."""
    n = _points(h, x)
    _check_encoder_io(h, n, None, g_gamma, g_dgamma, g_d2gamma, grad_params)
    ws_ptr, ws_bytes = _ws(bwd_workspace)
    check(load().hashenc_backward_counted(h, n, _dev_ptr(x, "x"), _dev_ptr(g_gamma, "g_gamma"),
                                          _dev_ptr(g_dgamma, "g_dgamma"), _dev_ptr(g_d2gamma, "g_d2gamma"),
                                          _dev_ptr(grad_params, "grad_params"), ws_ptr, ws_bytes,
                                          _stream(stream)))


def hashenc_backward_noalloc(h: Handle, x: torch.Tensor, g_gamma=None, g_dgamma=None, g_d2gamma=None,
                             grad_params=None, stream=None) -> None:
    """The binned backward on the library's static scratch (no workspace, nothing allocated);
    calls on one GPU must not overlap."""
    n = _points(h, x)
    _check_encoder_io(h, n, None, g_gamma, g_dgamma, g_d2gamma, grad_params)
    check(load().hashenc_backward_noalloc(h, n, _dev_ptr(x, "x"), _dev_ptr(g_gamma, "g_gamma"),
                                          _dev_ptr(g_dgamma, "g_dgamma"), _dev_ptr(g_d2gamma, "g_d2gamma"),
                                          _dev_ptr(grad_params, "grad_params"), _stream(stream)))


@dataclass
class Mlp:
    n_in: int
    hidden: int
    depth: int
    omega: float

    def as_c(self) -> _lib.HashencMlp:
        m = _lib.HashencMlp()
        m.in_, m.hidden, m.depth, m.out, m.omega, m.reserved = self.n_in, self.hidden, self.depth, 1, self.omega, 0
        return m


def hashenc_residual_workspace_size(h: Handle, mlp: Mlp, n: int) -> int:
    b = ctypes.c_size_t()
    m = mlp.as_c()
    check(load().hashenc_residual_workspace_size(h, ctypes.byref(m), n, ctypes.byref(b)))
    return int(b.value)


def hashenc_residual(h: Handle, mlp: Mlp, x: torch.Tensor, params: torch.Tensor,
                     mlp_params: torch.Tensor, residual, loss: torch.Tensor, grad_params,
                     grad_mlp, workspace: torch.Tensor, stream=None) -> None:
    n = _points(h, x)
    _check_encoder_io(h, n, params, grad_params=grad_params)
    n_mlp = mlp_param_count(mlp.n_in, mlp.hidden, mlp.depth)
    _expect(mlp_params, n_mlp, "mlp_params")
    _expect(grad_mlp, n_mlp, "grad_mlp")
    _expect(residual, n, "residual")
    _expect(loss, 1, "loss")
    m = mlp.as_c()
    check(load().hashenc_residual(h, ctypes.byref(m), n, _dev_ptr(x, "x"),
                                  _dev_ptr(params, "params"), _dev_ptr(mlp_params, "mlp_params"),
                                  _dev_ptr(residual, "residual"), _dev_ptr(loss, "loss"),
                                  _dev_ptr(grad_params, "grad_params"), _dev_ptr(grad_mlp, "grad_mlp"),
                                  _dev_ptr(workspace, "workspace", dtype=workspace.dtype),
                                  workspace.numel() * workspace.element_size(), _stream(stream)))


def hashenc_fd_residual_workspace_size(h: Handle, mlp: Mlp, n: int) -> int:
    b = ctypes.c_size_t()
    m = mlp.as_c()
    check(load().hashenc_fd_residual_workspace_size(h, ctypes.byref(m), n, ctypes.byref(b)))
    return int(b.value)


def hashenc_fd_residual(h: Handle, mlp: Mlp, eps: float, x: torch.Tensor, params: torch.Tensor,
                        mlp_params: torch.Tensor, u_stencil, residual, loss: torch.Tensor, grad_params,
                        grad_mlp, workspace: torch.Tensor, stream=None) -> None:
    n = _points(h, x)
    _check_encoder_io(h, n, params, grad_params=grad_params)
    n_mlp = mlp_param_count(mlp.n_in, mlp.hidden, mlp.depth)
    _expect(mlp_params, n_mlp, "mlp_params")
    _expect(grad_mlp, n_mlp, "grad_mlp")
    _expect(u_stencil, n * (2 * int(h.spec["d"]) + 1), "u_stencil")
    _expect(residual, n, "residual")
    _expect(loss, 1, "loss")
    m = mlp.as_c()
    check(load().hashenc_fd_residual(h, ctypes.byref(m), float(eps), n, _dev_ptr(x, "x"),
                                     _dev_ptr(params, "params"), _dev_ptr(mlp_params, "mlp_params"),
                                     _dev_ptr(u_stencil, "u_stencil"), _dev_ptr(residual, "residual"),
                                     _dev_ptr(loss, "loss"), _dev_ptr(grad_params, "grad_params"),
                                     _dev_ptr(grad_mlp, "grad_mlp"),
                                     _dev_ptr(workspace, "workspace", dtype=workspace.dtype),
                                     workspace.numel() * workspace.element_size(), _stream(stream)))


def hashenc_debug_indices(h: Handle, x: torch.Tensor, order: int, out_rows: torch.Tensor,
                          stream=None) -> None:
    n = _points(h, x)
    _expect(out_rows, n * int(h.spec["L"]) * (1 << int(h.spec["d"])), "out_rows")
    check(load().hashenc_debug_indices(h, n, _dev_ptr(x, "x"), order,
                                       _dev_ptr(out_rows, "out_rows", dtype=torch.int32), _stream(stream)))


def hashenc_diag_binned_workspace_size(h: Handle, n: int) -> int:
    b = ctypes.c_size_t()
    check(load().hashenc_diag_binned_workspace_size(h, n, ctypes.byref(b)))
    return int(b.value)


def hashenc_diag_backward_binned(h: Handle, x: torch.Tensor, g_gamma=None, g_dgamma=None, g_d2gamma=None,
                                 grad_params=None, workspace: torch.Tensor | None = None, stream=None) -> None:
    """The binned backward at any batch size (diagnostics: its kernels on small batches)."""
    n = _points(h, x)
    _check_encoder_io(h, n, None, g_gamma, g_dgamma, g_d2gamma, grad_params)
    if workspace is None:
        b = hashenc_diag_binned_workspace_size(h, n)
        workspace = torch.empty(max(b, 1), dtype=torch.uint8, device=x.device)
    ws_ptr, ws_bytes = _ws(workspace)
    check(load().hashenc_diag_backward_binned(h, n, _dev_ptr(x, "x"), _dev_ptr(g_gamma, "g_gamma"),
                                              _dev_ptr(g_dgamma, "g_dgamma"), _dev_ptr(g_d2gamma, "g_d2gamma"),
                                              _dev_ptr(grad_params, "grad_params"), ws_ptr, ws_bytes,
                                              _stream(stream)))


def hashenc_diag_copy(src: torch.Tensor, dst: torch.Tensor, stream=None) -> None:
    _expect(dst, src.numel(), "dst")
    check(load().hashenc_diag_copy(_dev_ptr(src, "src"), _dev_ptr(dst, "dst"), src.numel(), _stream(stream)))


def hashenc_diag_cache_read(buf: torch.Tensor, reps: int, out: torch.Tensor, stream=None) -> None:
    check(load().hashenc_diag_cache_read(_dev_ptr(buf, "buf"), buf.numel(), int(reps), _dev_ptr(out, "out"),
                                         _stream(stream)))


class HashGridEncoding:
    """Convenience wrapper: a handle plus output allocation (torch tensors on the GPU)."""

    def __init__(self, spec: dict):
        self.spec = dict(spec)
        self._full = hashenc_create(spec)
        self.handle = self._full
        self.n_params, self.out_width, self.resolutions = hashenc_info(self.handle)
        if spec.get("active_levels") is not None:
            self.set_active_levels(spec["active_levels"])
        self.d = int(spec["d"])
        self.hermite = spec["kind"] == "hermite"
        self.derivatives = spec["kind"] in ("hermite", "rbf")  # outputs grad gamma, d2 gamma
        self.diag = spec.get("d2_mode") == "diag"

    def set_active_levels(self, n_active: int) -> None:
        """Coarse-to-fine activation: compute only levels l < n_active from now on (outputs
        keep the full width; inactive columns are zero and get no gradient)."""
        n_active = int(n_active)
        self.handle = self._full if n_active == len(self.resolutions) else hashenc_derive_active(self._full, n_active)

    @property
    def active_levels(self) -> int:
        return hashenc_active_levels(self.handle)

    def output_shapes(self, n: int) -> dict:
        s = {"gamma": (n, self.out_width)}
        if self.derivatives:
            s["dgamma"] = (n, self.d, self.out_width)
            s["d2gamma"] = (n, self.d, self.out_width) if self.diag else (n, self.out_width)
        return s

    def forward(self, x: torch.Tensor, params: torch.Tensor, stream=None) -> dict:
        out = {k: torch.empty(v, device=x.device, dtype=torch.float32)
               for k, v in self.output_shapes(x.shape[0]).items()}
        hashenc_forward(self.handle, x, params, out["gamma"], out.get("dgamma"), out.get("d2gamma"), stream)
        return out

    def backward(self, x: torch.Tensor, grad_params: torch.Tensor, g_gamma=None, g_dgamma=None,
                 g_d2gamma=None, stream=None) -> torch.Tensor:
        """Atomic scatter-add backward (no workspace)."""
        hashenc_backward(self.handle, x, g_gamma, g_dgamma, g_d2gamma, grad_params, stream)
        return grad_params

    def forward_workspace(self, n: int) -> torch.Tensor | None:
        b = hashenc_forward_workspace_size(self.handle, n)
        return torch.empty(b, dtype=torch.uint8, device="cuda") if b else None

    def backward_workspace(self, n: int) -> torch.Tensor | None:
        b = hashenc_backward_workspace_size(self.handle, n)
        return torch.empty(b, dtype=torch.uint8, device="cuda") if b else None

    def workspace(self, n: int) -> torch.Tensor | None:
        """A device workspace for forward_ws and backward_ws on n points (None when neither
        uses one); the two calls may share it when they do not overlap."""
        b = max(hashenc_backward_workspace_size(self.handle, n), hashenc_forward_workspace_size(self.handle, n))
        return torch.empty(b, dtype=torch.uint8, device="cuda") if b else None

    def forward_ws(self, x: torch.Tensor, params: torch.Tensor, workspace=None, stream=None) -> dict:
        out = {k: torch.empty(v, device=x.device, dtype=torch.float32)
               for k, v in self.output_shapes(x.shape[0]).items()}
        if workspace is None:
            workspace = self.workspace(x.shape[0])
        hashenc_forward_ws(self.handle, x, params, out["gamma"], out.get("dgamma"), out.get("d2gamma"),
                           workspace, stream)
        return out

    def forward_packed(self, x: torch.Tensor, params: torch.Tensor, workspace=None, stream=None) -> dict:
        """The workspace forward with the packed tables whatever the batch size (diagnostics)."""
        out = {k: torch.empty(v, device=x.device, dtype=torch.float32)
               for k, v in self.output_shapes(x.shape[0]).items()}
        if workspace is None:
            workspace = self.workspace(x.shape[0])
        hashenc_diag_forward_packed(self.handle, x, params, out["gamma"], out.get("dgamma"), out.get("d2gamma"),
                                    workspace, stream)
        return out

    def forward_counting(self, x: torch.Tensor, params: torch.Tensor, workspace: torch.Tensor,
                         bwd_workspace: torch.Tensor, stream=None) -> dict:
        """forward_ws that also prepares backward_counted on the same x (two separate, non-overlapping
        workspaces: forward_workspace(n) and backward_workspace(n))."""
        out = {k: torch.empty(v, device=x.device, dtype=torch.float32)
               for k, v in self.output_shapes(x.shape[0]).items()}
        hashenc_forward_counting(self.handle, x, params, out["gamma"], out.get("dgamma"), out.get("d2gamma"),
                                 workspace, bwd_workspace, stream)
        return out

    def backward_counted(self, x: torch.Tensor, grad_params: torch.Tensor, g_gamma=None, g_dgamma=None,
                         g_d2gamma=None, bwd_workspace=None, stream=None) -> torch.Tensor:
        """backward_ws after forward_counting on the same x and bwd_workspace."""
        hashenc_backward_counted(self.handle, x, g_gamma, g_dgamma, g_d2gamma, grad_params, bwd_workspace, stream)
        return grad_params

    def backward_binned(self, x: torch.Tensor, grad_params: torch.Tensor, g_gamma=None, g_dgamma=None,
                        g_d2gamma=None, stream=None) -> torch.Tensor:
        """The binned backward whatever the batch size (diagnostics)."""
        hashenc_diag_backward_binned(self.handle, x, g_gamma, g_dgamma, g_d2gamma, grad_params, None, stream)
        return grad_params

    def backward_ws(self, x: torch.Tensor, grad_params: torch.Tensor, g_gamma=None, g_dgamma=None,
                    g_d2gamma=None, workspace=None, stream=None) -> torch.Tensor:
        """Binned backward (no global atomics on the hot part); allocates a workspace when
        none is given."""
        if workspace is None:
            workspace = self.workspace(x.shape[0])
        hashenc_backward_ws(self.handle, x, g_gamma, g_dgamma, g_d2gamma, grad_params, workspace, stream)
        return grad_params
