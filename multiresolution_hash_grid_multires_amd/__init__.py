"""Multiresolution hash-grid encoding (Instant-NGP d-linear and Hermite-NGP) for MI355X.

The computation lives in the HIP library ``libhashenc.so`` (C ABI: ``include/hashenc.h``);
this package is its thin ctypes binding plus seeded synthetic workloads.
"""
from .api import (  # noqa: F401
    HashGridEncoding,
    Mlp,
    hashenc_backward,
    hashenc_backward_workspace_size,
    hashenc_backward_ws,
    hashenc_create,
    hashenc_debug_indices,
    hashenc_destroy,
    hashenc_diag_cache_read,
    hashenc_diag_copy,
    hashenc_forward,
    hashenc_forward_workspace_size,
    hashenc_forward_ws,
    hashenc_info,
    hashenc_param_layout,
    hashenc_residual,
    hashenc_residual_workspace_size,
)
from ._lib import HashencError, LIB_PATH  # noqa: F401
