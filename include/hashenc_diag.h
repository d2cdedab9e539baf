/*
 * hashenc diagnostics: entry points for parity testing and bandwidth calibration.
 * Same conventions as hashenc.h (device pointers owned by the caller, 0 / HASHENC_E*
 * return codes, asynchronous on `stream`).
 */
#ifndef HASHENC_DIAG_H
#define HASHENC_DIAG_H

#include "hashenc.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Export the lookup stage: for every point and level, the row of table `order` that each of
 * the 2^d cell corners maps to (dense 1:1 index or spatial hash mod T; see hashenc.h for
 * the rules).  out_rows [n, L, 2^d] int32, corner bit i = +1 along axis i.  Computed by
 * the same device code the forward and backward kernels use. */
HASHENC_API int hashenc_debug_indices(const hashenc* h, int64_t n, const float* x, int32_t order,
                          int32_t* out_rows, hashenc_stream_t stream);

/* The binned backward of hashenc_backward_ws at any n, for testing its kernels on small
 * batches (which hashenc_backward_ws itself may hand to the atomic scatter-add).  Same
 * arguments and result as hashenc_backward_ws; HASHENC_EUNSUPPORTED when the configuration
 * has no binned plan.  hashenc_diag_binned_workspace_size gives the workspace it needs. */
HASHENC_API int hashenc_diag_binned_workspace_size(const hashenc* h, int64_t n, size_t* bytes);
HASHENC_API int hashenc_diag_backward_binned(const hashenc* h, int64_t n, const float* x, const float* g_gamma,
                                             const float* g_dgamma, const float* g_d2gamma, float* grad_params,
                                             void* workspace, size_t workspace_bytes, hashenc_stream_t stream);

/* The workspace forward of hashenc_forward_ws with the packed order tables at any n, for
 * testing the packed path on small batches (which hashenc_forward_ws itself hands to the
 * direct forward below 32768 points for 2D and 3D Hermite grids).  Same arguments, workspace
 * (hashenc_forward_workspace_size) and results as hashenc_forward_ws. */
HASHENC_API int hashenc_diag_forward_packed(const hashenc* h, int64_t n, const float* x, const float* params,
                                            float* gamma, float* dgamma, float* d2gamma, void* workspace,
                                            size_t workspace_bytes, hashenc_stream_t stream);

/* Plain streaming copy dst[i] = src[i], i < n_floats (both 16-byte aligned, no overlap).
 * Used to measure achievable HBM bandwidth and to calibrate memory counters. */
HASHENC_API int hashenc_diag_copy(const float* src, float* dst, int64_t n_floats, hashenc_stream_t stream);

/* L2-resident read: buf (n_floats, a positive multiple of 32, 16-byte aligned) is cut into
 * 8 equal slices, one per XCD, and each XCD's workgroups read their slice `reps` times
 * (reps >= 1), so that with slices of at most a few MB every pass after the first is served
 * by the XCD's L2.  Gives the L2 read ceiling (bytes = 4 * n_floats * reps) and, under a
 * counter run, the L2 request rate the gather kernels are compared with.  buf should hold
 * ones: out (one float) is written only if the sum is -1, which such a buffer cannot give. */
HASHENC_API int hashenc_diag_cache_read(const float* buf, int64_t n_floats, int32_t reps, float* out,
                                        hashenc_stream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* HASHENC_DIAG_H */
