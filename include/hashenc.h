/*
 * hashenc — multiresolution hash-grid encoding on AMD Instinct MI355X (gfx950).
 *
 * C ABI.  Plain pointers and sizes only.  Unless a comment says "host", every pointer
 * argument is a DEVICE pointer to memory owned by the caller; the library never frees or
 * retains it.  The handle owns host metadata only (no device memory), is immutable after
 * creation, and may be used from several threads on several streams at once.
 *
 * The method (sources are the public pages this library was written from):
 *  - Instant-NGP multiresolution hash encoding: "SIGGRAPH 2022 | InstantNGP and
 *    multiresolution hash encoding" (nxrte.com), section on the encoding pipeline
 *    (per level: the 2^d cell vertices around x, table lookup, d-linear interpolation,
 *    concatenation over levels; the 1:1 map at coarse levels and the spatial hash at fine
 *    ones), and the Instant-NGP news article (antipu.com.cn), paragraphs on adaptivity
 *    (L levels of up to T F-dimensional vectors; colliding gradients combine) and on
 *    efficiency (no control flow; all levels looked up in parallel), and the Figure 3
 *    paragraph (levels in geometric progression between N_min and N_max).
 *  - Hermite-NGP gradient-augmented encoding: "Hermite-NGP: Gradient-Augmented Hash
 *    Encoding for Learning PDEs" notes (m0rtzz.github.io), key design 1 (tables bucketed
 *    by derivative order holding all 2^d mixed partials per vertex; tensor-product cubic
 *    Hermite reconstruction with the Delta x^{|alpha|} scaling) and key design 2 (analytic
 *    first and second derivatives of the basis; SIREN chain rule).
 *
 * Readings fixed by this library where the pages lost the formula (stated once here):
 *  - N_l = floor(N_min * b^l + 1e-6) in fp64, b = exp((ln N_max - ln N_min)/(L-1)) unless
 *    a growth factor b or an explicit list is given;
 *  - spatial hash of integer vertex v: XOR over axes of (v_i * pi_i mod 2^32),
 *    pi = (1, 2654435761, 805459861), reduced mod T;
 *  - a (table, level) is a dense 1:1 grid iff (N_l+1)^d <= T; then row = sum_i v_i (N_l+1)^i;
 *    it stores min(T, (N_l+1)^d) rows;
 *  - vertices sit at v / N_l; p = x * N_l is ONE rounded fp32 multiply, base =
 *    min(floor(p), N_l - 1), t = p - base; x is clamped to [0, 1] (NaN -> 0);
 *  - Hermite: d+1 tables, table k holds the C(d,k) derivative slots of order k in
 *    lexicographic axis order (x, y, z | xy, xz, yz | xyz), each slot F floats;
 *  - colliding rows receive the SUM of their gradient contributions.
 *
 * Return codes: 0 on success, a negative HASHENC_E* code otherwise; hashenc_last_error()
 * then returns a message (thread-local).  All argument checks happen before any launch.
 * Launches are asynchronous on `stream` (NULL = the null stream); device faults surface at
 * the caller's next synchronisation.  Nothing throws or aborts across this boundary.
 */
#ifndef HASHENC_H
#define HASHENC_H

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__)
#define HASHENC_API __attribute__((visibility("default")))
#else
#define HASHENC_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* hashenc_stream_t; /* a hipStream_t */

enum {
  HASHENC_OK = 0,
  HASHENC_EINVAL = -1,       /* bad configuration, size or NULL required pointer */
  HASHENC_EALIGN = -2,       /* a device pointer is not 16-byte aligned */
  HASHENC_ENOMEM = -3,       /* host allocation failed */
  HASHENC_EHIP = -4,         /* a HIP runtime / launch error (message has hipGetErrorString) */
  HASHENC_EUNSUPPORTED = -5  /* valid request the library does not implement */
};

/* HASHENC_RBF: the DInf-Grid Gaussian-RBF interpolant (DInf-Grid summary, sections
 * 可微的径向基函数插值 and 多分辨率特征网格): per level, the features of the vertices of the
 * point's k-ring neighbourhood -- the (2k)^d vertex box around its cell, clipped to the grid
 * -- weighted by phi(r) / sum phi, phi(r) = exp(-(eps r)^2), r the distance in units of the
 * level's grid spacing; one table of F floats per vertex per level (dense 1:1 where the
 * vertices fit table_size[0], else hashed as d-linear); outputs gamma, grad gamma and the
 * second derivatives like the Hermite kind. */
typedef enum { HASHENC_DLINEAR = 0, HASHENC_HERMITE = 1, HASHENC_RBF = 2 } hashenc_kind;
typedef enum { HASHENC_D2_LAPLACIAN = 1, HASHENC_D2_DIAG = 2 } hashenc_d2_mode;

#define HASHENC_MAX_LEVELS 32

typedef struct hashenc_config {
  int32_t d;             /* spatial dimension: 2 or 3; the Hermite kind also 4 (space-time:
                            Hermite-NGP notes, 局限与展望 -- 16 coefficients per vertex) */
  int32_t n_levels;      /* L: 1..32 */
  int32_t n_features;    /* F: 1, 2, 4 or 8 features per derivative slot */
  int32_t kind;          /* hashenc_kind */
  int32_t d2_mode;       /* Hermite and RBF: hashenc_d2_mode of the second-order output */
  int32_t n_min;         /* N_min >= 1: coarsest resolution */
  int32_t n_max;         /* N_max >= N_min: finest resolution (used when growth <= 0) */
  int32_t reserved;      /* must be 0 */
  double growth;         /* b > 0: N_l = floor(N_min b^l + 1e-6); <= 0: derived from n_max */
  uint32_t table_size[5];/* T_k >= 1 rows for table k (derivative order k); d-linear and RBF
                            use [0]; Hermite uses [0..d].  Powers of two take a mask fast path */
  const int32_t* resolutions; /* host, optional: explicit N_l[L] (each 1..2^20); overrides
                                 n_min/n_max/growth when not NULL */
  double rbf_eps;        /* RBF only: shape parameter eps > 0 (finite); ignored otherwise */
  int32_t rbf_rings;     /* RBF only: neighbourhood rings k, 1..4; ignored otherwise */
  int32_t reserved2;     /* must be 0 */
} hashenc_config;

typedef struct hashenc hashenc; /* opaque */

/* Validate `cfg` (host) and build a handle.  *out is set only on success. */
HASHENC_API int hashenc_create(const hashenc_config* cfg, hashenc** out);

/* Release a handle.  NULL is accepted. */
HASHENC_API void hashenc_destroy(hashenc* h);

/* Sizes (host outputs, each may be NULL): total parameter floats, output width L*F, and the
 * level resolutions N_l (array of L). */
HASHENC_API int hashenc_info(const hashenc* h, int64_t* n_params, int32_t* out_width, int32_t* resolutions);

/* Coarse-to-fine level activation (Hermite-NGP reading notes, section 方法详解, key design 3:
 * train the coarse levels first and activate finer ones step by step).
 *
 * hashenc_derive_active: a new handle (*out, host; release with hashenc_destroy) that
 * shares h's configuration and parameter layout but computes only the first n_active
 * levels (levels l < n_active; 1 <= n_active <= L).  Every entry point keeps the full L*F
 * row width: on such a handle the forward writes zeros in the columns of the inactive
 * levels, the backward adds nothing to their parameter blocks (and ignores the upstream
 * there), and the fused residual feeds zeros to the network for them.  Deriving from a
 * derived handle counts levels of the same configuration.  No device memory is involved.
 * HASHENC_EINVAL on a NULL pointer or n_active outside 1..L. */
HASHENC_API int hashenc_derive_active(const hashenc* h, int32_t n_active, hashenc** out);

/* Active level count of a handle (host output): L unless derived with fewer. */
HASHENC_API int hashenc_active_levels(const hashenc* h, int32_t* n_active);

/* The schedule L_active(t) = min(L, L0 + floor(t / tau)) of the same passage, as a count of
 * active levels at training step `step` (host output).  HASHENC_EINVAL unless n_levels >= 1,
 * l0 >= 1, step >= 0 and tau >= 1. */
HASHENC_API int hashenc_c2f_active_levels(int32_t n_levels, int32_t l0, int64_t step, int64_t tau,
                                          int32_t* n_active);

/* Where table `order` (derivative order k; 0 for d-linear) of level `level` lives in the
 * flat parameter (and gradient) buffer: float offset, rows, floats per row (C(d,k) * F) and
 * whether it is a dense 1:1 grid.  Host outputs, each may be NULL. */
HASHENC_API int hashenc_param_layout(const hashenc* h, int32_t order, int32_t level, int64_t* offset,
                         int64_t* rows, int32_t* row_width, int32_t* is_dense);

/* Forward encoding of n points: per level the cell around x, the lookup of its corners and
 * the interpolant, concatenated over levels (Instant-NGP explainer, encoding pipeline steps
 * 1-4; Hermite kind: Hermite-NGP notes, key design 1 for the value and key design 2 for the
 * analytic first and second derivatives; RBF kind: DInf-Grid summary, section
 * 可微的径向基函数插值).
 *   x       [n, d] fp32, row-major
 *   params  [n_params] fp32 in the layout above
 *   gamma   [n, L*F]  level-major then feature (may be NULL)
 *   dgamma  Hermite and RBF: [n, d, L*F] spatial gradient (may be NULL; must be NULL for
 *           d-linear)
 *   d2gamma Hermite and RBF: Laplacian [n, L*F] or diagonal [n, d, L*F] per cfg.d2_mode
 *           (may be NULL; must be NULL for d-linear)
 * Outputs are overwritten.  n == 0 is a no-op. */
HASHENC_API int hashenc_forward(const hashenc* h, int64_t n, const float* x, const float* params,
                    float* gamma, float* dgamma, float* d2gamma, hashenc_stream_t stream);

/* Device workspace (bytes) that hashenc_forward_ws needs for n points (0: none used). */
HASHENC_API int hashenc_forward_workspace_size(const hashenc* h, int64_t n, size_t* bytes);

/* Same outputs as hashenc_forward.  With a workspace the d-linear encoding is computed
 * level by level into a level-major staging buffer [L][n][F] (every store writes whole
 * cache lines) and then rearranged into gamma [n, L*F] in one pass.  A Hermite handle with
 * d = 2 or 3 also stages its outputs level-major ([L][n][M][F], M = 1 + d + (d or 1)) and,
 * when every order table has the order-0 table's size or is a power of two no larger than it,
 * first packs the tables into the workspace (one contiguous row of every order table per
 * vertex) and reads the corners from that copy.  A d = 4 Hermite handle with F <= 2 and such
 * table sizes packs its five tables the same way (16 F floats per vertex) and writes its
 * outputs directly; with F > 2 it needs no workspace.  An RBF handle needs no workspace (size
 * 0) and runs as hashenc_forward.  2D and 3D Hermite batches of fewer than 32768 points run
 * as hashenc_forward (the workspace is then not touched): for them the pass over every order
 * table that the packing costs outweighs the faster gather.
 * workspace: >= hashenc_forward_workspace_size bytes, 256-byte aligned; calls sharing it
 * must not overlap.  Results are bit-identical to hashenc_forward. */
HASHENC_API int hashenc_forward_ws(const hashenc* h, int64_t n, const float* x, const float* params,
                                   float* gamma, float* dgamma, float* d2gamma, void* workspace,
                                   size_t workspace_bytes, hashenc_stream_t stream);

/* Backward: grad_params += d<G, forward(theta)>/d theta for the upstream gradients G
 * (shapes as the forward outputs; NULL = zero): the transpose of the forward's interpolation
 * (same passages as hashenc_forward).  Contributions of colliding vertices sum (Instant-NGP
 * news article, adaptivity paragraph: gradients of colliding points combine).
 * Accumulated with fp32 atomics: the summation order, and so the last bits, vary from
 * run to run.  The caller zeroes grad_params when it wants a fresh gradient. */
HASHENC_API int hashenc_backward(const hashenc* h, int64_t n, const float* x, const float* g_gamma,
                     const float* g_dgamma, const float* g_d2gamma, float* grad_params,
                     hashenc_stream_t stream);

/* Device workspace (bytes) that hashenc_backward_ws needs for n points (0 when this handle's
 * configuration, or a d-linear batch with n * L < 2^18, does not use one;
 * hashenc_backward_ws then takes the atomic path).  Configurations without a binned plan:
 * the RBF kind, order-table rows wider than 24 floats (d = 4 with F = 8), and grids whose
 * bins or LDS staging exceed the workgroup budgets.  A workspace sized for n points serves
 * every smaller n. */
HASHENC_API int hashenc_backward_workspace_size(const hashenc* h, int64_t n, size_t* bytes);

/* Same result as hashenc_backward (grad_params += dL/dtheta), computed without global
 * atomics on the hot part: the contributions are counted and sorted into bins of rows
 * small enough for the LDS of one workgroup, then each bin is accumulated on chip and added
 * to grad_params.  workspace: >= hashenc_backward_workspace_size bytes, 256-byte aligned,
 * owned by the caller, contents irrelevant on entry; calls sharing a workspace must not
 * overlap.  Points are processed in chunks of 2^21 (fewer when a chunk would hold 2^31
 * entries).  Small d-linear batches (n * L < 2^18) take the atomic path, which is faster
 * there. */
HASHENC_API int hashenc_backward_ws(const hashenc* h, int64_t n, const float* x, const float* g_gamma,
                                    const float* g_dgamma, const float* g_d2gamma, float* grad_params,
                                    void* workspace, size_t workspace_bytes, hashenc_stream_t stream);

/* Training pair for the d-linear kind: a forward that also prepares the binned backward of
 * the same points, and that backward.  The forward of one point and level already computes
 * the corner rows of its cell (Instant-NGP explainer, encoding pipeline steps 1-2); the
 * binned backward's first pass (a per-tile histogram of those rows over the bins of rows that
 * one workgroup accumulates) needs exactly these rows, so hashenc_forward_counting writes the
 * histogram into bwd_workspace while it gathers, and hashenc_backward_counted starts from it.
 *
 * hashenc_forward_counting: outputs and workspace as hashenc_forward_ws (bit-identical
 *   results); bwd_workspace: >= hashenc_backward_workspace_size(h, n) bytes, 256-byte aligned,
 *   caller-owned, contents irrelevant on entry, not overlapping workspace; it is written.
 * hashenc_backward_counted: result and arguments as hashenc_backward_ws (grad_params +=
 *   dL/dtheta, the same passages), with bwd_workspace the one the counting forward wrote.
 * Contract: between the two calls x, n and bwd_workspace stay the same and nothing else
 * writes the workspace.  Broken, the gradient is undefined but every write stays inside
 * bwd_workspace and grad_params (the backward's stores are bounds-guarded).
 * Where the counts would not apply -- other kinds, batches that take the atomic path or more
 * than one 2^21-point chunk, forward passes with more than 512 bins -- the two calls behave
 * exactly as hashenc_forward_ws and hashenc_backward_ws (the forward then leaves bwd_workspace
 * untouched); both decide from (h, n) alone. */
HASHENC_API int hashenc_forward_counting(const hashenc* h, int64_t n, const float* x, const float* params,
                                         float* gamma, float* dgamma, float* d2gamma, void* workspace,
                                         size_t workspace_bytes, void* bwd_workspace, size_t bwd_workspace_bytes,
                                         hashenc_stream_t stream);
HASHENC_API int hashenc_backward_counted(const hashenc* h, int64_t n, const float* x, const float* g_gamma,
                                         const float* g_dgamma, const float* g_d2gamma, float* grad_params,
                                         void* bwd_workspace, size_t bwd_workspace_bytes, hashenc_stream_t stream);

/* Allocation-free variant of hashenc_backward_ws, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  Same arguments as hashenc_backward (all device pointers owned by the caller)
 * and the same result as hashenc_backward_ws: grad_params += dL/dtheta.  In place of a
 * workspace argument it uses a file-scope static device array of
 * HASHENC_NOALLOC_SCRATCH_BYTES, which every GPU the library runs on holds from the first
 * call on that GPU until the process ends; points run in chunks small enough for the binned
 * backward's workspace to fit it (the chunk size depends on the configuration; more chunks
 * cost more passes over the gradient).  Configurations the binned path does not cover take
 * the atomic path, as hashenc_backward_ws does.  Nothing is allocated: no hipMalloc,
 * hipFree or allocating library routine is called.  No part of the scratch needs to start
 * at zero, and each call leaves its last chunk's plan in it.  All calls on one GPU share
 * that GPU's array: calls that overlap on one GPU (different streams or threads) race and
 * give wrong results; the caller serialises them.  HASHENC_EINVAL (before any launch) when
 * even a 1024-point chunk of this configuration needs more scratch than the array holds. */
#define HASHENC_NOALLOC_SCRATCH_BYTES ((size_t)256 << 20)
HASHENC_API int hashenc_backward_noalloc(const hashenc* h, int64_t n, const float* x, const float* g_gamma,
                                         const float* g_dgamma, const float* g_d2gamma, float* grad_params,
                                         hashenc_stream_t stream);

/* SIREN decoder of the fused PINN residual (Hermite-NGP key design 2; loss section):
 * `depth` hidden layers of width `hidden`, activation sin(omega (W v + b)), then a linear
 * output of width 1.  `in` must equal L*F. */
typedef struct hashenc_mlp {
  int32_t in;
  int32_t hidden;  /* 16, 32 or 64 */
  int32_t depth;   /* 1..4 */
  int32_t out;     /* must be 1 */
  float omega;     /* e.g. 30 */
  int32_t reserved;/* must be 0 */
} hashenc_mlp;

/* Device workspace (bytes) hashenc_residual needs for n points. */
HASHENC_API int hashenc_residual_workspace_size(const hashenc* h, const hashenc_mlp* mlp, int64_t n,
                                    size_t* bytes);

/* One fused PINN residual step for the Poisson problem Lap u = g with the manufactured
 * source g(x) = -d pi^2 prod_i sin(pi x_i), on a Hermite handle:
 *   encode (gamma, grad gamma, Lap gamma) -> SIREN in forward mode (u, grad u, Lap u) ->
 *   r = Lap u - g -> loss = mean r^2 -> reverse sweep -> encoder backward.
 *   mlp_params  packed W1[hidden][in], b1, (Wk[hidden][hidden], bk)..., Wo[1][hidden], bo
 *   residual    [n] r (may be NULL)
 *   loss        [1] mean r^2 (overwritten)
 *   grad_params += dloss/dtheta;  grad_mlp += dloss/dmlp_params (same packing)
 *   workspace   >= hashenc_residual_workspace_size bytes, 256-byte aligned
 * n must be >= 1. */
HASHENC_API int hashenc_residual(const hashenc* h, const hashenc_mlp* mlp, int64_t n, const float* x,
                     const float* params, const float* mlp_params, float* residual,
                     float* loss, float* grad_params, float* grad_mlp, void* workspace,
                     size_t workspace_bytes, hashenc_stream_t stream);

/* INGP-FD comparator (Hermite-NGP reading notes, the 现有痛点 paragraph and key design 2's
 * comparison: Instant-NGP + central finite differences needs 2d+1 forward passes per
 * Laplacian).  The same Poisson residual step as hashenc_residual, on a d-LINEAR handle: each
 * point's 2d+1 stencil points x, x + eps e_i, x - eps e_i (s = 0, 2i+1, 2i+2; the shifted
 * coordinate is one fp32 addition, then the encoder's usual clamp) are encoded and pushed
 * through the SIREN (value only: a = sin(omega (W v + b)), u = Wo a + bo), and
 *   Lap u = sum_i (u(x + eps e_i) - 2 u(x) + u(x - eps e_i)) / eps^2,  r = Lap u - g(x),
 *   loss = mean r^2, with g as for hashenc_residual; the reverse sweep runs through all
 *   2d+1 stencil points' networks and encodings.  The output bias cancels in the stencil:
 *   its gradient is zero.
 *   mlp          depth 1..4 (1 and 2 on the matrix cores, 3 and 4 on the vector ALUs),
 *                hidden <= 64, in == L*F <= 64
 *   eps          FD step (> 0, finite)
 *   u_stencil    [n, 2d+1] u at the stencil points (may be NULL)
 *   residual     [n] r (may be NULL);  loss [1] (overwritten)
 *   grad_params  += dloss/dtheta;  grad_mlp += dloss/dmlp_params (either may be NULL)
 *   workspace    >= hashenc_fd_residual_workspace_size bytes, 256-byte aligned
 * HASHENC_EUNSUPPORTED for a Hermite handle or depth > 4.  n must be >= 1. */
HASHENC_API int hashenc_fd_residual_workspace_size(const hashenc* h, const hashenc_mlp* mlp, int64_t n,
                                                   size_t* bytes);
HASHENC_API int hashenc_fd_residual(const hashenc* h, const hashenc_mlp* mlp, float eps, int64_t n,
                                    const float* x, const float* params, const float* mlp_params,
                                    float* u_stencil, float* residual, float* loss, float* grad_params,
                                    float* grad_mlp, void* workspace, size_t workspace_bytes,
                                    hashenc_stream_t stream);

/* Message for the last non-zero return on this thread ("" if none). */
HASHENC_API const char* hashenc_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* HASHENC_H */
