// Library-private declarations shared by the host code and the kernels: the per-handle
// grid description passed to kernels by value, device helpers for the lookup stage, and
// the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "hashenc.h"

namespace hg {

constexpr int kMaxLevels = HASHENC_MAX_LEVELS;
constexpr int kMaxTables = 5;  // order tables: d + 1 for Hermite, up to d = 4
constexpr int kBlock = 256;

// The spatial-hash primes, one per axis; the first is 1 so the x axis maps to itself.
constexpr uint32_t kPrime1 = 2654435761u;
constexpr uint32_t kPrime2 = 805459861u;

// Everything a kernel needs to find a (table, level) block and the rows of a cell.
// Passed by value as a kernel argument (about 1.3 KB, well inside the kernarg limit);
// kernels index it only with wave-uniform level numbers, so it stays in scalar loads.
// L counts the levels the kernels compute; Lrow the levels of an encoding row (the
// configured level count).  L < Lrow under coarse-to-fine activation: levels l >= L are
// inactive, their columns of every output row are zero and their blocks get no gradient.
struct Grid {
  int32_t L;
  int32_t Lrow;
  int32_t n_tables;
  int32_t N[kMaxLevels];        // resolution N_l
  float Nf[kMaxLevels];         // N_l as fp32 (exact: N_l <= 2^20)
  float invN[kMaxLevels];       // fl32(1 / N_l) = Delta x_l
  uint32_t T[kMaxTables];       // rows of a hashed block of table k
  uint32_t Tmask[kMaxTables];   // T - 1 when T is a power of two > 1, else 0
  uint32_t dense[kMaxTables];   // bit l set: level l of table k is a dense 1:1 grid
  int64_t off[kMaxTables][kMaxLevels];  // float offset of block (k, l) in params / grads
  float rbf_e2;                 // Gaussian RBF: eps^2
  int32_t rings;                // Gaussian RBF: neighbourhood rings k
};

// v plus the value of the neighbouring lane (lane ^ 1): a DPP quad permutation [1, 0, 3, 2],
// one VALU operation instead of an LDS permute round trip.  Both lanes of the pair must be
// active.
__device__ __forceinline__ float add_lane_pair(float v) {
  return v + __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xf, 0xf, false));
}

// One rounded fp32 product, never fused into a neighbouring add: the cell a point falls in
// must not depend on the compiler's contraction choices.
__device__ __forceinline__ float mul_rn(float a, float b) {
#pragma clang fp contract(off)
  return a * b;
}

// Cell of point x at a level: base vertex and local coordinate t in [0, 1].
template <int D>
__device__ __forceinline__ void locate(const float (&x)[D], int32_t N, float Nf,
                                       uint32_t (&base)[D], float (&t)[D]) {
#pragma unroll
  for (int i = 0; i < D; ++i) {
    const float xi = fminf(fmaxf(x[i], 0.0f), 1.0f);  // clamp; NaN -> 0
    const float p = mul_rn(xi, Nf);
    const int32_t b = min((int32_t)floorf(p), N - 1);
    base[i] = (uint32_t)b;
    t[i] = p - (float)b;  // exact
  }
}

// Per-axis ingredients of the corner rows of one cell, from which the row of any corner
// c (bit i = +1 along axis i) of any table follows with a few integer ops.
template <int D>
struct CellKeys {
  uint32_t dense0;        // dense row of corner 0
  uint32_t stride[D];     // (N+1)^i
  uint32_t hx[2], hy[2], hz[2];  // per-axis hash terms of the two vertex coordinates
};

template <int D>
__device__ __forceinline__ CellKeys<D> cell_keys(const uint32_t (&base)[D], int32_t N) {
  CellKeys<D> k;
  const uint32_t N1 = (uint32_t)N + 1u;
  k.stride[0] = 1u;
  if (D > 1) k.stride[1] = N1;
  if (D > 2) k.stride[2] = N1 * N1;
  uint32_t d0 = base[0];
  if (D > 1) d0 += base[1] * N1;
  if (D > 2) d0 += base[2] * N1 * N1;
  k.dense0 = d0;
  k.hx[0] = base[0];
  k.hx[1] = base[0] + 1u;
  k.hy[0] = k.hy[1] = k.hz[0] = k.hz[1] = 0u;
  if (D > 1) { k.hy[0] = base[1] * kPrime1; k.hy[1] = k.hy[0] + kPrime1; }
  if (D > 2) { k.hz[0] = base[2] * kPrime2; k.hz[1] = k.hz[0] + kPrime2; }
  return k;
}

// Row of corner C in a table whose block at this level is dense (1:1) or hashed.
template <int D, int C>
__device__ __forceinline__ uint32_t corner_row(const CellKeys<D>& k, bool dense, uint32_t T,
                                               uint32_t Tmask) {
  if (dense) {
    uint32_t r = k.dense0;
#pragma unroll
    for (int i = 0; i < D; ++i)
      if ((C >> i) & 1) r += k.stride[i];
    return r;
  }
  uint32_t h = k.hx[C & 1];
  if (D > 1) h ^= k.hy[(C >> 1) & 1];
  if (D > 2) h ^= k.hz[(C >> 2) & 1];
  return Tmask ? (h & Tmask) : (h % T);
}

// Same, with a run-time corner number (used by the index export only).
template <int D>
__device__ __forceinline__ uint32_t corner_row_rt(const CellKeys<D>& k, int c, bool dense,
                                                  uint32_t T, uint32_t Tmask) {
  if (dense) {
    uint32_t r = k.dense0;
    for (int i = 0; i < D; ++i)
      if ((c >> i) & 1) r += k.stride[i];
    return r;
  }
  uint32_t h = k.hx[c & 1];
  if (D > 1) h ^= k.hy[(c >> 1) & 1];
  if (D > 2) h ^= k.hz[(c >> 2) & 1];
  return Tmask ? (h & Tmask) : (h % T);
}

// Unreturned fp32 atomic add at device scope (hardware float atomic, no CAS loop).
__device__ __forceinline__ void atomic_add_f32(float* p, float v) {
  __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------- launchers
// All launchers assume validated arguments (host side) and n >= 1.
// scratch: NULL, or dlinear_forward_workspace_bytes for the level-major staging of the output
// ([L][n][F], active levels); with scratch and gamma NULL the output stays level-major there.
size_t dlinear_forward_workspace_bytes(const Grid& g, int d, int F, int64_t n);
hipError_t launch_dlinear_forward(const Grid& g, int d, int F, int64_t n, const float* x,
                                  const float* params, float* gamma, float* scratch, hipStream_t s);
// u_levels: NULL, or the upstream level-major ([L][n][F], active levels) instead of g_gamma
hipError_t launch_dlinear_backward(const Grid& g, int d, int F, int64_t n, const float* x,
                                   const float* g_gamma, const float* u_levels, float* grad, hipStream_t s);
// Hermite tables of equal size: the packed copy (one contiguous row of all order tables per
// vertex) that the forward can read instead of the tables; 0 bytes when not packable.
bool hermite_packable(const Grid& g, int d);
size_t hermite_packed_bytes(const Grid& g, int d, int F);
hipError_t launch_hermite_pack(const Grid& g, int d, int F, const float* params, float* packed, hipStream_t s);
// Smallest batch for which a 2D or 3D call packs the tables: below it the pack's fixed cost
// (a pass over every order table) exceeds the packed gather's saving.
constexpr int64_t kPackMinPoints = int64_t(1) << 15;
// Level-major output staging of the Hermite forward: [L][n][M][F] floats, M = 1 + d + (d or 1).
size_t hermite_stage_bytes(const Grid& g, int d, int F, int d2_mode, int64_t n);
// packed: NULL to read params directly, else the packed copy of params.  stage: NULL to write
// the point-major outputs directly; else the outputs go level-major into stage and, when
// to_rows, are then rearranged into gamma / dgamma / d2gamma.
hipError_t launch_hermite_forward(const Grid& g, int d, int F, int d2_mode, int64_t n,
                                  const float* x, const float* params, const float* packed, float* stage,
                                  bool to_rows, float* gamma, float* dgamma, float* d2gamma, hipStream_t s);
// u_levels: NULL, or the upstream level-major ([L][n][M][F]) in place of the three arrays
hipError_t launch_hermite_backward(const Grid& g, int d, int F, int d2_mode, int64_t n,
                                   const float* x, const float* g_gamma, const float* g_dgamma,
                                   const float* g_d2gamma, const float* u_levels, float* grad, hipStream_t s);
// Space-time Hermite (d = 4: five order tables, 16 coefficients per vertex).  packed: NULL to
// read the tables, else room for the packed copy (hermite4_packed_bytes, nonzero for F <= 2 and
// packable table sizes), which the forward writes and then reads.
size_t hermite4_packed_bytes(const Grid& g, int F);
hipError_t launch_hermite4_forward(const Grid& g, int F, int d2_mode, int64_t n, const float* x,
                                   const float* params, float* packed, float* gamma, float* dgamma, float* d2gamma,
                                   hipStream_t s);
hipError_t launch_hermite4_backward(const Grid& g, int F, int d2_mode, int64_t n, const float* x,
                                    const float* g_gamma, const float* g_dgamma, const float* g_d2gamma,
                                    float* grad, hipStream_t s);
hipError_t launch_debug_indices4(const Grid& g, int order, int64_t n, const float* x, int32_t* out, hipStream_t s);
// Gaussian RBF (one table per level, derivative outputs as the Hermite ones; fp32-atomic backward)
hipError_t launch_rbf_forward(const Grid& g, int d, int F, int d2_mode, int64_t n, const float* x,
                              const float* params, float* gamma, float* dgamma, float* d2gamma, hipStream_t s);
hipError_t launch_rbf_backward(const Grid& g, int d, int F, int d2_mode, int64_t n, const float* x,
                               const float* g_gamma, const float* g_dgamma, const float* g_d2gamma, float* grad,
                               hipStream_t s);
hipError_t launch_debug_indices(const Grid& g, int d, int order, int64_t n, const float* x,
                                int32_t* out, hipStream_t s);
hipError_t launch_copy(const float* src, float* dst, int64_t n, hipStream_t s);
// n must be a multiple of cache_read_granule() floats
int64_t cache_read_granule();
hipError_t launch_cache_read(const float* buf, int64_t n, int32_t reps, float* out, hipStream_t s);
// Zero columns [from, row_floats) of rows rows x row_floats floats (inactive levels).
hipError_t launch_zero_columns(float* out, int64_t rows, int32_t row_floats, int32_t from, hipStream_t s);

// Fused PINN residual (Hermite handle): workspace size and the full step.
int64_t mlp_param_count(int in, int H, int depth);
// INGP-FD comparator (d-linear handle, SIREN depth 1..2): workspace size and the full step.
size_t fd_residual_workspace_bytes(const Grid& g, int d, int F, int64_t n, int in, int H, int depth, bool binned);
hipError_t run_fd_residual(const Grid& g, int d, int F, int64_t n, const float* x, const float* params, int in,
                           int H, int depth, float omega, float eps, const float* mlp, float* u_stencil,
                           float* residual, float* loss, float* grad_params, float* grad_mlp, void* workspace,
                           bool binned, hipStream_t s);
size_t residual_workspace_bytes(const Grid& g, int d, int F, int64_t n, int in, int H, int depth,
                                bool binned);
hipError_t run_residual(const Grid& g, int d, int F, int64_t n, const float* x, const float* params,
                        int in, int H, int depth, float omega, const float* mlp, float* residual,
                        float* loss, float* grad_params, float* grad_mlp, void* workspace,
                        bool binned, hipStream_t s);

}  // namespace hg
