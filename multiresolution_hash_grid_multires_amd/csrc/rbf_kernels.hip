// Gaussian-RBF multi-resolution grid (DInf-Grid), forward and backward, gfx950.
//
// Method: DInf-Grid summary (shdxiang-github-io), section 可微的径向基函数插值: the feature
// at x is a normalised Gaussian-weighted sum of the vertex features of a precomputed k-ring
// neighbourhood, w_v = phi(|p - v|) / sum_u phi(|p - u|), phi(r) = exp(-(eps r)^2), which is
// infinitely differentiable; section 多分辨率特征网格: the levels are concatenated.  Distances
// are in units of the level's grid spacing (p = x N_l); the neighbourhood of a point is the
// (2k)^d vertex box around its cell, clipped to the grid.
//
// Mapping: one lane per (point, level), workgroups ordered level-major as the other
// forwards.  The Gaussian factorises over axes, and the box is a product of per-axis ranges,
// so every sum is evaluated axis by axis: per-axis factors g, dg/dx, d2g/dx2 (x-space, the
// chain-rule factors N_l and N_l^2 folded in), the normaliser S = prod_i S_i, and the
// weighted sums of the vertex features accumulated along x inside a row, then over y, then
// over z.  The x-runs of a box row are contiguous rows of a dense level.  The quotient rule
// turns the sums into gamma, d gamma/dx_i and d^2 gamma/dx_i^2.  The backward distributes the
// upstream through the same factors (no vertex-dependent division), pre-aggregates a
// workgroup's contributions in LDS where its points' neighbourhoods fit, and adds them to the
// table with fp32 atomics.
#include "hashenc_internal.h"
#include "vec_io.h"

namespace hg {
namespace {

constexpr int kMaxSide = 8;  // 2k for k <= 4

// Factors of one axis at box position m (vertex base - k + 1 + m): value, x-derivative,
// second x-derivative of exp(-eps^2 (p - v)^2); zero outside the grid.  Every factor is
// scaled by exp(eps^2 m0^2), m0 = min(t, 1 - t) the distance to the nearest vertex along the
// axis (base or base + 1, both always inside the grid): the weights are ratios to the sum,
// so the scale cancels, and the largest factor is exactly 1 (no fp32 underflow of the sum
// for sharp kernels).
struct AxisG {
  float g, g1, g2;
};

__device__ __forceinline__ AxisG rbf_axis(float t, int32_t base, int k, int m, int32_t N, float e2, float Nf) {
  AxisG a;
  const int32_t v = base - k + 1 + m;
  const float del = t + (float)(k - 1 - m);  // p - v, exact
  const float m0 = fminf(t, 1.0f - t);
  const bool in = v >= 0 && v <= N;
  const float e = in ? expf(-e2 * (del * del - m0 * m0)) : 0.0f;
  a.g = e;
  a.g1 = -2.0f * e2 * del * e * Nf;
  a.g2 = (4.0f * e2 * e2 * del * del - 2.0f * e2) * e * (Nf * Nf);
  return a;
}

struct AxisSums {
  float S, S1, S2;
};

__device__ __forceinline__ AxisSums rbf_axis_sums(float t, int32_t base, int k, int32_t N, float e2, float Nf) {
  AxisSums s{0.0f, 0.0f, 0.0f};
  for (int m = 0; m < 2 * k; ++m) {
    const AxisG a = rbf_axis(t, base, k, m, N, e2, Nf);
    s.S += a.g;
    s.S1 += a.g1;
    s.S2 += a.g2;
  }
  return s;
}

// Everything of one point at one level that does not depend on the features.
template <int D>
struct RbfSetup {
  uint32_t base[D];
  float t[D];
  AxisSums ax[D];
  float S;           // prod of the axis sums
  float dS[D];       // d S / dx_i
  float d2S[D];      // d^2 S / dx_i^2
};

template <int D>
__device__ __forceinline__ void rbf_setup(const Grid& g, int l, const float (&xp)[D], RbfSetup<D>& s) {
  locate<D>(xp, g.N[l], g.Nf[l], s.base, s.t);
#pragma unroll
  for (int i = 0; i < D; ++i) s.ax[i] = rbf_axis_sums(s.t[i], (int32_t)s.base[i], g.rings, g.N[l], g.rbf_e2, g.Nf[l]);
  s.S = 1.0f;
#pragma unroll
  for (int i = 0; i < D; ++i) s.S *= s.ax[i].S;
#pragma unroll
  for (int i = 0; i < D; ++i) {
    float others = 1.0f;
#pragma unroll
    for (int j = 0; j < D; ++j)
      if (j != i) others *= s.ax[j].S;
    s.dS[i] = s.ax[i].S1 * others;
    s.d2S[i] = s.ax[i].S2 * others;
  }
}

// Row of vertex (vx, row key) on a dense or hashed level: dense key = (N+1)(vy + (N+1) vz),
// hashed key = vy * pi_1 ^ vz * pi_2.
__device__ __forceinline__ uint32_t rbf_row(uint32_t vx, uint32_t key, bool dense, uint32_t T, uint32_t Tmask) {
  if (dense) return key + vx;
  const uint32_t h = vx ^ key;
  return Tmask ? (h & Tmask) : (h % T);
}

__device__ __forceinline__ uint32_t rbf_key(uint32_t vy, uint32_t vz, int32_t N, bool dense) {
  const uint32_t N1 = (uint32_t)N + 1u;
  return dense ? N1 * (vy + N1 * vz) : (vy * kPrime1) ^ (vz * kPrime2);
}

// Forward.  Sums over the box: A (value), A_i (first x_i-derivative factor on axis i), A_ii
// (second); then gamma = A / S, d_i gamma = (A_i - gamma d_i S) / S,
// d_ii gamma = (A_ii - 2 d_i gamma d_i S - gamma d_ii S) / S.
template <int D, int F>
__global__ __launch_bounds__(kBlock) void rbf_forward_kernel(const Grid g, int64_t n, int32_t n_tiles, int d2_mode,
                                                             const float* __restrict__ x,
                                                             const float* __restrict__ params,
                                                             float* __restrict__ gamma, float* __restrict__ dgamma,
                                                             float* __restrict__ d2gamma) {
  const int l = blockIdx.x / n_tiles;
  const int64_t p = (int64_t)(blockIdx.x % n_tiles) * kBlock + threadIdx.x;
  if (p >= n) return;
  float xp[D];
#pragma unroll
  for (int i = 0; i < D; ++i) xp[i] = x[p * D + i];
  RbfSetup<D> s;
  rbf_setup<D>(g, l, xp, s);
  const int k = g.rings, side = 2 * k;
  const int32_t N = g.N[l];
  const float e2 = g.rbf_e2, Nf = g.Nf[l];
  const bool dense = (g.dense[0] >> l) & 1u;
  const float* tab = params + g.off[0][l];
  AxisG gx[kMaxSide];
#pragma unroll
  for (int m = 0; m < kMaxSide; ++m)
    gx[m] = m < side ? rbf_axis(s.t[0], (int32_t)s.base[0], k, m, N, e2, Nf) : AxisG{0.0f, 0.0f, 0.0f};
  // A[0] value, A[1 + i] first derivative along i, A[1 + D + i] second derivative along i
  float A[1 + 2 * D][F];
#pragma unroll
  for (int c = 0; c < 1 + 2 * D; ++c)
#pragma unroll
    for (int f = 0; f < F; ++f) A[c][f] = 0.0f;
  const int zs = D > 2 ? side : 1;
  for (int mz = 0; mz < zs; ++mz) {
    AxisG gz{1.0f, 0.0f, 0.0f};
    uint32_t vz = 0;
    if constexpr (D > 2) {
      gz = rbf_axis(s.t[2], (int32_t)s.base[2], k, mz, N, e2, Nf);
      if (gz.g == 0.0f) continue;  // outside the grid
      vz = s.base[2] - k + 1 + mz;
    }
    // sums over y (and x) of this z-slab: Y[0] value, Y[1] d/dx, Y[2] d2/dx2, Y[3] d/dy, Y[4] d2/dy2
    float Y[5][F];
#pragma unroll
    for (int c = 0; c < 5; ++c)
#pragma unroll
      for (int f = 0; f < F; ++f) Y[c][f] = 0.0f;
    for (int my = 0; my < side; ++my) {
      const AxisG gy = rbf_axis(s.t[1], (int32_t)s.base[1], k, my, N, e2, Nf);
      if (gy.g == 0.0f) continue;
      const uint32_t vy = s.base[1] - k + 1 + my;
      const uint32_t key = rbf_key(vy, vz, N, dense);
      float vals[kMaxSide][F];
#pragma unroll
      for (int m = 0; m < kMaxSide; ++m) {
        if (m < side && gx[m].g != 0.0f) {
          const uint32_t row = rbf_row(s.base[0] - k + 1 + m, key, dense, g.T[0], g.Tmask[0]);
          load_vec<F>(tab + (size_t)row * F, vals[m]);
        } else {
#pragma unroll
          for (int f = 0; f < F; ++f) vals[m][f] = 0.0f;
        }
      }
      float R0[F], R1[F], R2[F];
#pragma unroll
      for (int f = 0; f < F; ++f) R0[f] = R1[f] = R2[f] = 0.0f;
#pragma unroll
      for (int m = 0; m < kMaxSide; ++m)
#pragma unroll
        for (int f = 0; f < F; ++f) {
          R0[f] = fmaf(gx[m].g, vals[m][f], R0[f]);
          R1[f] = fmaf(gx[m].g1, vals[m][f], R1[f]);
          R2[f] = fmaf(gx[m].g2, vals[m][f], R2[f]);
        }
#pragma unroll
      for (int f = 0; f < F; ++f) {
        Y[0][f] = fmaf(gy.g, R0[f], Y[0][f]);
        Y[1][f] = fmaf(gy.g, R1[f], Y[1][f]);
        Y[2][f] = fmaf(gy.g, R2[f], Y[2][f]);
        Y[3][f] = fmaf(gy.g1, R0[f], Y[3][f]);
        Y[4][f] = fmaf(gy.g2, R0[f], Y[4][f]);
      }
    }
#pragma unroll
    for (int f = 0; f < F; ++f) {
      A[0][f] = fmaf(gz.g, Y[0][f], A[0][f]);
      A[1][f] = fmaf(gz.g, Y[1][f], A[1][f]);          // d/dx
      A[2][f] = fmaf(gz.g, Y[3][f], A[2][f]);          // d/dy
      A[1 + D][f] = fmaf(gz.g, Y[2][f], A[1 + D][f]);  // d2/dx2
      A[2 + D][f] = fmaf(gz.g, Y[4][f], A[2 + D][f]);  // d2/dy2
      if constexpr (D > 2) {
        A[3][f] = fmaf(gz.g1, Y[0][f], A[3][f]);          // d/dz
        A[3 + D][f] = fmaf(gz.g2, Y[0][f], A[3 + D][f]);  // d2/dz2
      }
    }
  }
  const float inv = 1.0f / s.S;
  float v0[F], v1[D][F], v2[D][F];
#pragma unroll
  for (int f = 0; f < F; ++f) {
    v0[f] = A[0][f] * inv;
#pragma unroll
    for (int i = 0; i < D; ++i) {
      v1[i][f] = (A[1 + i][f] - v0[f] * s.dS[i]) * inv;
      v2[i][f] = (A[1 + D + i][f] - 2.0f * v1[i][f] * s.dS[i] - v0[f] * s.d2S[i]) * inv;
    }
  }
  const int64_t LF = (int64_t)g.Lrow * F;
  const int64_t col = (int64_t)l * F;
  if (gamma) store_vec<F>(gamma + p * LF + col, v0);
  if (dgamma) {
#pragma unroll
    for (int i = 0; i < D; ++i) store_vec<F>(dgamma + (p * D + i) * LF + col, v1[i]);
  }
  if (d2gamma) {
    if (d2_mode == HASHENC_D2_DIAG) {
#pragma unroll
      for (int i = 0; i < D; ++i) store_vec<F>(d2gamma + (p * D + i) * LF + col, v2[i]);
    } else {
      float lap[F];
#pragma unroll
      for (int f = 0; f < F; ++f) {
        float sum = 0.0f;
#pragma unroll
        for (int i = 0; i < D; ++i) sum += v2[i][f];
        lap[f] = sum;
      }
      store_vec<F>(d2gamma + p * LF + col, lap);
    }
  }
}

// Backward.  With G0, G1_i, G2_i the upstream of gamma, d_i gamma, d_ii gamma at this level,
// vertex v receives
//   phi_v a + sum_i dphi_v/dx_i b_i + sum_i d2phi_v/dx_i^2 c_i,
//   a = G0/S - sum_i (dS_i G1_i + d2S_i G2_i)/S^2 + 2 sum_i dS_i^2 G2_i / S^3,
//   b_i = G1_i/S - 2 dS_i G2_i / S^2,   c_i = G2_i / S,
// the transpose of the forward's quotient rule, with the per-axis factors of phi.
//
// A workgroup owns kRbfBwdBlock consecutive points at one level.  Neighbouring points share
// most of their box vertices, so the workgroup first takes the bounding box of its points'
// boxes; when that fits kRbfLdsValues it accumulates there with LDS atomics and then adds every
// touched vertex to the table once (one global atomic per vertex feature instead of one per
// point, vertex and feature); otherwise every contribution goes straight to the table.  The
// accumulator is fp64: on gfx950 LDS fp64 adds run several times faster than fp32 ones
// (measured 1.57 T against 0.20 T lane operations per second at random addresses), and the
// box sums stay exact far below the fp32 result.  96 KB leaves one 512-lane workgroup per CU.
constexpr int kRbfLdsValues = 12288;  // 96 KB of fp64
constexpr int kRbfBwdBlock = 512;

template <int D, int F>
__global__ __launch_bounds__(kRbfBwdBlock) void rbf_backward_kernel(const Grid g, int64_t n, int32_t n_tiles, int d2_mode,
                                                              const float* __restrict__ x,
                                                              const float* __restrict__ g_gamma,
                                                              const float* __restrict__ g_dgamma,
                                                              const float* __restrict__ g_d2gamma,
                                                              float* __restrict__ grad) {
  __shared__ double acc[kRbfLdsValues];
  __shared__ int32_t bounds[2 * D][kRbfBwdBlock / 64];
  const int l = blockIdx.x / n_tiles;
  const int64_t p = (int64_t)(blockIdx.x % n_tiles) * kRbfBwdBlock + threadIdx.x;
  const bool on = p < n;
  const int k = g.rings, side = 2 * k;
  const int32_t N = g.N[l];
  float xp[D];
#pragma unroll
  for (int i = 0; i < D; ++i) xp[i] = on ? x[p * D + i] : 0.0f;
  RbfSetup<D> s;
  rbf_setup<D>(g, l, xp, s);

  // bounding box of the workgroup's k-ring boxes (clipped to the grid)
  int32_t lo[D], ext[D];
  {
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
#pragma unroll
    for (int i = 0; i < D; ++i) {
      int32_t mn = on ? (int32_t)s.base[i] : INT32_MAX, mx = on ? (int32_t)s.base[i] : INT32_MIN;
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) {
        mn = min(mn, __shfl_xor(mn, off, 64));
        mx = max(mx, __shfl_xor(mx, off, 64));
      }
      if (lane == 0) { bounds[2 * i][wv] = mn; bounds[2 * i + 1][wv] = mx; }
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < D; ++i) {
      int32_t mn = bounds[2 * i][0], mx = bounds[2 * i + 1][0];
      for (int w = 1; w < kRbfBwdBlock / 64; ++w) {
        mn = min(mn, bounds[2 * i][w]);
        mx = max(mx, bounds[2 * i + 1][w]);
      }
      lo[i] = max(mn - k + 1, 0);
      ext[i] = min(mx + k, N) - lo[i] + 1;
    }
  }
  int64_t vol = F;
#pragma unroll
  for (int i = 0; i < D; ++i) vol *= ext[i];
  const bool use_lds = vol <= kRbfLdsValues;  // uniform over the workgroup
  if (use_lds) {
    for (int i = threadIdx.x; i < (int)vol; i += kRbfBwdBlock) acc[i] = 0.0;
    __syncthreads();
  }

  const bool dense = (g.dense[0] >> l) & 1u;
  float* tab = grad + g.off[0][l];
  if (on) {
    const int64_t LF = (int64_t)g.Lrow * F;
    const int64_t col = (int64_t)l * F;
    float G0[F], G1[D][F], G2[D][F];
#pragma unroll
    for (int f = 0; f < F; ++f) {
      G0[f] = 0.0f;
#pragma unroll
      for (int i = 0; i < D; ++i) G1[i][f] = G2[i][f] = 0.0f;
    }
    if (g_gamma) load_vec<F>(g_gamma + p * LF + col, G0);
    if (g_dgamma) {
#pragma unroll
      for (int i = 0; i < D; ++i) load_vec<F>(g_dgamma + (p * D + i) * LF + col, G1[i]);
    }
    if (g_d2gamma) {
      if (d2_mode == HASHENC_D2_DIAG) {
#pragma unroll
        for (int i = 0; i < D; ++i) load_vec<F>(g_d2gamma + (p * D + i) * LF + col, G2[i]);
      } else {
        load_vec<F>(g_d2gamma + p * LF + col, G2[0]);
#pragma unroll
        for (int i = 1; i < D; ++i)
#pragma unroll
          for (int f = 0; f < F; ++f) G2[i][f] = G2[0][f];
      }
    }
    const float inv = 1.0f / s.S;
    float ca[F], cb[D][F], cc[D][F];
#pragma unroll
    for (int f = 0; f < F; ++f) {
      float a = G0[f] * inv;
#pragma unroll
      for (int i = 0; i < D; ++i) {
        a -= (s.dS[i] * G1[i][f] + s.d2S[i] * G2[i][f]) * inv * inv;
        a += 2.0f * s.dS[i] * s.dS[i] * G2[i][f] * inv * inv * inv;
        cb[i][f] = G1[i][f] * inv - 2.0f * s.dS[i] * G2[i][f] * inv * inv;
        cc[i][f] = G2[i][f] * inv;
      }
      ca[f] = a;
    }
    const float e2 = g.rbf_e2, Nf = g.Nf[l];
    AxisG gx[kMaxSide];
#pragma unroll
    for (int m = 0; m < kMaxSide; ++m)
      gx[m] = m < side ? rbf_axis(s.t[0], (int32_t)s.base[0], k, m, N, e2, Nf) : AxisG{0.0f, 0.0f, 0.0f};
    // lanes walk the box rows in rotated orders (start row = lane % 2k along y and
    // lane / 2k % 2k along z): lanes whose points share a cell then add into different
    // rows at the same instruction instead of serialising on one LDS address
    const int lane = threadIdx.x & 63;
    const int rot_y = lane % side, rot_z = (lane / side) % side;
    const int zs = D > 2 ? side : 1;
    for (int mz0 = 0; mz0 < zs; ++mz0) {
      AxisG gz{1.0f, 0.0f, 0.0f};
      uint32_t vz = 0;
      if constexpr (D > 2) {
        const int mz = (mz0 + rot_z) % side;
        gz = rbf_axis(s.t[2], (int32_t)s.base[2], k, mz, N, e2, Nf);
        if (gz.g == 0.0f) continue;
        vz = s.base[2] - k + 1 + mz;
      }
      for (int my0 = 0; my0 < side; ++my0) {
        const int my = (my0 + rot_y) % side;
        const AxisG gy = rbf_axis(s.t[1], (int32_t)s.base[1], k, my, N, e2, Nf);
        if (gy.g == 0.0f) continue;
        const uint32_t vy = s.base[1] - k + 1 + my;
        // this row's part, independent of x: P multiplies (gx a + g1x b_x + g2x c_x), Q
        // multiplies gx
        const float P = gy.g * gz.g;
        float Q[F];
#pragma unroll
        for (int f = 0; f < F; ++f) {
          float q = (gy.g1 * cb[1][f] + gy.g2 * cc[1][f]) * gz.g;
          if constexpr (D > 2) q += gy.g * (gz.g1 * cb[2][f] + gz.g2 * cc[2][f]);
          Q[f] = q;
        }
        if (use_lds) {
          int32_t lrow = (int32_t)vy - lo[1];
          if constexpr (D > 2) lrow += ext[1] * ((int32_t)vz - lo[2]);
          const int32_t lbase = lrow * ext[0] + ((int32_t)s.base[0] - k + 1 - lo[0]);
#pragma unroll
          for (int m = 0; m < kMaxSide; ++m) {
            if (m < side && gx[m].g != 0.0f) {
#pragma unroll
              for (int f = 0; f < F; ++f) {
                const float c = P * (gx[m].g * ca[f] + gx[m].g1 * cb[0][f] + gx[m].g2 * cc[0][f]) + gx[m].g * Q[f];
                atomicAdd(&acc[(lbase + m) * F + f], (double)c);
              }
            }
          }
        } else {
          const uint32_t key = rbf_key(vy, vz, N, dense);
#pragma unroll
          for (int m = 0; m < kMaxSide; ++m) {
            if (m < side && gx[m].g != 0.0f) {
              const uint32_t row = rbf_row(s.base[0] - k + 1 + m, key, dense, g.T[0], g.Tmask[0]);
#pragma unroll
              for (int f = 0; f < F; ++f) {
                const float c = P * (gx[m].g * ca[f] + gx[m].g1 * cb[0][f] + gx[m].g2 * cc[0][f]) + gx[m].g * Q[f];
                atomic_add_f32(tab + (size_t)row * F + f, c);
              }
            }
          }
        }
      }
    }
  }
  if (!use_lds) return;
  __syncthreads();
  // one global add per touched vertex feature, consecutive threads on consecutive features
  for (int i = threadIdx.x; i < (int)vol; i += kRbfBwdBlock) {
    const float v = (float)acc[i];
    if (v == 0.0f) continue;
    const int f = i % F;
    int32_t r = i / F;
    const uint32_t vx = (uint32_t)(lo[0] + r % ext[0]);
    r /= ext[0];
    uint32_t vy = 0, vz = 0;
    if constexpr (D > 1) { vy = (uint32_t)(lo[1] + r % ext[1]); r /= ext[1]; }
    if constexpr (D > 2) vz = (uint32_t)(lo[2] + r);
    const uint32_t row = rbf_row(vx, rbf_key(vy, vz, N, dense), dense, g.T[0], g.Tmask[0]);
    atomic_add_f32(tab + (size_t)row * F + f, v);
  }
}

template <int D, int F>
hipError_t launch_fwd(const Grid& g, int d2_mode, int64_t n, const float* x, const float* params, float* gamma,
                      float* dgamma, float* d2gamma, hipStream_t s) {
  const int64_t tiles = (n + kBlock - 1) / kBlock;
  if (tiles * g.L > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL((rbf_forward_kernel<D, F>), dim3((unsigned)(tiles * g.L)), dim3(kBlock), 0, s, g, n,
                     (int32_t)tiles, d2_mode, x, params, gamma, dgamma, d2gamma);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || g.L == g.Lrow) return e;
  // inactive levels (coarse-to-fine): zero their columns
  const int RF = g.Lrow * F, AF = g.L * F;
  if (gamma) e = launch_zero_columns(gamma, n, RF, AF, s);
  if (e == hipSuccess && dgamma) e = launch_zero_columns(dgamma, n * D, RF, AF, s);
  if (e == hipSuccess && d2gamma)
    e = launch_zero_columns(d2gamma, n * (d2_mode == HASHENC_D2_DIAG ? D : 1), RF, AF, s);
  return e;
}

template <int D, int F>
hipError_t launch_bwd(const Grid& g, int d2_mode, int64_t n, const float* x, const float* gg, const float* gd,
                      const float* g2, float* grad, hipStream_t s) {
  const int64_t tiles = (n + kRbfBwdBlock - 1) / kRbfBwdBlock;
  if (tiles * g.L > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL((rbf_backward_kernel<D, F>), dim3((unsigned)(tiles * g.L)), dim3(kRbfBwdBlock), 0, s, g, n,
                     (int32_t)tiles, d2_mode, x, gg, gd, g2, grad);
  return hipGetLastError();
}

}  // namespace

#define HASHENC_DISPATCH_DF(d, F, FN, ...)       \
  do {                                           \
    if (d == 2) {                                \
      switch (F) {                               \
        case 1: return FN<2, 1>(__VA_ARGS__);    \
        case 2: return FN<2, 2>(__VA_ARGS__);    \
        case 4: return FN<2, 4>(__VA_ARGS__);    \
        case 8: return FN<2, 8>(__VA_ARGS__);    \
      }                                          \
    } else if (d == 3) {                         \
      switch (F) {                               \
        case 1: return FN<3, 1>(__VA_ARGS__);    \
        case 2: return FN<3, 2>(__VA_ARGS__);    \
        case 4: return FN<3, 4>(__VA_ARGS__);    \
        case 8: return FN<3, 8>(__VA_ARGS__);    \
      }                                          \
    }                                            \
    return hipErrorInvalidValue;                 \
  } while (0)

hipError_t launch_rbf_forward(const Grid& g, int d, int F, int d2_mode, int64_t n, const float* x,
                              const float* params, float* gamma, float* dgamma, float* d2gamma, hipStream_t s) {
  HASHENC_DISPATCH_DF(d, F, launch_fwd, g, d2_mode, n, x, params, gamma, dgamma, d2gamma, s);
}

hipError_t launch_rbf_backward(const Grid& g, int d, int F, int d2_mode, int64_t n, const float* x,
                               const float* g_gamma, const float* g_dgamma, const float* g_d2gamma, float* grad,
                               hipStream_t s) {
  HASHENC_DISPATCH_DF(d, F, launch_bwd, g, d2_mode, n, x, g_gamma, g_dgamma, g_d2gamma, grad, s);
}

}  // namespace hg
