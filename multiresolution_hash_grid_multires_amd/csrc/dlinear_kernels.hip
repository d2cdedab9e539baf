// Instant-NGP d-linear hash-grid encoding: forward gather + interpolation and backward
// scatter-add, gfx950.
//
// Method: Instant-NGP explainer (nxrte.com), encoding pipeline steps 1-4 (per level, the
// 2^d vertices around x, table lookup, d-linear interpolation, concatenation over levels);
// Instant-NGP news article (antipu.com.cn), efficiency paragraph (no control flow, all
// levels looked up independently) and adaptivity paragraph (colliding gradients combine:
// here they sum).
//
// Mapping: one lane per point, the level loop wave-uniform so the per-level block
// description stays in scalar registers; the 2^d corner gathers of a level are
// independent loads issued back to back; x-adjacent corners usually share a cache line.
#include "hashenc_internal.h"
#include "vec_io.h"

namespace hg {
namespace {

template <int D, int F>
__global__ __launch_bounds__(kBlock) void dlinear_forward_kernel(const Grid g, int64_t n,
                                                                 const float* __restrict__ x,
                                                                 const float* __restrict__ params,
                                                                 float* __restrict__ gamma) {
  const int64_t p = (int64_t)blockIdx.x * kBlock + threadIdx.x;
  if (p >= n) return;
  float xp[D];
#pragma unroll
  for (int i = 0; i < D; ++i) xp[i] = x[p * D + i];
  const int64_t LF = (int64_t)g.L * F;
  float* out = gamma + p * LF;
  for (int l = 0; l < g.L; ++l) {
    uint32_t base[D];
    float t[D];
    locate<D>(xp, g.N[l], g.Nf[l], base, t);
    const CellKeys<D> keys = cell_keys<D>(base, g.N[l]);
    const bool dense = (g.dense[0] >> l) & 1u;
    const float* tab = params + g.off[0][l];
    float rows[1 << D][F];
    // issue every gather of the level before using any of them
    [&]<int... C>(std::integer_sequence<int, C...>) {
      ((load_vec<F>(tab + (size_t)corner_row<D, C>(keys, dense, g.T[0], g.Tmask[0]) * F, rows[C])), ...);
    }(std::make_integer_sequence<int, 1 << D>{});
    float acc[F];
#pragma unroll
    for (int f = 0; f < F; ++f) acc[f] = 0.0f;
#pragma unroll
    for (int c = 0; c < (1 << D); ++c) {
      float w = 1.0f;
#pragma unroll
      for (int i = 0; i < D; ++i) w *= ((c >> i) & 1) ? t[i] : 1.0f - t[i];
#pragma unroll
      for (int f = 0; f < F; ++f) acc[f] = fmaf(w, rows[c][f], acc[f]);
    }
    store_vec<F>(out + (int64_t)l * F, acc);
  }
}

// Backward.  Fp32 atomics are issued as one memory request per 64-byte segment that the
// lanes of an instruction touch, and the request rate -- not the dword count -- bounds the
// scatter-add.  The two corners of a cell that differ only along x sit in adjacent rows on
// dense levels and within one aligned row octet on hashed levels (the x coordinate enters
// the hash through XOR with prime 1), so 2F lanes cooperate on one point: lane
// (c0, f) owns feature f of the x-corner c0 of every (y, z) corner pair, and each atomic
// instruction then covers 64 / (2F) points with 2F contiguous dwords each.
template <int D, int F>
__global__ __launch_bounds__(kBlock) void dlinear_backward_kernel(const Grid g, int64_t n,
                                                                  const float* __restrict__ x,
                                                                  const float* __restrict__ g_gamma,
                                                                  float* __restrict__ grad) {
  constexpr int LANES = 2 * F;  // lanes per point
  const int64_t gid = (int64_t)blockIdx.x * kBlock + threadIdx.x;
  const int64_t p = gid / LANES;
  if (p >= n) return;
  const int sub = (int)(gid % LANES);
  const int c0 = sub / F;  // x-corner bit of this lane
  const int f = sub % F;   // feature of this lane
  float xp[D];
#pragma unroll
  for (int i = 0; i < D; ++i) xp[i] = x[p * D + i];
  const int64_t LF = (int64_t)g.L * F;
  const float* up = g_gamma + p * LF + f;
  for (int l = 0; l < g.L; ++l) {
    const float G = up[(int64_t)l * F];
    uint32_t base[D];
    float t[D];
    locate<D>(xp, g.N[l], g.Nf[l], base, t);
    const CellKeys<D> keys = cell_keys<D>(base, g.N[l]);
    const bool dense = (g.dense[0] >> l) & 1u;
    float* tab = grad + g.off[0][l] + f;
    const float wx = G * (c0 ? t[0] : 1.0f - t[0]);
#pragma unroll
    for (int yz = 0; yz < (1 << (D - 1)); ++yz) {
      float w = wx;
#pragma unroll
      for (int i = 1; i < D; ++i) w *= ((yz >> (i - 1)) & 1) ? t[i] : 1.0f - t[i];
      const uint32_t row = corner_row_rt<D>(keys, c0 | (yz << 1), dense, g.T[0], g.Tmask[0]);
      atomic_add_f32(tab + (size_t)row * F, w);
    }
  }
}

template <int D, int F>
hipError_t launch_fwd(const Grid& g, int64_t n, const float* x, const float* params, float* gamma,
                      hipStream_t s) {
  const dim3 grid((unsigned)((n + kBlock - 1) / kBlock));
  hipLaunchKernelGGL((dlinear_forward_kernel<D, F>), grid, dim3(kBlock), 0, s, g, n, x, params, gamma);
  return hipGetLastError();
}

template <int D, int F>
hipError_t launch_bwd(const Grid& g, int64_t n, const float* x, const float* gg, float* grad,
                      hipStream_t s) {
  const int64_t lanes = n * 2 * F;
  const dim3 grid((unsigned)((lanes + kBlock - 1) / kBlock));
  hipLaunchKernelGGL((dlinear_backward_kernel<D, F>), grid, dim3(kBlock), 0, s, g, n, x, gg, grad);
  return hipGetLastError();
}

}  // namespace

#define HASHENC_DISPATCH_DF(d, F, FN, ...)                            \
  do {                                                                \
    if (d == 2) {                                                     \
      switch (F) {                                                    \
        case 1: return FN<2, 1>(__VA_ARGS__);                         \
        case 2: return FN<2, 2>(__VA_ARGS__);                         \
        case 4: return FN<2, 4>(__VA_ARGS__);                         \
        case 8: return FN<2, 8>(__VA_ARGS__);                         \
      }                                                               \
    } else if (d == 3) {                                              \
      switch (F) {                                                    \
        case 1: return FN<3, 1>(__VA_ARGS__);                         \
        case 2: return FN<3, 2>(__VA_ARGS__);                         \
        case 4: return FN<3, 4>(__VA_ARGS__);                         \
        case 8: return FN<3, 8>(__VA_ARGS__);                         \
      }                                                               \
    }                                                                 \
    return hipErrorInvalidValue;                                      \
  } while (0)

hipError_t launch_dlinear_forward(const Grid& g, int d, int F, int64_t n, const float* x,
                                  const float* params, float* gamma, hipStream_t s) {
  HASHENC_DISPATCH_DF(d, F, launch_fwd, g, n, x, params, gamma, s);
}

hipError_t launch_dlinear_backward(const Grid& g, int d, int F, int64_t n, const float* x,
                                   const float* g_gamma, float* grad, hipStream_t s) {
  HASHENC_DISPATCH_DF(d, F, launch_bwd, g, n, x, g_gamma, grad, s);
}

}  // namespace hg
