// Hermite-NGP gradient-augmented hash-grid encoding, gfx950: one pass gives gamma, its
// spatial gradient and its second derivatives (diagonal or Laplacian); the backward
// scatter-adds into the order-bucketed tables.
//
// Method: "Hermite-NGP: Gradient-Augmented Hash Encoding for Learning PDEs" notes
// (m0rtzz.github.io), key design 1: every vertex stores all 2^d mixed partials f^(alpha),
// alpha in {0,1}^d, bucketed into tables by |alpha|; the level field is
//   gamma_l(x) = sum_g sum_alpha theta^(alpha)_{l,h(g)} H^(alpha)((x - x_g)/Dx_l) Dx_l^|alpha|
// with H^(alpha) = prod_i h^(alpha_i), far-corner value basis 3t^2 - 2t^3 and derivative
// basis t^3 - t^2 (the near corner uses their reflections); key design 2: derivatives
// follow from the factorised basis derivatives, d/dx_i = N_l d/dt_i.
//
// Evaluation is sum-factorised: with m_i = 2 c_i + alpha_i in 0..3 (corner bit, derivative
// bit) the coefficient tensor theta[m_0][m_1]...[F] is contracted one axis at a time
// against per-axis basis vectors B_i[m], B'_i[m], B''_i[m] that already carry the
// Dx^alpha_i scaling and the N_l chain-rule factors, so no per-term power or product chain
// is evaluated.  Corners are visited in x-adjacent pairs (the axis-0 contraction needs
// exactly one pair), which bounds the live coefficient registers to 2 * 2^d * F.
#include <algorithm>

#include "binned_backward.h"
#include "hashenc_internal.h"
#include "vec_io.h"

namespace hg {
namespace {

// Per-axis basis at local coordinate t, indexed m = 2 c + a.  Values include Dx^a;
// first derivatives are d/dx (factor N); second derivatives d^2/dx^2 (factor N^2).
struct AxisBasis {
  float B[4], dB[4], d2B[4];
};

__device__ __forceinline__ AxisBasis axis_basis(float t, float N, float invN) {
  const float s = 1.0f - t;
  const float t2 = t * t;
  AxisBasis a;
  // near corner, value: 1 - 3t^2 + 2t^3 = (1 + 2t)(1 - t)^2
  const float h00 = (1.0f + 2.0f * t) * s * s;
  const float h00p = -6.0f * t * s;
  const float h00pp = 12.0f * t - 6.0f;
  // near corner, derivative: t - 2t^2 + t^3 = t (1 - t)^2
  const float h10 = t * s * s;
  const float h10p = s * (1.0f - 3.0f * t);
  const float h10pp = 6.0f * t - 4.0f;
  // far corner, value: 3t^2 - 2t^3
  const float h01 = t2 * (3.0f - 2.0f * t);
  // far corner, derivative: t^3 - t^2
  const float h11 = -t2 * s;
  const float h11p = t * (3.0f * t - 2.0f);
  const float h11pp = 6.0f * t - 2.0f;
  const float N2 = N * N;
  a.B[0] = h00;          a.dB[0] = N * h00p;   a.d2B[0] = N2 * h00pp;
  a.B[1] = invN * h10;   a.dB[1] = h10p;       a.d2B[1] = N * h10pp;
  a.B[2] = h01;          a.dB[2] = -N * h00p;  a.d2B[2] = -N2 * h00pp;
  a.B[3] = invN * h11;   a.dB[3] = h11p;       a.d2B[3] = N * h11pp;
  return a;
}

__host__ __device__ constexpr int popc(int a) { return (a & 1) + ((a >> 1) & 1) + ((a >> 2) & 1); }

// Slot of derivative multi-index `alpha` (bit i = axis i) inside its order table's row:
// order 1: x, y, z; order 2: xy, xz, yz (lexicographic axis tuples).
__host__ __device__ constexpr int slot_of(int alpha) {
  return alpha == 0 ? 0 : alpha == 1 ? 0 : alpha == 2 ? 1 : alpha == 4 ? 2
       : alpha == 3 ? 0 : alpha == 5 ? 1 : alpha == 6 ? 2 : 0;
}

__host__ __device__ constexpr int binom_d(int D, int k) {
  return D == 2 ? (k == 1 ? 2 : 1) : (k == 1 || k == 2 ? 3 : 1);
}

// Coefficient rows of one corner: table k holds binom(D,k) slots of F floats.
template <int D, int F>
struct CornerRows {
  float r0[F];
  float r1[binom_d(D, 1) * F];
  float r2[binom_d(D, 2) * F];
  float r3[(D == 3 ? 1 : 1) * F];  // order-3 row (D = 3 only)

  template <int ALPHA>
  __device__ __forceinline__ float get(int f) const {
    constexpr int k = popc(ALPHA);
    constexpr int s = slot_of(ALPHA);
    if constexpr (k == 0) return r0[f];
    else if constexpr (k == 1) return r1[s * F + f];
    else if constexpr (k == 2) return r2[s * F + f];
    else return r3[f];
  }
  template <int ALPHA>
  __device__ __forceinline__ float& at(int f) {
    constexpr int k = popc(ALPHA);
    constexpr int s = slot_of(ALPHA);
    if constexpr (k == 0) return r0[f];
    else if constexpr (k == 1) return r1[s * F + f];
    else if constexpr (k == 2) return r2[s * F + f];
    else return r3[f];
  }
};

// Per-level table lookup state for all order tables.
struct TableSel {
  const float* base[kMaxTables];
  bool dense[kMaxTables];
};

template <int D, int F, int C>
__device__ __forceinline__ void gather_corner(const Grid& g, const CellKeys<D>& keys,
                                              const TableSel& ts, CornerRows<D, F>& cr) {
  load_vec<F>(ts.base[0] + (size_t)corner_row<D, C>(keys, ts.dense[0], g.T[0], g.Tmask[0]) * F, cr.r0);
  load_vec<binom_d(D, 1) * F>(
      ts.base[1] + (size_t)corner_row<D, C>(keys, ts.dense[1], g.T[1], g.Tmask[1]) * (binom_d(D, 1) * F), cr.r1);
  load_vec<binom_d(D, 2) * F>(
      ts.base[2] + (size_t)corner_row<D, C>(keys, ts.dense[2], g.T[2], g.Tmask[2]) * (binom_d(D, 2) * F), cr.r2);
  if constexpr (D == 3)
    load_vec<F>(ts.base[3] + (size_t)corner_row<D, C>(keys, ts.dense[3], g.T[3], g.Tmask[3]) * F, cr.r3);
}

// Packed copy of the order tables: row r of level l -- the row a vertex has in the order-0
// table -- holds [order 0: F | order 1: C(d,1) F | order 2: C(d,2) F | order 3: F]
// contiguously, 2^d F floats (one 64-byte sector for d = 3, F = 2), so the forward reads a
// corner's coefficients in one contiguous access instead of one per order table.  With
// equal table sizes a vertex has the same row everywhere.  A smaller order table (power-of-
// two sizes no larger than the order-0 one, as in the pages' best 14-14-10 sizing) is hashed
// wherever the order-0 table is, with a row that is the order-0 row modulo its size, and a
// dense order-0 row names its vertex: so the vertex's row in every table follows from r, and
// the smaller table's rows are repeated across the packed rows that share them.
struct PackPlan {
  int64_t poff[kMaxLevels + 1];  // float offset of level l in the packed copy
};

template <int D, int F>
__device__ __forceinline__ void gather_corner_packed(const float* __restrict__ base, uint32_t row,
                                                     CornerRows<D, F>& cr) {
  constexpr int W1 = binom_d(D, 1) * F, W2 = binom_d(D, 2) * F;
  constexpr int RW = (1 << D) * F;
  float v[RW];
  load_vec<RW>(base + (size_t)row * RW, v);
#pragma unroll
  for (int j = 0; j < F; ++j) cr.r0[j] = v[j];
#pragma unroll
  for (int j = 0; j < W1; ++j) cr.r1[j] = v[F + j];
#pragma unroll
  for (int j = 0; j < W2; ++j) cr.r2[j] = v[F + W1 + j];
  if constexpr (D == 3) {
#pragma unroll
    for (int j = 0; j < F; ++j) cr.r3[j] = v[F + W1 + W2 + j];
  }
}

// One thread per packed row: gather the row's slots from the d + 1 order tables.  Packed row
// t sits at float t * RW across all levels, so a workgroup's rows form one contiguous block:
// they are parked in LDS (pitch RW + 4 floats against bank conflicts) and written out as
// consecutive 16-byte pieces, whole lines per store instruction, where each lane storing its
// own row would touch one line per lane and instruction.
template <int D, int F>
__global__ __launch_bounds__(kBlock) void hermite_pack_kernel(const Grid g, const PackPlan pp,
                                                              const float* __restrict__ params,
                                                              float* __restrict__ packed) {
  constexpr int W1 = binom_d(D, 1) * F, W2 = binom_d(D, 2) * F;
  constexpr int RW = (1 << D) * F;
  constexpr int PITCH = RW + 4;
  __shared__ float stage[kBlock * PITCH];
  const int64_t total = pp.poff[g.L] / RW;  // packed rows
  const int64_t t0 = (int64_t)blockIdx.x * kBlock;
  const int64_t t = t0 + threadIdx.x;
  if (t < total) {
    int l = 0;
    while (l + 1 < g.L && t * RW >= pp.poff[l + 1]) ++l;
    const int64_t r = t - pp.poff[l] / RW;
    // row of the same vertex (or hash bucket) in table k
    auto row_in = [&](int k) -> int64_t {
      if (g.T[k] == g.T[0]) return r;
      if (!((g.dense[0] >> l) & 1u)) return r & (int64_t)(g.T[k] - 1);  // both hashed, T_k | T_0
      if ((g.dense[k] >> l) & 1u) return r;                                // both dense
      const uint32_t N1 = (uint32_t)g.N[l] + 1u;                           // dense row -> vertex
      uint32_t h = (uint32_t)(r % N1);
      if (D > 1) h ^= (uint32_t)((r / N1) % N1) * kPrime1;
      if (D > 2) h ^= (uint32_t)(r / ((int64_t)N1 * N1)) * kPrime2;
      return h & (g.T[k] - 1u);
    };
    float v[RW];
    load_vec_at<F>(params + g.off[0][l] + r * F, v, 0);
    load_vec_at<W1>(params + g.off[1][l] + row_in(1) * W1, v, F);
    load_vec_at<W2>(params + g.off[2][l] + row_in(2) * W2, v, F + W1);
    if constexpr (D == 3) load_vec_at<F>(params + g.off[3][l] + row_in(3) * F, v, F + W1 + W2);
    store_vec<RW>(stage + threadIdx.x * PITCH, v);
  }
  __syncthreads();
  const int nr = (int)(total - t0 < kBlock ? total - t0 : kBlock);
  constexpr int Q = RW / 4;  // 16-byte pieces per row
  float4* dst = reinterpret_cast<float4*>(packed + t0 * RW);
  for (int q = threadIdx.x; q < nr * Q; q += kBlock) {
    const int row = q / Q, c = q - row * Q;
    dst[q] = *reinterpret_cast<const float4*>(stage + row * PITCH + 4 * c);
  }
}

template <int D, int F, int C>
__device__ __forceinline__ void scatter_corner(const Grid& g, const CellKeys<D>& keys,
                                               float* const (&base)[kMaxTables],
                                               const bool (&dense)[kMaxTables],
                                               CornerRows<D, F>& cr) {
  float* p0 = base[0] + (size_t)corner_row<D, C>(keys, dense[0], g.T[0], g.Tmask[0]) * F;
#pragma unroll
  for (int j = 0; j < F; ++j) atomic_add_f32(p0 + j, cr.r0[j]);
  constexpr int W1 = binom_d(D, 1) * F;
  float* p1 = base[1] + (size_t)corner_row<D, C>(keys, dense[1], g.T[1], g.Tmask[1]) * W1;
#pragma unroll
  for (int j = 0; j < W1; ++j) atomic_add_f32(p1 + j, cr.r1[j]);
  constexpr int W2 = binom_d(D, 2) * F;
  float* p2 = base[2] + (size_t)corner_row<D, C>(keys, dense[2], g.T[2], g.Tmask[2]) * W2;
#pragma unroll
  for (int j = 0; j < W2; ++j) atomic_add_f32(p2 + j, cr.r2[j]);
  if constexpr (D == 3) {
    float* p3 = base[3] + (size_t)corner_row<D, C>(keys, dense[3], g.T[3], g.Tmask[3]) * F;
#pragma unroll
    for (int j = 0; j < F; ++j) atomic_add_f32(p3 + j, cr.r3[j]);
  }
}

// ------------------------------------------------------------------ forward
// Outputs of one level: value, d gradient components, d second-derivative components.
template <int D, int F>
struct LevelOut {
  float v[F];
  float g[D][F];
  float h[D][F];
};

// Accumulate the contribution of the x-adjacent corner pair (0, Y) with Y the corner bits
// of axes 1.. (Y = c1 | c2 << 1).
template <int D, int F, int Y, bool PACKED>
__device__ __forceinline__ void fwd_pair(const Grid& g, const CellKeys<D>& keys, const TableSel& ts,
                                         const float* __restrict__ pbase, const AxisBasis (&ab)[D],
                                         LevelOut<D, F>& o) {
  CornerRows<D, F> lo, hi;
  if constexpr (PACKED) {
    gather_corner_packed<D, F>(pbase, corner_row<D, (Y << 1)>(keys, ts.dense[0], g.T[0], g.Tmask[0]), lo);
    gather_corner_packed<D, F>(pbase, corner_row<D, (Y << 1) | 1>(keys, ts.dense[0], g.T[0], g.Tmask[0]), hi);
  } else {
    gather_corner<D, F, (Y << 1)>(g, keys, ts, lo);
    gather_corner<D, F, (Y << 1) | 1>(g, keys, ts, hi);
  }
  constexpr int c1 = Y & 1;
  constexpr int c2 = (Y >> 1) & 1;
  constexpr int NA = 1 << (D - 1);  // derivative patterns over axes 1..D-1
  [&]<int... A>(std::integer_sequence<int, A...>) {
    (([&] {
       constexpr int a1 = A & 1;
       constexpr int a2 = (A >> 1) & 1;
       constexpr int m1 = 2 * c1 + a1;
       constexpr int m2 = 2 * c2 + a2;
       constexpr int al0 = (a1 << 1) | (a2 << 2);  // alpha with a0 = 0
       constexpr int al1 = al0 | 1;                 // alpha with a0 = 1
       float S[F], S1[F], S2[F];
#pragma unroll
       for (int f = 0; f < F; ++f) {
         // contraction over m0 = 2 c0 + a0
         const float t00 = lo.template get<al0>(f), t01 = lo.template get<al1>(f);
         const float t10 = hi.template get<al0>(f), t11 = hi.template get<al1>(f);
         S[f] = ab[0].B[0] * t00 + ab[0].B[1] * t01 + ab[0].B[2] * t10 + ab[0].B[3] * t11;
         S1[f] = ab[0].dB[0] * t00 + ab[0].dB[1] * t01 + ab[0].dB[2] * t10 + ab[0].dB[3] * t11;
         S2[f] = ab[0].d2B[0] * t00 + ab[0].d2B[1] * t01 + ab[0].d2B[2] * t10 + ab[0].d2B[3] * t11;
       }
       if constexpr (D == 2) {
         const float w = ab[1].B[m1], wd = ab[1].dB[m1], wdd = ab[1].d2B[m1];
#pragma unroll
         for (int f = 0; f < F; ++f) {
           o.v[f] = fmaf(S[f], w, o.v[f]);
           o.g[0][f] = fmaf(S1[f], w, o.g[0][f]);
           o.h[0][f] = fmaf(S2[f], w, o.h[0][f]);
           o.g[1][f] = fmaf(S[f], wd, o.g[1][f]);
           o.h[1][f] = fmaf(S[f], wdd, o.h[1][f]);
         }
       } else {
         const float b1 = ab[1].B[m1], b2 = ab[2].B[m2];
         const float w = b1 * b2;
         const float w1 = ab[1].dB[m1] * b2, w11 = ab[1].d2B[m1] * b2;
         const float w2 = b1 * ab[2].dB[m2], w22 = b1 * ab[2].d2B[m2];
#pragma unroll
         for (int f = 0; f < F; ++f) {
           o.v[f] = fmaf(S[f], w, o.v[f]);
           o.g[0][f] = fmaf(S1[f], w, o.g[0][f]);
           o.h[0][f] = fmaf(S2[f], w, o.h[0][f]);
           o.g[1][f] = fmaf(S[f], w1, o.g[1][f]);
           o.h[1][f] = fmaf(S[f], w11, o.h[1][f]);
           o.g[2][f] = fmaf(S[f], w2, o.g[2][f]);
           o.h[2][f] = fmaf(S[f], w22, o.h[2][f]);
         }
       }
     }()),
     ...);
  }(std::make_integer_sequence<int, NA>{});
}

template <int D>
__device__ __forceinline__ void level_setup(const Grid& g, int l, const float (&xp)[D],
                                            CellKeys<D>& keys, AxisBasis (&ab)[D]) {
  uint32_t base[D];
  float t[D];
  locate<D>(xp, g.N[l], g.Nf[l], base, t);
  keys = cell_keys<D>(base, g.N[l]);
#pragma unroll
  for (int i = 0; i < D; ++i) ab[i] = axis_basis(t[i], g.Nf[l], g.invN[l]);
}

// Level-major order as in the d-linear forward: workgroup b handles level b / n_tiles, so
// the chip streams one level's order tables at a time (they stay in L2 / Infinity Cache).
// PACKED: read the corner rows from the packed copy (params points at it; pp gives the
// level offsets) instead of the d + 1 order tables.
// LM: write the level's outputs level-major into stage[l][p][m][F], m = value, d gradient
// components, then the second-derivative components (d diagonal ones or the Laplacian):
// whole lines per workgroup, where the point-major rows take 8-byte pieces of many lines.
// The workgroup's outputs are one contiguous run there; they are parked in LDS and written
// as consecutive 16-byte pieces (a lane storing its own point's M F floats would touch one
// line per lane and store instruction).
template <int D, int F, bool PACKED, bool LM>
__global__ __launch_bounds__(kBlock) void hermite_forward_kernel(
    const Grid g, const PackPlan pp, int64_t n, int32_t n_tiles, int d2_mode, const float* __restrict__ x,
    const float* __restrict__ params, float* __restrict__ gamma, float* __restrict__ dgamma,
    float* __restrict__ d2gamma, float* __restrict__ stage) {
  constexpr int PTS = kBlock / 2;  // points per workgroup: two lanes per point
  const int l = blockIdx.x / n_tiles;
  const int half = threadIdx.x & 1;  // which half of the cell's x-corner pairs this lane gathers
  const int64_t p0 = (int64_t)(blockIdx.x % n_tiles) * PTS;
  const int64_t p = p0 + (threadIdx.x >> 1);
  if constexpr (!LM) {
    if (p >= n) return;  // both lanes of a point leave together
  }
  // with LM every lane reaches the staging barrier: lanes past the end evaluate the last point
  const int64_t pc = p < n ? p : n - 1;
  float xp[D];
#pragma unroll
  for (int i = 0; i < D; ++i) xp[i] = x[pc * D + i];
  const int64_t LF = (int64_t)g.Lrow * F;
  CellKeys<D> keys;
  AxisBasis ab[D];
  level_setup<D>(g, l, xp, keys, ab);
  TableSel ts;
#pragma unroll
  for (int k = 0; k <= D; ++k) {
    ts.base[k] = params + g.off[k][l];
    ts.dense[k] = (g.dense[k] >> l) & 1u;
  }
  LevelOut<D, F> o;
#pragma unroll
  for (int f = 0; f < F; ++f) {
    o.v[f] = 0.0f;
#pragma unroll
    for (int i = 0; i < D; ++i) o.g[i][f] = o.h[i][f] = 0.0f;
  }
  const float* pbase = PACKED ? params + pp.poff[l] : nullptr;
  // lane 0 of the point: pairs 0 .. NP/2 - 1, lane 1: the rest; the partial sums meet through
  // one cross-lane add per output value (fewer registers per lane, twice the wavefronts in
  // flight on the gathers)
  if (half == 0) {
    fwd_pair<D, F, 0, PACKED>(g, keys, ts, pbase, ab, o);
    if constexpr (D == 3) fwd_pair<D, F, 1, PACKED>(g, keys, ts, pbase, ab, o);
  } else if constexpr (D == 3) {
    fwd_pair<D, F, 2, PACKED>(g, keys, ts, pbase, ab, o);
    fwd_pair<D, F, 3, PACKED>(g, keys, ts, pbase, ab, o);
  } else {
    fwd_pair<D, F, 1, PACKED>(g, keys, ts, pbase, ab, o);
  }
#pragma unroll
  for (int f = 0; f < F; ++f) {
    o.v[f] = add_lane_pair(o.v[f]);
#pragma unroll
    for (int i = 0; i < D; ++i) {
      o.g[i][f] = add_lane_pair(o.g[i][f]);
      o.h[i][f] = add_lane_pair(o.h[i][f]);
    }
  }
  if constexpr (LM) {
    __shared__ __align__(16) float ob[PTS * (1 + 2 * D) * F];
    const bool diag = d2_mode == HASHENC_D2_DIAG;
    const int M = 1 + D + (diag ? D : 1);
    const int MF = M * F;
    if (!half) {
      float* o_pt = ob + (threadIdx.x >> 1) * MF;
#pragma unroll
      for (int f = 0; f < F; ++f) o_pt[f] = o.v[f];
#pragma unroll
      for (int i = 0; i < D; ++i)
#pragma unroll
        for (int f = 0; f < F; ++f) o_pt[(1 + i) * F + f] = o.g[i][f];
      if (diag) {
#pragma unroll
        for (int i = 0; i < D; ++i)
#pragma unroll
          for (int f = 0; f < F; ++f) o_pt[(1 + D + i) * F + f] = o.h[i][f];
      } else {
#pragma unroll
        for (int f = 0; f < F; ++f) {
          float s = 0.0f;
#pragma unroll
          for (int i = 0; i < D; ++i) s += o.h[i][f];
          o_pt[(1 + D) * F + f] = s;
        }
      }
    }
    __syncthreads();
    const int np = (int)(n - p0 < PTS ? n - p0 : PTS);
    const int tot = np * MF;
    float* dst = stage + ((int64_t)l * n + p0) * MF;
    if (((n * MF) & 3) == 0 && (tot & 3) == 0) {  // the run starts and ends on 16-byte boundaries
      for (int q = threadIdx.x; q < (tot >> 2); q += kBlock)
        reinterpret_cast<float4*>(dst)[q] = reinterpret_cast<const float4*>(ob)[q];
    } else {
      for (int e = threadIdx.x; e < tot; e += kBlock) dst[e] = ob[e];
    }
    return;
  }
  if (half) return;
  const int64_t col = (int64_t)l * F;
  if (gamma) store_vec<F>(gamma + p * LF + col, o.v);
  if (dgamma) {
#pragma unroll
    for (int i = 0; i < D; ++i) store_vec<F>(dgamma + (p * D + i) * LF + col, o.g[i]);
  }
  if (d2gamma) {
    if (d2_mode == HASHENC_D2_DIAG) {
#pragma unroll
      for (int i = 0; i < D; ++i) store_vec<F>(d2gamma + (p * D + i) * LF + col, o.h[i]);
    } else {
      float lap[F];
#pragma unroll
      for (int f = 0; f < F; ++f) {
        float s = 0.0f;
#pragma unroll
        for (int i = 0; i < D; ++i) s += o.h[i][f];
        lap[f] = s;
      }
      store_vec<F>(d2gamma + p * LF + col, lap);
    }
  }
}

// ------------------------------------------------------------------ backward
template <int D, int F>
struct LevelUp {
  float v[F];
  float g[D][F];
  float h[D][F];
};

// max |u| over a level's upstream, as fp32 bits (NaN above inf above every finite value)
template <int D, int F>
__device__ __forceinline__ uint32_t level_up_absmax(const LevelUp<D, F>& u) {
  uint32_t m = 0u;
#pragma unroll
  for (int f = 0; f < F; ++f) {
    m = max(m, abs_bits(u.v[f]));
#pragma unroll
    for (int i = 0; i < D; ++i) m = max(m, max(abs_bits(u.g[i][f]), abs_bits(u.h[i][f])));
  }
  return m;
}

// Reverse of fwd_pair: distribute the level upstream onto the coefficients of corner pair
// (0, Y) and scatter-add them.
template <int D, int F, int Y, class Sink>
__device__ __forceinline__ void bwd_pair(Sink& sink, const AxisBasis (&ab)[D], const LevelUp<D, F>& u) {
  CornerRows<D, F> lo, hi;
  constexpr int c1 = Y & 1;
  constexpr int c2 = (Y >> 1) & 1;
  constexpr int NA = 1 << (D - 1);
  [&]<int... A>(std::integer_sequence<int, A...>) {
    (([&] {
       constexpr int a1 = A & 1;
       constexpr int a2 = (A >> 1) & 1;
       constexpr int m1 = 2 * c1 + a1;
       constexpr int m2 = 2 * c2 + a2;
       constexpr int al0 = (a1 << 1) | (a2 << 2);
       constexpr int al1 = al0 | 1;
       float S[F], S1[F], S2[F];
       if constexpr (D == 2) {
         const float w = ab[1].B[m1], wd = ab[1].dB[m1], wdd = ab[1].d2B[m1];
#pragma unroll
         for (int f = 0; f < F; ++f) {
           S[f] = u.v[f] * w + u.g[1][f] * wd + u.h[1][f] * wdd;
           S1[f] = u.g[0][f] * w;
           S2[f] = u.h[0][f] * w;
         }
       } else {
         const float b1 = ab[1].B[m1], b2 = ab[2].B[m2];
         const float w = b1 * b2;
         const float w1 = ab[1].dB[m1] * b2, w11 = ab[1].d2B[m1] * b2;
         const float w2 = b1 * ab[2].dB[m2], w22 = b1 * ab[2].d2B[m2];
#pragma unroll
         for (int f = 0; f < F; ++f) {
           S[f] = u.v[f] * w + u.g[1][f] * w1 + u.h[1][f] * w11 + u.g[2][f] * w2 + u.h[2][f] * w22;
           S1[f] = u.g[0][f] * w;
           S2[f] = u.h[0][f] * w;
         }
       }
#pragma unroll
       for (int f = 0; f < F; ++f) {
         lo.template at<al0>(f) = S[f] * ab[0].B[0] + S1[f] * ab[0].dB[0] + S2[f] * ab[0].d2B[0];
         lo.template at<al1>(f) = S[f] * ab[0].B[1] + S1[f] * ab[0].dB[1] + S2[f] * ab[0].d2B[1];
         hi.template at<al0>(f) = S[f] * ab[0].B[2] + S1[f] * ab[0].dB[2] + S2[f] * ab[0].d2B[2];
         hi.template at<al1>(f) = S[f] * ab[0].B[3] + S1[f] * ab[0].dB[3] + S2[f] * ab[0].d2B[3];
       }
     }()),
     ...);
  }(std::make_integer_sequence<int, NA>{});
  sink.template emit<(Y << 1)>(lo);
  sink.template emit<(Y << 1) | 1>(hi);
}

// Table-K part of bwd_pair: the coefficient gradients of order table K (slots with
// |alpha| = K) of the x-corner pair (0, Y), lower corner into lo, upper into hi.
template <int D, int F, int Y, int K>
__device__ __forceinline__ void bwd_pair_table(const AxisBasis (&ab)[D], const LevelUp<D, F>& u,
                                               float (&lo)[binom_d(D, K) * F],
                                               float (&hi)[binom_d(D, K) * F]) {
  constexpr int c1 = Y & 1;
  constexpr int c2 = (Y >> 1) & 1;
  constexpr int NA = 1 << (D - 1);
  [&]<int... A>(std::integer_sequence<int, A...>) {
    (([&] {
       constexpr int a1 = A & 1;
       constexpr int a2 = (A >> 1) & 1;
       constexpr int m1 = 2 * c1 + a1;
       constexpr int m2 = 2 * c2 + a2;
       constexpr int al0 = (a1 << 1) | (a2 << 2);
       constexpr int al1 = al0 | 1;
       constexpr bool want0 = popc(al0) == K, want1 = popc(al1) == K;
       if constexpr (want0 || want1) {
         float S[F], S1[F], S2[F];
         if constexpr (D == 2) {
           const float w = ab[1].B[m1], wd = ab[1].dB[m1], wdd = ab[1].d2B[m1];
#pragma unroll
           for (int f = 0; f < F; ++f) {
             S[f] = u.v[f] * w + u.g[1][f] * wd + u.h[1][f] * wdd;
             S1[f] = u.g[0][f] * w;
             S2[f] = u.h[0][f] * w;
           }
         } else {
           const float b1 = ab[1].B[m1], b2 = ab[2].B[m2];
           const float w = b1 * b2;
           const float w1 = ab[1].dB[m1] * b2, w11 = ab[1].d2B[m1] * b2;
           const float w2 = b1 * ab[2].dB[m2], w22 = b1 * ab[2].d2B[m2];
#pragma unroll
           for (int f = 0; f < F; ++f) {
             S[f] = u.v[f] * w + u.g[1][f] * w1 + u.h[1][f] * w11 + u.g[2][f] * w2 + u.h[2][f] * w22;
             S1[f] = u.g[0][f] * w;
             S2[f] = u.h[0][f] * w;
           }
         }
#pragma unroll
         for (int f = 0; f < F; ++f) {
           if constexpr (want0) {
             lo[slot_of(al0) * F + f] = S[f] * ab[0].B[0] + S1[f] * ab[0].dB[0] + S2[f] * ab[0].d2B[0];
             hi[slot_of(al0) * F + f] = S[f] * ab[0].B[2] + S1[f] * ab[0].dB[2] + S2[f] * ab[0].d2B[2];
           }
           if constexpr (want1) {
             lo[slot_of(al1) * F + f] = S[f] * ab[0].B[1] + S1[f] * ab[0].dB[1] + S2[f] * ab[0].d2B[1];
             hi[slot_of(al1) * F + f] = S[f] * ab[0].B[3] + S1[f] * ab[0].dB[3] + S2[f] * ab[0].d2B[3];
           }
         }
       }
     }()),
     ...);
  }(std::make_integer_sequence<int, NA>{});
}

// Backward sink: fp32 atomics straight into the gradient tables.
template <int D, int F>
struct AtomicSink {
  const Grid& g;
  const CellKeys<D>& keys;
  float* base[kMaxTables];
  bool dense[kMaxTables];
  template <int C>
  __device__ __forceinline__ void emit(CornerRows<D, F>& cr) {
    scatter_corner<D, F, C>(g, keys, base, dense, cr);
  }
};

// Upstream of one point at one level (NULL arrays read as zero; the Laplacian upstream is
// the same for every diagonal term).
template <int D, int F>
__device__ __forceinline__ LevelUp<D, F> load_level_up(const Grid& g, int64_t p, int l, int d2_mode,
                                                       const float* __restrict__ g_gamma,
                                                       const float* __restrict__ g_dgamma,
                                                       const float* __restrict__ g_d2gamma) {
  const int64_t LF = (int64_t)g.Lrow * F;
  const int64_t col = (int64_t)l * F;
  LevelUp<D, F> u;
#pragma unroll
  for (int f = 0; f < F; ++f) {
    u.v[f] = 0.0f;
#pragma unroll
    for (int i = 0; i < D; ++i) u.g[i][f] = u.h[i][f] = 0.0f;
  }
  if (g_gamma) load_vec<F>(g_gamma + p * LF + col, u.v);
  if (g_dgamma) {
#pragma unroll
    for (int i = 0; i < D; ++i) load_vec<F>(g_dgamma + (p * D + i) * LF + col, u.g[i]);
  }
  if (g_d2gamma) {
    if (d2_mode == HASHENC_D2_DIAG) {
#pragma unroll
      for (int i = 0; i < D; ++i) load_vec<F>(g_d2gamma + (p * D + i) * LF + col, u.h[i]);
    } else {
      load_vec<F>(g_d2gamma + p * LF + col, u.h[0]);
#pragma unroll
      for (int i = 1; i < D; ++i)
#pragma unroll
        for (int f = 0; f < F; ++f) u.h[i][f] = u.h[0][f];
    }
  }
  return u;
}

// Upstream of the binned scatter, rearranged level-major: U[l][p][m][F] with components
// m = value, d gradient components, then the d diagonal second derivatives (d2_mode
// diagonal) or the one Laplacian.  One workgroup owns P consecutive points: it reads their
// rows of every upstream array (contiguous runs) into LDS and writes each level's
// P * M * F floats as one contiguous run, so the scatter, which runs level by level, reads
// each level's upstream once and in whole lines instead of 8 bytes from every point's row
// per level.  Rows are Lrow * F floats; only the L active levels are rearranged.
template <int F, int D, int M>
__global__ __launch_bounds__(kBlock) void hermite_upstream_levels_kernel(int32_t L, int32_t Lrow, int64_t n,
                                                                         int32_t P,
                                                                         const float* __restrict__ gg,
                                                                         const float* __restrict__ gd,
                                                                         const float* __restrict__ g2,
                                                                         float* __restrict__ U) {
  // LDS holds each point's upstream already in output order: tile[i * pitch + l * M * F +
  // m * F + f], so the write phase reads consecutive words.
  extern __shared__ float tile[];
  constexpr int MF = M * F;
  constexpr int D2 = M - 1 - D;  // second-derivative components (d or 1)
  const int AF = L * F;         // active floats of a row
  const int LF = Lrow * F;      // row stride
  const int pitch = L * MF + 1;
  const int64_t p0 = (int64_t)blockIdx.x * P;
  const int np = (int)min((int64_t)P, n - p0);
  if (((LF | AF) & 3) == 0) {
    // read phase: the tile's rows of each upstream array form one contiguous block (C rows of
    // LF floats per point); lanes take consecutive 16-byte pieces of it, four loads in flight
    // per lane before the LDS writes, and skip the pieces of inactive levels (columns >= AF)
    const int q_row = LF >> 2;  // 16-byte pieces per row
#pragma unroll
    for (int sidx = 0; sidx < 3; ++sidx) {
      const int C = sidx == 0 ? 1 : sidx == 1 ? D : D2;  // rows per point of this array
      const int m0 = sidx == 0 ? 0 : sidx == 1 ? 1 : 1 + D;
      const float* src = sidx == 0 ? gg : sidx == 1 ? gd : g2;
      if (!src) {  // absent upstream reads as zero
        for (int e = threadIdx.x; e < np * C * AF; e += kBlock) {
          const int row = e / AF, c = e - row * AF;
          const int i = row / C, m = m0 + row - i * C;
          tile[i * pitch + (c / F) * MF + m * F + c % F] = 0.0f;
        }
        continue;
      }
      const float4* s4 = reinterpret_cast<const float4*>(src + p0 * C * LF);
      const int total = np * C * q_row;
      for (int q0 = threadIdx.x; q0 < total; q0 += 4 * kBlock) {
        float4 v[4];
        int rowv[4], cv[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int q = q0 + u * kBlock;
          rowv[u] = q / q_row;
          cv[u] = 4 * (q - rowv[u] * q_row);
          if (q < total && cv[u] < AF) v[u] = s4[q];
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          if (q0 + u * kBlock >= total) break;
          if (cv[u] >= AF) continue;
          const int i = rowv[u] / C, m = m0 + rowv[u] - i * C;
          float* t = tile + i * pitch + m * F;
          const float e[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int l = (cv[u] + j) / F, f = (cv[u] + j) - l * F;
            t[l * MF + f] = e[j];
          }
        }
      }
    }
  } else {
    // one thread per (point, component) row of L*F floats
    for (int row = threadIdx.x; row < np * M; row += kBlock) {
      const int i = row / M, m = row - i * M;
      const int64_t p = p0 + i;
      const float* src = m == 0 ? (gg ? gg + p * LF : nullptr)
                       : m <= D ? (gd ? gd + (p * D + (m - 1)) * LF : nullptr)
                                : (g2 ? g2 + (p * D2 + (m - 1 - D)) * LF : nullptr);
      float* t = tile + i * pitch + m * F;
      for (int c = 0; c < AF; ++c) {
        const int l = c / F, f = c - l * F;
        t[l * MF + f] = src ? src[c] : 0.0f;
      }
    }
  }
  __syncthreads();
  for (int l = 0; l < L; ++l) {
    float* dst = U + ((int64_t)l * n + p0) * MF;
    for (int e = threadIdx.x; e < np * MF; e += kBlock) {
      const int i = e / MF, q = e - i * MF;
      dst[e] = tile[i * pitch + l * MF + q];
    }
  }
}

// The forward's level-major staging [l][p][m][F] -> gamma [n, L*F], dgamma [n, d, L*F],
// d2gamma [n, d2, L*F] (NULL outputs skipped).  A workgroup owns P consecutive points: it
// reads each level's P * M * F contiguous floats into LDS (each point's rows in output
// order, pitch M * L * F + 1) and writes the tile's rows of each output array, one
// contiguous block per array; both phases move consecutive 16-byte pieces across the lanes
// when the runs are 16-byte aligned, so every load and store instruction covers whole
// lines.  Rows are Lrow * F floats: the columns of the inactive levels L..Lrow-1 are
// written as zeros.
template <int F, int D, int M>
__global__ __launch_bounds__(kBlock) void hermite_levels_to_rows_kernel(int32_t L, int32_t Lrow, int64_t n,
                                                                        int32_t P,
                                                                        const float* __restrict__ stage,
                                                                        float* __restrict__ gamma,
                                                                        float* __restrict__ dgamma,
                                                                        float* __restrict__ d2gamma) {
  extern __shared__ float tile[];
  constexpr int MF = M * F;
  constexpr int D2 = M - 1 - D;
  const int LF = L * F;     // active floats of a row (LDS layout)
  const int RF = Lrow * F;  // output row stride
  const int pitch = M * LF + 1;
  const int64_t p0 = (int64_t)blockIdx.x * P;
  const int np = (int)min((int64_t)P, n - p0);
  // read phase: each level's run of the tile (np * MF floats) is contiguous; lanes take
  // consecutive 16-byte pieces, four loads in flight per lane before the LDS writes
  if (((n * MF) & 3) == 0 && ((np * MF) & 3) == 0 && ((P * MF) & 3) == 0) {
    const int q_per = (np * MF) >> 2;
    const int total = L * q_per;
    for (int q0 = threadIdx.x; q0 < total; q0 += 4 * kBlock) {
      float4 v[4];
      int lv[4], ev[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int q = q0 + u * kBlock;
        lv[u] = q / q_per;
        ev[u] = 4 * (q - lv[u] * q_per);  // float index inside the level's run
        if (q < total) v[u] = *reinterpret_cast<const float4*>(stage + ((int64_t)lv[u] * n + p0) * MF + ev[u]);
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if (q0 + u * kBlock >= total) break;
        const float e[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int i = (ev[u] + k) / MF, r = (ev[u] + k) - i * MF;
          const int m = r / F, f = r - m * F;
          tile[i * pitch + m * LF + lv[u] * F + f] = e[k];
        }
      }
    }
  } else {
    // one thread per (level, point): its M * F contiguous floats
    for (int pr = threadIdx.x; pr < L * np; pr += kBlock) {
      const int l = pr / np, i = pr - l * np;
      float v[MF];
      load_vec<MF>(stage + ((int64_t)l * n + p0 + i) * MF, v);
      float* t = tile + i * pitch + l * F;
#pragma unroll
      for (int m = 0; m < M; ++m)
#pragma unroll
        for (int f = 0; f < F; ++f) t[m * LF + f] = v[m * F + f];
    }
  }
  __syncthreads();
  // write phase: each output array's rows for the tile (np * C rows of RF floats, C components
  // per point) form one contiguous block; lanes write its consecutive 16-byte pieces
#pragma unroll
  for (int aidx = 0; aidx < 3; ++aidx) {
    const int C = aidx == 0 ? 1 : aidx == 1 ? D : D2;
    const int m0 = aidx == 0 ? 0 : aidx == 1 ? 1 : 1 + D;
    float* out = aidx == 0 ? gamma : aidx == 1 ? dgamma : d2gamma;
    if (!out) continue;
    float* dst = out + p0 * C * RF;
    if (((LF | RF) & 3) == 0) {
      const int qr = RF >> 2;  // pieces per row
      for (int q = threadIdx.x; q < np * C * qr; q += kBlock) {
        const int row = q / qr, c = 4 * (q - row * qr);
        const int i = row / C, m = m0 + row - i * C;
        const float* t = tile + i * pitch + m * LF;
        const float4 w = c < LF ? make_float4(t[c], t[c + 1], t[c + 2], t[c + 3]) : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        reinterpret_cast<float4*>(dst)[q] = w;
      }
    } else {
      for (int e = threadIdx.x; e < np * C * RF; e += kBlock) {
        const int row = e / RF, c = e - row * RF;
        const int i = row / C, m = m0 + row - i * C;
        dst[e] = c < LF ? tile[i * pitch + m * LF + c] : 0.0f;
      }
    }
  }
}

// Upstream of one point at one level from the level-major copy (the Laplacian upstream is
// the same for every diagonal term).
template <int D, int F>
__device__ __forceinline__ LevelUp<D, F> load_level_up_lm(const float* __restrict__ U, int64_t n, int64_t p, int l,
                                                          bool diag) {
  constexpr int MD = 1 + 2 * D;
  LevelUp<D, F> u;
  if (diag) {
    float v[MD * F];
    load_vec<MD * F>(U + ((int64_t)l * n + p) * MD * F, v);
#pragma unroll
    for (int f = 0; f < F; ++f) {
      u.v[f] = v[f];
#pragma unroll
      for (int i = 0; i < D; ++i) {
        u.g[i][f] = v[(1 + i) * F + f];
        u.h[i][f] = v[(1 + D + i) * F + f];
      }
    }
  } else {
    constexpr int ML = 2 + D;
    float v[ML * F];
    load_vec<ML * F>(U + ((int64_t)l * n + p) * ML * F, v);
#pragma unroll
    for (int f = 0; f < F; ++f) {
      u.v[f] = v[f];
#pragma unroll
      for (int i = 0; i < D; ++i) {
        u.g[i][f] = v[(1 + i) * F + f];
        u.h[i][f] = v[(1 + D) * F + f];
      }
    }
  }
  return u;
}

// u_levels: NULL, or the upstream level-major ([L][n][M][F]); then the row pointers are unused.
template <int D, int F>
__global__ __launch_bounds__(kBlock) void hermite_backward_kernel(
    const Grid g, int64_t n, int d2_mode, const float* __restrict__ x,
    const float* __restrict__ g_gamma, const float* __restrict__ g_dgamma,
    const float* __restrict__ g_d2gamma, const float* __restrict__ u_levels, float* __restrict__ grad) {
  const int64_t p = (int64_t)blockIdx.x * kBlock + threadIdx.x;
  if (p >= n) return;
  float xp[D];
#pragma unroll
  for (int i = 0; i < D; ++i) xp[i] = x[p * D + i];
  for (int l = 0; l < g.L; ++l) {
    const LevelUp<D, F> u = u_levels ? load_level_up_lm<D, F>(u_levels, n, p, l, d2_mode == HASHENC_D2_DIAG)
                                     : load_level_up<D, F>(g, p, l, d2_mode, g_gamma, g_dgamma, g_d2gamma);
    CellKeys<D> keys;
    AxisBasis ab[D];
    level_setup<D>(g, l, xp, keys, ab);
    AtomicSink<D, F> sink{g, keys};
#pragma unroll
    for (int k = 0; k < kMaxTables; ++k) {
      sink.base[k] = grad + (k <= D ? g.off[k][l] : 0);
      sink.dense[k] = (g.dense[k] >> l) & 1u;
    }
    bwd_pair<D, F, 0>(sink, ab, u);
    bwd_pair<D, F, 1>(sink, ab, u);
    if constexpr (D == 3) {
      bwd_pair<D, F, 2>(sink, ab, u);
      bwd_pair<D, F, 3>(sink, ab, u);
    }
  }
}

// End of a count workgroup: its LDS histogram becomes the tile's row of per-bin counts for
// levels l0..l1 of every order table.  A fine histogram (equal table sizes) gives each table's
// bin counts as sums of consecutive fine bins.
__device__ __forceinline__ void store_tile_counts(const BinPlan& bp, int l0, int l1, bool fine,
                                                  const int32_t* hist, int32_t* __restrict__ row) {
  if (!fine) {
    for (int k = 0; k < bp.ntab; ++k)
      for (int i = bp.seg_bin0[k * bp.L + l0] + threadIdx.x; i < bp.seg_bin0[k * bp.L + l1]; i += kBinThreads)
        row[i] = hist[i];
    return;
  }
  for (int sg = 0; sg < bp.nseg; ++sg) {
    const int k = sg / bp.L, l = sg % bp.L;
    if (l < l0 || l >= l1) continue;
    const int ratio_shift = bp.cshift[k] - bp.fine_shift;
    const int32_t f0 = bp.fine_bin0[l], f1 = bp.fine_bin0[l + 1];
    const int32_t b0 = bp.seg_bin0[sg], nb = bp.seg_bin0[sg + 1] - b0;
    for (int jb = threadIdx.x; jb < nb; jb += kBinThreads) {
      const int32_t lo = f0 + (jb << ratio_shift);
      const int32_t hi = min(f1, f0 + ((jb + 1) << ratio_shift));
      int32_t c = 0;
      for (int i = lo; i < hi; ++i) c += hist[i];
      row[b0 + jb] = c;
    }
  }
}

// Binned backward, count pass: a workgroup histograms the entries of its tile of `tile`
// points (one per corner and order table) at its group of lpg levels (blockIdx.y) in LDS.
// With equal table sizes (bp.fine_shift >= 0) the rows are histogrammed once per level in
// fine chunks and each table's bin counts are sums of consecutive fine bins.
template <int D>
__global__ __launch_bounds__(kBinThreads) void hermite_count_kernel(const Grid g, const BinPlan bp, int64_t n,
                                                                    int32_t tile, int32_t nblk, int32_t lpg,
                                                                    const float* __restrict__ x,
                                                                    int32_t* __restrict__ counts) {
  extern __shared__ int32_t hist[];
  const int blk = bin_tile_of_block(blockIdx.x, nblk);
  const int l0 = blockIdx.y * lpg, l1 = min(g.L, l0 + lpg);
  const bool fine = bp.fine_shift >= 0;
  const int nh = fine ? bp.fine_bin0[g.L] : bp.nbins;
  for (int i = threadIdx.x; i < nh; i += kBinThreads) hist[i] = 0;
  __syncthreads();
  for (int j = threadIdx.x; j < tile; j += kBinThreads) {
    const int64_t p = (int64_t)blk * tile + j;
    if (p >= n) break;
    float xp[D];
#pragma unroll
    for (int i = 0; i < D; ++i) xp[i] = x[p * D + i];
    for (int l = l0; l < l1; ++l) {
      uint32_t base[D];
      float t[D];
      locate<D>(xp, g.N[l], g.Nf[l], base, t);
      const CellKeys<D> keys = cell_keys<D>(base, g.N[l]);
      if (fine) {
        const bool dense = (g.dense[0] >> l) & 1u;
        const bool few = bp.fine_bin0[l + 1] - bp.fine_bin0[l] <= kFewBins;
        // x-corner pairs (Y, Y | 1) usually share a bin: one LDS atomic of 2 then
        [&]<int... Y>(std::integer_sequence<int, Y...>) {
          ((
               [&] {
                 const int32_t b0 = bp.fine_bin0[l] +
                                    (int32_t)(corner_row<D, (Y << 1)>(keys, dense, g.T[0], g.Tmask[0]) >> bp.fine_shift);
                 const int32_t b1 = bp.fine_bin0[l] + (int32_t)(corner_row<D, (Y << 1) | 1>(keys, dense, g.T[0],
                                                                                              g.Tmask[0]) >>
                                                                bp.fine_shift);
                 if (few) {
                   wave_aggregated_add<false>(hist, b0);
                   wave_aggregated_add<false>(hist, b1);
                 } else if (b0 == b1) {
                   atomicAdd(&hist[b0], 2);
                 } else {
                   atomicAdd(&hist[b0], 1);
                   atomicAdd(&hist[b1], 1);
                 }
               }()),
           ...);
        }(std::make_integer_sequence<int, 1 << (D - 1)>{});
        continue;
      }
#pragma unroll
      for (int k = 0; k <= D; ++k) {
        const bool dense = (g.dense[k] >> l) & 1u;
        const bool few = bp.seg_bin0[k * bp.L + l + 1] - bp.seg_bin0[k * bp.L + l] <= kFewBins;
        [&]<int... C>(std::integer_sequence<int, C...>) {
          ((
               [&] {
                 int32_t bin;
                 uint32_t local;
                 bin_of(bp, k, l, corner_row<D, C>(keys, dense, g.T[k], g.Tmask[k]), bin, local);
                 if (few) wave_aggregated_add<false>(hist, bin);
                 else atomicAdd(&hist[bin], 1);
               }()),
           ...);
        }(std::make_integer_sequence<int, 1 << D>{});
      }
    }
  }
  __syncthreads();
  store_tile_counts(bp, l0, l1, fine, hist, counts + (int64_t)blk * bp.nbins);
}

// LDS layout of the Hermite scatter workgroup (P points).  The bins of one level's segments
// (order tables in turn) are held side by side.
template <int D, int F, int P>
struct HScatterLds {
  int32_t* delta;   // [max_level_bins] slot s of a bin goes to entry delta + s
  int32_t* lcur;    // [max_level_bins] slot cursors: the tile's exclusive prefix over the level
  int32_t* wsum;    // [P / 64]
  float* st_rec;    // [P * 2^D * widest staged record]
  __device__ HScatterLds(int32_t* lds, int mb) {
    delta = lds;
    lcur = lds + mb;
    wsum = lds + 2 * mb;
    st_rec = reinterpret_cast<float*>(lds + ((2 * mb + P / 64 + 3) & ~3));  // 16-byte aligned
  }
};

// Per level: the tile's slot ranges in every bin of the level's segments, from the count
// pass (one round of global reads per level rather than one per order table).  The level's
// bins (order tables in turn) are numbered 0 .. lo; bin i is read by thread i % P into
// register slot i / P (NPB slots; bins past NPB * P are read when applied).  Loading and
// applying are separate so that the next level's reads can be issued a level ahead: waiting
// for them then does not wait for the record stores issued in between.
template <int NPB>
struct LevelBinRegs {
  int32_t start[NPB], cur[NPB], nxt[NPB];
};

// global bin of level-bin i (order tables in turn), or -1 past the level's bins
template <int D>
__device__ __forceinline__ int32_t level_bin_global(const BinPlan& bp, int l, int i) {
  int lo = 0;
#pragma unroll
  for (int k = 0; k <= D; ++k) {
    const int32_t b0 = bp.seg_bin0[k * bp.L + l];
    const int nb = bp.seg_bin0[k * bp.L + l + 1] - b0;
    if (i < lo + nb) return b0 + (i - lo);
    lo += nb;
  }
  return -1;
}

template <int D, int P, int NPB>
__device__ __forceinline__ void level_bins_load(const BinPlan& bp, int l, int blk, int nblk,
                                                const int32_t* __restrict__ counts,
                                                const int32_t* __restrict__ totals,
                                                const int32_t* __restrict__ bin_start, LevelBinRegs<NPB>& r) {
#pragma unroll
  for (int q = 0; q < NPB; ++q) {
    const int32_t b = level_bin_global<D>(bp, l, threadIdx.x + q * P);
    if (b >= 0) {
      r.start[q] = bin_start[b];
      r.cur[q] = counts[(int64_t)blk * bp.nbins + b];
      r.nxt[q] = blk + 1 < nblk ? counts[(int64_t)(blk + 1) * bp.nbins + b] : totals[b];
    }
  }
}

// base[k]: the first slot of table k, so that table k's records take staging slots
// 0 .. np * NC.
template <int D, int P, int NPB>
__device__ __forceinline__ void level_bins_apply(const BinPlan& bp, int l, int blk, int nblk,
                                                 const int32_t* __restrict__ counts,
                                                 const int32_t* __restrict__ totals,
                                                 const int32_t* __restrict__ bin_start, const LevelBinRegs<NPB>& r,
                                                 int32_t* delta, int32_t* lcur, int32_t* wsum, int32_t (&base)[D + 1]) {
  int lo = 0;
#pragma unroll
  for (int k = 0; k <= D; ++k) lo += bp.seg_bin0[k * bp.L + l + 1] - bp.seg_bin0[k * bp.L + l];
#pragma unroll
  for (int q = 0; q < NPB; ++q) {
    const int i = threadIdx.x + q * P;
    if (i < lo) {
      delta[i] = r.start[q] + r.cur[q];
      lcur[i] = r.nxt[q] - r.cur[q];
    }
  }
  for (int i = threadIdx.x + NPB * P; i < lo; i += P) {  // bins beyond the register slots
    const int32_t b = level_bin_global<D>(bp, l, i);
    const int32_t pre = counts[(int64_t)blk * bp.nbins + b];
    const int32_t nxt = blk + 1 < nblk ? counts[(int64_t)(blk + 1) * bp.nbins + b] : totals[b];
    delta[i] = bin_start[b] + pre;
    lcur[i] = nxt - pre;
  }
  __syncthreads();
  block_exclusive_scan<P>(lcur, lo, wsum);
  for (int i = threadIdx.x; i < lo; i += P) delta[i] -= lcur[i];
  lo = 0;
#pragma unroll
  for (int k = 0; k <= D; ++k) {
    base[k] = lcur[lo];  // before any cursor moves
    lo += bp.seg_bin0[k * bp.L + l + 1] - bp.seg_bin0[k * bp.L + l];
  }
  __syncthreads();
}

template <int D, int P>
__device__ __forceinline__ void hermite_level_bins(const BinPlan& bp, int l, int blk, int nblk,
                                                   const int32_t* __restrict__ counts,
                                                   const int32_t* __restrict__ totals,
                                                   const int32_t* __restrict__ bin_start, int32_t* delta,
                                                   int32_t* lcur, int32_t* wsum, int32_t (&base)[D + 1]) {
  LevelBinRegs<1> r;
  level_bins_load<D, P, 1>(bp, l, blk, nblk, counts, totals, bin_start, r);
  level_bins_apply<D, P, 1>(bp, l, blk, nblk, counts, totals, bin_start, r, delta, lcur, wsum, base);
}

// Stage the two records of corner pair (0, Y) for order table K.  lo_k: the table's first bin
// in the level's LDS arrays; b0: its first global bin.
template <int D, int F, int K, int Y>
__device__ __forceinline__ void stage_pair(const Grid& g, const BinPlan& bp, int l, bool dense, bool few,
                                           int32_t b0, int lo_k, int32_t base, const CellKeys<D>& keys,
                                           const AxisBasis (&ab)[D], const LevelUp<D, F>& u, int32_t* lcur,
                                           const int32_t* delta, float* st_rec, float& vmx) {
  constexpr int W = binom_d(D, K) * F;
  constexpr int R = hermite_rec_width(W);
  constexpr int RS = hermite_stage_width(W);
  float v[2][W];
  bwd_pair_table<D, F, Y, K>(ab, u, v[0], v[1]);
#pragma unroll
  for (int j = 0; j < W; ++j) vmx = fmaxf(vmx, fmaxf(fabsf(v[0][j]), fabsf(v[1][j])));
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    int32_t bin;
    uint32_t local;
    const uint32_t row = h ? corner_row<D, (Y << 1) | 1>(keys, dense, g.T[K], g.Tmask[K])
                           : corner_row<D, (Y << 1)>(keys, dense, g.T[K], g.Tmask[K]);
    bin_of(bp, K, l, row, bin, local);
    const int i = lo_k + (bin - b0);
    const int32_t slot = few ? wave_aggregated_add<true>(lcur + lo_k, bin - b0) : atomicAdd(&lcur[i], 1);
    const int32_t lp = slot - base;
    float rec[RS];
    rec[0] = __uint_as_float(local);
#pragma unroll
    for (int j = 0; j < W; ++j) rec[1 + j] = v[h][j];
    rec[R] = __int_as_float(delta[i] + slot);  // the record's entry in the segment
#pragma unroll
    for (int j = R + 1; j < RS; ++j) rec[j] = 0.0f;
    store_vec<RS>(st_rec + (int64_t)lp * RS, rec);
  }
}

// One (level, order table K) phase of the scatter workgroup: stage the tile's table-K
// records sorted by bin, then copy them out.
template <int D, int F, int P, int K>
__device__ __forceinline__ void scatter_table(const Grid& g, const BinPlan& bp, int l, bool on, int np, int lo_k,
                                              int32_t base, const CellKeys<D>& keys, const AxisBasis (&ab)[D],
                                              const LevelUp<D, F>& u, const BinState* __restrict__ st,
                                              float* __restrict__ vals_out, const HScatterLds<D, F, P>& sh,
                                              uint32_t* vsh, uint32_t nf) {
  constexpr int W = binom_d(D, K) * F;
  constexpr int R = hermite_rec_width(W);
  constexpr int RS = hermite_stage_width(W);
  constexpr int NC = 1 << D;
  const int sg = K * bp.L + l;
  const int32_t b0 = bp.seg_bin0[sg];
  const int nb = bp.seg_bin0[sg + 1] - b0;
  const bool dense = (g.dense[K] >> l) & 1u;
  const bool few = nb <= kFewBins;
  float vmx = 0.0f;  // largest |value| of this lane's records (NaN values aside: nf)
  if (on) {
    stage_pair<D, F, K, 0>(g, bp, l, dense, few, b0, lo_k, base, keys, ab, u, sh.lcur, sh.delta, sh.st_rec, vmx);
    stage_pair<D, F, K, 1>(g, bp, l, dense, few, b0, lo_k, base, keys, ab, u, sh.lcur, sh.delta, sh.st_rec, vmx);
    if constexpr (D == 3) {
      stage_pair<D, F, K, 2>(g, bp, l, dense, few, b0, lo_k, base, keys, ab, u, sh.lcur, sh.delta, sh.st_rec, vmx);
      stage_pair<D, F, K, 3>(g, bp, l, dense, few, b0, lo_k, base, keys, ab, u, sh.lcur, sh.delta, sh.st_rec, vmx);
    }
  }
  raise_seg_vmax(vsh, sg, max(__float_as_uint(vmx), nf));
  __syncthreads();
  const int32_t ebase = st->seg_ebase[sg];
  float* vseg = vals_out + st->seg_vbase[sg];
  // copy out one record per lane: consecutive lanes hold consecutive records of a bin's run,
  // so the R stores of a wavefront fill the run's lines between them (a word per lane, for
  // whole-line stores, measured slower)
  const int32_t recs = np * NC;
  auto put = [&](const float (&v)[RS]) {
    float* dst = vseg + (int64_t)(__float_as_int(v[R]) - ebase) * R;
#pragma unroll
    for (int j = 0; j < R; ++j) dst[j] = v[j];
  };
  int32_t q = threadIdx.x;
  for (; q + P < recs; q += 2 * P) {  // two records' LDS reads in flight before their stores
    float v0[RS], v1[RS];
    load_vec<RS>(sh.st_rec + (int64_t)q * RS, v0);
    load_vec<RS>(sh.st_rec + (int64_t)(q + P) * RS, v1);
    put(v0);
    put(v1);
  }
  if (q < recs) {
    float v[RS];
    load_vec<RS>(sh.st_rec + (int64_t)q * RS, v);
    put(v);
  }
  __syncthreads();
}

// Binned backward, scatter pass.  One lane per point of a P-point tile.  Per level the tile's
// slot ranges in all of the level's bins are set up at once; then per order table K the
// tile's records {local row, W values} are computed (table K's part of the pair reverse),
// sorted by bin in LDS and copied out as flat words: consecutive lanes write consecutive
// words of each bin's contiguous run, so lines are written whole apart from run ends.
template <int D, int F, int P>
__global__ __launch_bounds__(P) void hermite_scatter_kernel(
    const Grid g, const BinPlan bp, int64_t n, int32_t nblk, int32_t lpg, bool diag, const float* __restrict__ x,
    const float* __restrict__ U, const int32_t* __restrict__ counts,
    const int32_t* __restrict__ totals, const int32_t* __restrict__ bin_start,
    const BinState* __restrict__ st, float* __restrict__ vals_out, uint32_t* __restrict__ vmax) {
  extern __shared__ int32_t lds[];
  const HScatterLds<D, F, P> sh(lds, bp.max_level_bins);
  __shared__ uint32_t vsh[kMaxSeg];  // the workgroup's segment bounds
  for (int i = threadIdx.x; i < kMaxSeg; i += P) vsh[i] = 0u;
  __syncthreads();
  const int blk = bin_tile_of_block(blockIdx.x, nblk);
  const int64_t p = (int64_t)blk * P + threadIdx.x;
  const bool on = p < n;
  const int np = (int)min((int64_t)P, n - (int64_t)blk * P);
  float xp[D];
#pragma unroll
  for (int i = 0; i < D; ++i) xp[i] = on ? x[p * D + i] : 0.0f;
  const int l0 = blockIdx.y * lpg, l1 = min(g.L, l0 + lpg);  // this workgroup's levels
  // the next level's upstream and bin ranges are loaded while this level's records are
  // staged and stored
  constexpr int NPB = 2;
  LevelUp<D, F> un;
  LevelBinRegs<NPB> rn;
  if (l0 < l1) {
    if (on) un = load_level_up_lm<D, F>(U, n, p, l0, diag);
    level_bins_load<D, P, NPB>(bp, l0, blk, nblk, counts, totals, bin_start, rn);
  }
  for (int l = l0; l < l1; ++l) {
    const LevelUp<D, F> u = un;
    // NaN bound for the level's segments unless its values are finite
    const uint32_t nf = on ? hermite_nonfinite_floor(level_up_absmax<D, F>(u), g.Nf[l], D) : 0u;
    int32_t base[D + 1];
    level_bins_apply<D, P, NPB>(bp, l, blk, nblk, counts, totals, bin_start, rn, sh.delta, sh.lcur, sh.wsum, base);
    if (l + 1 < l1) {
      if (on) un = load_level_up_lm<D, F>(U, n, p, l + 1, diag);
      level_bins_load<D, P, NPB>(bp, l + 1, blk, nblk, counts, totals, bin_start, rn);
    }
    CellKeys<D> keys;
    AxisBasis ab[D];
    if (on) level_setup<D>(g, l, xp, keys, ab);
    int lo = 0;
    scatter_table<D, F, P, 0>(g, bp, l, on, np, lo, base[0], keys, ab, u, st, vals_out, sh, vsh, nf);
    lo += bp.seg_bin0[l + 1] - bp.seg_bin0[l];
    scatter_table<D, F, P, 1>(g, bp, l, on, np, lo, base[1], keys, ab, u, st, vals_out, sh, vsh, nf);
    lo += bp.seg_bin0[bp.L + l + 1] - bp.seg_bin0[bp.L + l];
    scatter_table<D, F, P, 2>(g, bp, l, on, np, lo, base[2], keys, ab, u, st, vals_out, sh, vsh, nf);
    if constexpr (D == 3) {
      lo += bp.seg_bin0[2 * bp.L + l + 1] - bp.seg_bin0[2 * bp.L + l];
      scatter_table<D, F, P, 3>(g, bp, l, on, np, lo, base[3], keys, ab, u, st, vals_out, sh, vsh, nf);
    }
  }
  __syncthreads();
  publish_seg_vmax(vsh, bp.nseg, vmax);
}

template <int D, int F>
hipError_t launch_bin(const Grid& g, const BinPlan& bp, const BinWorkspace& w, char* ws, int d2_mode,
                      bool scatter, int64_t n, const float* x, const float* gg, const float* gd,
                      const float* g2, const float* u_levels, hipStream_t s) {
  const dim3 grid((unsigned)w.nblk, (unsigned)w.lgroups);
  int32_t* counts = reinterpret_cast<int32_t*>(ws + w.counts);
  if (!scatter) {
    const size_t hist = sizeof(int32_t) * (size_t)(bp.fine_shift >= 0 ? bp.fine_bin0[g.L] : bp.nbins);
    hipLaunchKernelGGL((hermite_count_kernel<D>), grid, dim3(kBinThreads), hist, s,
                       g, bp, n, w.tile, w.nblk, w.lpg, x, counts);
    return hipGetLastError();
  }
  constexpr int P = hermite_scatter_points(F);
  if (w.tile != P) return hipErrorInvalidValue;
  const size_t lds = hermite_scatter_lds_bytes(bp, D, F);
  const int32_t* totals = reinterpret_cast<const int32_t*>(ws + w.totals);
  const int32_t* bin_start = reinterpret_cast<const int32_t*>(ws + w.bin_start);
  const BinState* st = reinterpret_cast<const BinState*>(ws + w.state);
  float* vals = reinterpret_cast<float*>(ws + w.vals);
  // upstream rearranged level-major for the level-by-level scatter (unless given so)
  const bool diag = d2_mode == HASHENC_D2_DIAG;
  const int M = 1 + D + (diag ? D : 1);
  const int LF = g.L * F;
  const int PU = (int)std::max(1, std::min(32, 8192 / (M * LF)));  // LDS tile <= 32 KB: several workgroups per CU
  const float* U = u_levels ? u_levels : reinterpret_cast<const float*>(ws + w.ups);
  float* Uw = reinterpret_cast<float*>(ws + w.ups);
  const size_t ulds = sizeof(float) * (size_t)PU * (M * LF + 1);
  const void* ukern = diag ? reinterpret_cast<const void*>(&hermite_upstream_levels_kernel<F, D, 1 + 2 * D>)
                           : reinterpret_cast<const void*>(&hermite_upstream_levels_kernel<F, D, 2 + D>);
  hipError_t e = hipSuccess;
  if (!u_levels) {
    e = hipFuncSetAttribute(ukern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)ulds);
    if (e != hipSuccess) return e;
    const dim3 ugrid((unsigned)((n + PU - 1) / PU));
    if (diag)
      hipLaunchKernelGGL((hermite_upstream_levels_kernel<F, D, 1 + 2 * D>), ugrid, dim3(kBlock), ulds, s, g.L,
                         g.Lrow, n, PU, gg, gd, g2, Uw);
    else
      hipLaunchKernelGGL((hermite_upstream_levels_kernel<F, D, 2 + D>), ugrid, dim3(kBlock), ulds, s, g.L, g.Lrow,
                         n, PU, gg, gd, g2, Uw);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  e = hipFuncSetAttribute(reinterpret_cast<const void*>(&hermite_scatter_kernel<D, F, P>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((hermite_scatter_kernel<D, F, P>), grid, dim3(P), lds, s, g, bp, n, w.nblk, w.lpg, diag, x, U,
                     counts, totals, bin_start, st, vals,
                     reinterpret_cast<BinState*>(ws + w.state)->vmax_bits);
  return hipGetLastError();
}

PackPlan make_pack_plan(const Grid& g, int d, int F) {
  PackPlan pp;
  pp.poff[0] = 0;
  for (int l = 0; l < g.L; ++l) {
    int64_t rows = g.T[0];
    if ((g.dense[0] >> l) & 1u) {
      rows = 1;
      for (int i = 0; i < d; ++i) rows *= (int64_t)g.N[l] + 1;
    }
    pp.poff[l + 1] = pp.poff[l] + rows * ((int64_t)1 << d) * F;
  }
  return pp;
}

template <int D, int F>
hipError_t launch_pack(const Grid& g, const float* params, float* packed, hipStream_t s) {
  const PackPlan pp = make_pack_plan(g, D, F);
  const int64_t rows = pp.poff[g.L] / ((1 << D) * F);
  hipLaunchKernelGGL((hermite_pack_kernel<D, F>), dim3((unsigned)((rows + kBlock - 1) / kBlock)), dim3(kBlock), 0, s,
                     g, pp, params, packed);
  return hipGetLastError();
}

// stage: NULL for point-major outputs; else the level-major staging buffer, and when
// to_rows also the rearrangement into gamma / dgamma / d2gamma
template <int D, int F>
hipError_t launch_fwd(const Grid& g, int d2_mode, int64_t n, const float* x, const float* params,
                      const float* packed, float* stage, bool to_rows, float* gamma, float* dgamma,
                      float* d2gamma, hipStream_t s) {
  const int64_t tiles = (n + kBlock / 2 - 1) / (kBlock / 2);  // two lanes per point
  if (tiles * g.L > 0x7fffffff) return hipErrorInvalidValue;
  const dim3 grid((unsigned)(tiles * g.L));
  const PackPlan pp = make_pack_plan(g, D, F);
  const float* tab = packed ? packed : params;
  if (packed && stage)
    hipLaunchKernelGGL((hermite_forward_kernel<D, F, true, true>), grid, dim3(kBlock), 0, s, g, pp, n,
                       (int32_t)tiles, d2_mode, x, tab, gamma, dgamma, d2gamma, stage);
  else if (packed)
    hipLaunchKernelGGL((hermite_forward_kernel<D, F, true, false>), grid, dim3(kBlock), 0, s, g, pp, n,
                       (int32_t)tiles, d2_mode, x, tab, gamma, dgamma, d2gamma, stage);
  else if (stage)
    hipLaunchKernelGGL((hermite_forward_kernel<D, F, false, true>), grid, dim3(kBlock), 0, s, g, pp, n,
                       (int32_t)tiles, d2_mode, x, tab, gamma, dgamma, d2gamma, stage);
  else
    hipLaunchKernelGGL((hermite_forward_kernel<D, F, false, false>), grid, dim3(kBlock), 0, s, g, pp, n,
                       (int32_t)tiles, d2_mode, x, tab, gamma, dgamma, d2gamma, stage);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || (stage && !to_rows)) return e;
  const bool diag = d2_mode == HASHENC_D2_DIAG;
  if (!stage) {  // point-major outputs: zero the inactive levels' columns
    if (g.L == g.Lrow) return e;
    const int RF = g.Lrow * F, AF = g.L * F;
    if (gamma) e = launch_zero_columns(gamma, n, RF, AF, s);
    if (e == hipSuccess && dgamma) e = launch_zero_columns(dgamma, n * D, RF, AF, s);
    if (e == hipSuccess && d2gamma) e = launch_zero_columns(d2gamma, n * (diag ? D : 1), RF, AF, s);
    return e;
  }
  const int M = 1 + D + (diag ? D : 1);
  const int LF = g.L * F;
  const int P = (int)std::max(1, std::min(32, 8192 / (M * LF)));  // LDS tile <= 32 KB: several workgroups per CU
  const size_t lds = sizeof(float) * (size_t)P * (M * LF + 1);
  const void* kern = diag ? reinterpret_cast<const void*>(&hermite_levels_to_rows_kernel<F, D, 1 + 2 * D>)
                          : reinterpret_cast<const void*>(&hermite_levels_to_rows_kernel<F, D, 2 + D>);
  e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  const dim3 tgrid((unsigned)((n + P - 1) / P));
  if (diag)
    hipLaunchKernelGGL((hermite_levels_to_rows_kernel<F, D, 1 + 2 * D>), tgrid, dim3(kBlock), lds, s, g.L, g.Lrow,
                       n, P, stage, gamma, dgamma, d2gamma);
  else
    hipLaunchKernelGGL((hermite_levels_to_rows_kernel<F, D, 2 + D>), tgrid, dim3(kBlock), lds, s, g.L, g.Lrow, n,
                       P, stage, gamma, dgamma, d2gamma);
  return hipGetLastError();
}

template <int D, int F>
hipError_t launch_bwd(const Grid& g, int d2_mode, int64_t n, const float* x, const float* gg,
                      const float* gd, const float* gdd, const float* u_levels, float* grad, hipStream_t s) {
  const dim3 grid((unsigned)((n + kBlock - 1) / kBlock));
  hipLaunchKernelGGL((hermite_backward_kernel<D, F>), grid, dim3(kBlock), 0, s, g, n, d2_mode, x,
                     gg, gd, gdd, u_levels, grad);
  return hipGetLastError();
}

// ------------------------------------------------------------------ space-time (d = 4)
// Hermite-NGP notes, section 局限与展望: in 4D the 2^d coefficients per vertex become 16, in
// five order tables (1, 4, 6, 4, 1 slots of F floats).  One lane per (point, level), level-major
// workgroups.  Per corner the 16 coefficients form a 2x2x2x2 tensor over the derivative bits;
// the forward contracts it with the per-axis bases one axis at a time (w, z, y, x), carrying
// only the derivative kinds that survive (value; first and second derivative along each axis
// already passed): 3 -> 5 -> 7 -> 9 results.  The backward runs the same contraction
// transposed, per coefficient, and either scatter-adds with fp32 atomics or writes binned
// records (one per point, level, corner and order table) for the binned reduce.
constexpr uint32_t kPrime3 = 3674653429u;

// alpha (bit i = derivative along axis i) of slot s of order table k, slots of one order in
// lexicographic order of their axis tuples
__host__ __device__ constexpr int alpha4_of_slot(int k, int s) {
  constexpr int o1[4] = {1, 2, 4, 8};
  constexpr int o2[6] = {3, 5, 9, 6, 10, 12};
  constexpr int o3[4] = {7, 11, 13, 14};
  return k == 0 ? 0 : k == 1 ? o1[s] : k == 2 ? o2[s] : k == 3 ? o3[s] : 15;
}
__host__ __device__ constexpr int slots4(int k) { return k == 0 || k == 4 ? 1 : k == 2 ? 6 : 4; }

// Corner rows of a cell from its base vertex: dense row dense0 + sum of the strides of the
// corner's bits, hashed XOR of the four per-axis terms.  Every choice by a corner bit is a
// select between two computed values (no indexing by a run-time bit, which would put the
// operands in scratch memory).
struct Keys4 {
  uint32_t dense0, s1, s2, s3;
  uint32_t h0, h1, h2, h3;  // per-axis hash terms of the base vertex
};

__device__ __forceinline__ Keys4 keys4(const uint32_t (&base)[4], int32_t N) {
  Keys4 k;
  const uint32_t N1 = (uint32_t)N + 1u;
  k.s1 = N1;
  k.s2 = N1 * N1;
  k.s3 = N1 * N1 * N1;
  k.dense0 = base[0] + base[1] * k.s1 + base[2] * k.s2 + base[3] * k.s3;
  k.h0 = base[0];
  k.h1 = base[1] * kPrime1;
  k.h2 = base[2] * kPrime2;
  k.h3 = base[3] * kPrime3;
  return k;
}

__device__ __forceinline__ uint32_t row4(const Keys4& k, int c, bool dense, uint32_t T, uint32_t Tmask) {
  const bool b0 = c & 1, b1 = (c >> 1) & 1, b2 = (c >> 2) & 1, b3 = (c >> 3) & 1;
  if (dense)
    return k.dense0 + (b0 ? 1u : 0u) + (b1 ? k.s1 : 0u) + (b2 ? k.s2 : 0u) + (b3 ? k.s3 : 0u);
  const uint32_t h = (b0 ? k.h0 + 1u : k.h0) ^ (b1 ? k.h1 + kPrime1 : k.h1) ^ (b2 ? k.h2 + kPrime2 : k.h2) ^
                     (b3 ? k.h3 + kPrime3 : k.h3);
  return Tmask ? (h & Tmask) : (h % T);
}

// The bases of one corner along one axis, indexed by the derivative bit: b[a] value basis,
// d[a] its x-derivative, d2[a] its second x-derivative; the same expressions as axis_basis,
// computed here for the corner bit chosen at run time.
struct CornerAxis {
  float b[2], d[2], d2[2];
};

__device__ __forceinline__ CornerAxis corner_axis(float t, float N, float invN, bool far) {
  const float s = 1.0f - t;
  const float t2 = t * t;
  const float h00 = (1.0f + 2.0f * t) * s * s, h00p = -6.0f * t * s, h00pp = 12.0f * t - 6.0f;
  const float h10 = t * s * s, h10p = s * (1.0f - 3.0f * t), h10pp = 6.0f * t - 4.0f;
  const float h01 = t2 * (3.0f - 2.0f * t);
  const float h11 = -t2 * s, h11p = t * (3.0f * t - 2.0f), h11pp = 6.0f * t - 2.0f;
  const float N2 = N * N;
  CornerAxis r;
  r.b[0] = far ? h01 : h00;
  r.b[1] = invN * (far ? h11 : h10);
  r.d[0] = far ? -N * h00p : N * h00p;
  r.d[1] = far ? h11p : h10p;
  r.d2[0] = far ? -N2 * h00pp : N2 * h00pp;
  r.d2[1] = N * (far ? h11pp : h10pp);
  return r;
}

// Packed copy of the five order tables for d = 4: packed row t of level l (t counts the
// order-0 table's rows) holds the vertex's rows of tables 0..4 side by side (16 F floats).
// A smaller power-of-two table's row follows from the order-0 row as in the 2D / 3D packing
// (a dense order-0 row names its vertex, which is hashed with the four primes).  Rows go
// through LDS and out as 16-byte pieces, whole lines per store instruction.
template <int F>
__global__ __launch_bounds__(kBlock) void hermite4_pack_kernel(const Grid g, const PackPlan pp,
                                                               const float* __restrict__ params,
                                                               float* __restrict__ packed) {
  constexpr int RW = 16 * F;
  constexpr int PITCH = RW + 4;
  __shared__ float stage[kBlock * PITCH];
  const int64_t total = pp.poff[g.L] / RW;
  const int64_t t0 = (int64_t)blockIdx.x * kBlock;
  const int64_t t = t0 + threadIdx.x;
  if (t < total) {
    int l = 0;
    while (l + 1 < g.L && t * RW >= pp.poff[l + 1]) ++l;
    const int64_t r = t - pp.poff[l] / RW;
    auto row_in = [&](int k) -> int64_t {
      if (g.T[k] == g.T[0]) return r;
      if (!((g.dense[0] >> l) & 1u)) return r & (int64_t)(g.T[k] - 1);  // both hashed, T_k | T_0
      if ((g.dense[k] >> l) & 1u) return r;                                // both dense
      const int64_t N1 = (int64_t)g.N[l] + 1;                              // dense row -> vertex
      const uint32_t h = (uint32_t)(r % N1) ^ (uint32_t)((r / N1) % N1) * kPrime1 ^
                         (uint32_t)((r / (N1 * N1)) % N1) * kPrime2 ^ (uint32_t)(r / (N1 * N1 * N1)) * kPrime3;
      return h & (g.T[k] - 1u);
    };
    float v[RW];
    int o = 0;
#pragma unroll
    for (int k = 0; k <= 4; ++k) {
      const int W = slots4(k) * F;
      const float* src = params + g.off[k][l] + row_in(k) * W;
#pragma unroll
      for (int j = 0; j < slots4(k) * F; ++j) v[o + j] = src[j];
      o += W;
    }
    store_vec<RW>(stage + threadIdx.x * PITCH, v);
  }
  __syncthreads();
  const int nr = (int)(total - t0 < kBlock ? total - t0 : kBlock);
  constexpr int Q = RW / 4;
  float4* dst = reinterpret_cast<float4*>(packed + t0 * RW);
  for (int q = threadIdx.x; q < nr * Q; q += kBlock) {
    const int row = q / Q, cq = q - row * Q;
    dst[q] = *reinterpret_cast<const float4*>(stage + row * PITCH + 4 * cq);
  }
}

// PACKED: the 16 coefficients of a vertex are read as one row of the packed copy (five order
// tables side by side, 16 F contiguous floats: one 128-byte line at F = 2) instead of one row
// of each of the five tables.
template <int F, bool PACKED>
__global__ __launch_bounds__(kBlock) void hermite4_forward_kernel(const Grid g, const PackPlan pp, int64_t n,
                                                                  int32_t n_tiles, int d2_mode,
                                                                  const float* __restrict__ x,
                                                                  const float* __restrict__ params,
                                                                  float* __restrict__ gamma,
                                                                  float* __restrict__ dgamma,
                                                                  float* __restrict__ d2gamma) {
  constexpr int D = 4;
  const int l = blockIdx.x / n_tiles;
  const int64_t p = (int64_t)(blockIdx.x % n_tiles) * kBlock + threadIdx.x;
  if (p >= n) return;
  float xp[D];
#pragma unroll
  for (int i = 0; i < D; ++i) xp[i] = x[p * D + i];
  uint32_t base[D];
  float t[D];
  locate<D>(xp, g.N[l], g.Nf[l], base, t);
  const float Nf = g.Nf[l], iN = g.invN[l];
  const Keys4 keys = keys4(base, g.N[l]);
  // results: 0 value, 1 + i first derivative along i, 5 + i second derivative along i
  float out[9][F];
#pragma unroll
  for (int r = 0; r < 9; ++r)
#pragma unroll
    for (int f = 0; f < F; ++f) out[r][f] = 0.0f;
#pragma unroll 1
  for (int c = 0; c < 16; ++c) {
    // the corner's 16 coefficients th[alpha][f]
    float th[16][F];
    if constexpr (PACKED) {
      const uint32_t row = row4(keys, c, (g.dense[0] >> l) & 1u, g.T[0], g.Tmask[0]);
      float v[16 * F];
      load_vec<16 * F>(params + pp.poff[l] + (size_t)row * (16 * F), v);
      int o = 0;
#pragma unroll
      for (int k = 0; k <= 4; ++k)
#pragma unroll
        for (int sl = 0; sl < slots4(k); ++sl, o += F)
#pragma unroll
          for (int f = 0; f < F; ++f) th[alpha4_of_slot(k, sl)][f] = v[o + f];
    } else {
#pragma unroll
      for (int k = 0; k <= 4; ++k) {
        const bool dense = (g.dense[k] >> l) & 1u;
        const uint32_t row = row4(keys, c, dense, g.T[k], g.Tmask[k]);
        const float* src = params + g.off[k][l] + (size_t)row * (slots4(k) * F);
#pragma unroll
        for (int sl = 0; sl < slots4(k); ++sl) load_vec<F>(src + sl * F, th[alpha4_of_slot(k, sl)]);
      }
    }
    const CornerAxis c0 = corner_axis(t[0], Nf, iN, c & 1), c1 = corner_axis(t[1], Nf, iN, (c >> 1) & 1);
    const CornerAxis c2 = corner_axis(t[2], Nf, iN, (c >> 2) & 1), c3 = corner_axis(t[3], Nf, iN, (c >> 3) & 1);
#pragma unroll
    for (int f = 0; f < F; ++f) {
      // axis 3 (w): kinds value, w', w''
      float a3[3][8];
#pragma unroll
      for (int a = 0; a < 8; ++a) {
        const float lo = th[a][f], hi = th[a | 8][f];
        a3[0][a] = c3.b[0] * lo + c3.b[1] * hi;
        a3[1][a] = c3.d[0] * lo + c3.d[1] * hi;
        a3[2][a] = c3.d2[0] * lo + c3.d2[1] * hi;
      }
      // axis 2 (z): value, w', w'', z', z''
      float a2[5][4];
#pragma unroll
      for (int a = 0; a < 4; ++a) {
#pragma unroll
        for (int q = 0; q < 3; ++q) a2[q][a] = c2.b[0] * a3[q][a] + c2.b[1] * a3[q][a | 4];
        a2[3][a] = c2.d[0] * a3[0][a] + c2.d[1] * a3[0][a | 4];
        a2[4][a] = c2.d2[0] * a3[0][a] + c2.d2[1] * a3[0][a | 4];
      }
      // axis 1 (y): value, w', w'', z', z'', y', y''
      float a1[7][2];
#pragma unroll
      for (int a = 0; a < 2; ++a) {
#pragma unroll
        for (int q = 0; q < 5; ++q) a1[q][a] = c1.b[0] * a2[q][a] + c1.b[1] * a2[q][a | 2];
        a1[5][a] = c1.d[0] * a2[0][a] + c1.d[1] * a2[0][a | 2];
        a1[6][a] = c1.d2[0] * a2[0][a] + c1.d2[1] * a2[0][a | 2];
      }
      // axis 0 (x): value, w', w'', z', z'', y', y'', x', x''
      float a0[9];
#pragma unroll
      for (int q = 0; q < 7; ++q) a0[q] = c0.b[0] * a1[q][0] + c0.b[1] * a1[q][1];
      a0[7] = c0.d[0] * a1[0][0] + c0.d[1] * a1[0][1];
      a0[8] = c0.d2[0] * a1[0][0] + c0.d2[1] * a1[0][1];
      out[0][f] += a0[0];
      out[1][f] += a0[7];  // d/dx
      out[2][f] += a0[5];  // d/dy
      out[3][f] += a0[3];  // d/dz
      out[4][f] += a0[1];  // d/dw
      out[5][f] += a0[8];
      out[6][f] += a0[6];
      out[7][f] += a0[4];
      out[8][f] += a0[2];
    }
  }
  const int64_t LF = (int64_t)g.Lrow * F;
  const int64_t col = (int64_t)l * F;
  if (gamma) store_vec<F>(gamma + p * LF + col, out[0]);
  if (dgamma) {
#pragma unroll
    for (int i = 0; i < D; ++i) store_vec<F>(dgamma + (p * D + i) * LF + col, out[1 + i]);
  }
  if (d2gamma) {
    if (d2_mode == HASHENC_D2_DIAG) {
#pragma unroll
      for (int i = 0; i < D; ++i) store_vec<F>(d2gamma + (p * D + i) * LF + col, out[5 + i]);
    } else {
      float lap[F];
#pragma unroll
      for (int f = 0; f < F; ++f) lap[f] = out[5][f] + out[6][f] + out[7][f] + out[8][f];
      store_vec<F>(d2gamma + p * LF + col, lap);
    }
  }
}

// Backward: 16 FL lanes per point (FL = min(F, 4)), lane (alpha, f) owning feature f (and
// f + 4 when F = 8) of the coefficient with derivative bits alpha of every corner.  Each lane
// runs the transposed contraction for its own bits only, so the lanes of a point add one
// order table's row (C(4,k) F contiguous floats) with one atomic instruction, one memory
// request per row, instead of one request per float of one point.
template <int F>
constexpr int h4_lanes() { return 16 * (F > 4 ? 4 : F); }

// Factors of one axis for a given corner bit and derivative bit: value basis, its x-derivative
// and second x-derivative (the expressions of axis_basis; selects between computed values).
__device__ __forceinline__ void axis_factor(float t, float N, float invN, bool far, bool deriv, float& b, float& d,
                                            float& d2) {
  const float s = 1.0f - t;
  const float t2 = t * t;
  const float h00 = (1.0f + 2.0f * t) * s * s, h00p = -6.0f * t * s, h00pp = 12.0f * t - 6.0f;
  const float h10 = t * s * s, h10p = s * (1.0f - 3.0f * t), h10pp = 6.0f * t - 4.0f;
  const float h01 = t2 * (3.0f - 2.0f * t);
  const float h11 = -t2 * s, h11p = t * (3.0f * t - 2.0f), h11pp = 6.0f * t - 2.0f;
  const float N2 = N * N;
  const float bv = far ? h01 : h00, dv = far ? -N * h00p : N * h00p, d2v = far ? -N2 * h00pp : N2 * h00pp;
  const float bd = invN * (far ? h11 : h10), dd = far ? h11p : h10p, d2d = N * (far ? h11pp : h10pp);
  b = deriv ? bd : bv;
  d = deriv ? dd : dv;
  d2 = deriv ? d2d : d2v;
}

template <int F>
__global__ __launch_bounds__(kBlock) void hermite4_backward_kernel(const Grid g, int64_t n, int32_t n_tiles,
                                                                   int d2_mode, const float* __restrict__ x,
                                                                   const float* __restrict__ g_gamma,
                                                                   const float* __restrict__ g_dgamma,
                                                                   const float* __restrict__ g_d2gamma,
                                                                   float* __restrict__ grad) {
  constexpr int D = 4;
  constexpr int FL = F > 4 ? 4 : F;  // lanes per coefficient
  constexpr int FJ = F / FL;         // features per lane
  constexpr int LP = h4_lanes<F>();  // lanes per point
  constexpr int PTS = kBlock / LP;
  const int l = blockIdx.x / n_tiles;
  const int64_t p = (int64_t)(blockIdx.x % n_tiles) * PTS + threadIdx.x / LP;
  const int sub = threadIdx.x % LP;
  const int alpha = sub / FL, f0 = sub % FL;
  if (p >= n) return;  // the lanes of a point leave together
  float xp[D];
#pragma unroll
  for (int i = 0; i < D; ++i) xp[i] = x[p * D + i];
  uint32_t base[D];
  float t[D];
  locate<D>(xp, g.N[l], g.Nf[l], base, t);
  const float Nf = g.Nf[l], iN = g.invN[l];
  const Keys4 keys = keys4(base, g.N[l]);
  const int64_t LF = (int64_t)g.Lrow * F;
  const int64_t col = (int64_t)l * F;
  // this lane's features of the upstream: G0, first derivatives G1[i], second G2[i]
  float G0[FJ], G1[D][FJ], G2[D][FJ];
#pragma unroll
  for (int j = 0; j < FJ; ++j) {
    const int64_t cf = col + f0 + FL * j;
    G0[j] = g_gamma ? g_gamma[p * LF + cf] : 0.0f;
#pragma unroll
    for (int i = 0; i < D; ++i) {
      G1[i][j] = g_dgamma ? g_dgamma[(p * D + i) * LF + cf] : 0.0f;
      G2[i][j] = !g_d2gamma ? 0.0f
                 : d2_mode == HASHENC_D2_DIAG ? g_d2gamma[(p * D + i) * LF + cf]
                                              : g_d2gamma[p * LF + cf];
    }
  }
  const bool ax = alpha & 1, ay = (alpha >> 1) & 1, az = (alpha >> 2) & 1, aw = (alpha >> 3) & 1;
  const int order = ax + ay + az + aw;
  // slot of alpha among the alphas of its order (lexicographic axis tuples), one nibble per
  // alpha: x y z w | xy xz xw yz yw zw | xyz xyw xzw yzw
  constexpr uint64_t kSlots4 = 0x0325142303120100ull;
  const int slot = (int)((kSlots4 >> (4 * alpha)) & 15u);
#pragma unroll 1
  for (int c = 0; c < 16; ++c) {
    float bx, dx, d2x, by, dy, d2y, bz, dz, d2z, bw, dw, d2w;
    axis_factor(t[0], Nf, iN, c & 1, ax, bx, dx, d2x);
    axis_factor(t[1], Nf, iN, (c >> 1) & 1, ay, by, dy, d2y);
    axis_factor(t[2], Nf, iN, (c >> 2) & 1, az, bz, dz, d2z);
    axis_factor(t[3], Nf, iN, (c >> 3) & 1, aw, bw, dw, d2w);
    // d theta[alpha] = sum over outputs of the upstream times the product of the per-axis
    // factors (value basis on every axis but the differentiated one)
    const float xyz = bx * by * bz, xyw = bx * by * bw, xzw = bx * bz * bw, yzw = by * bz * bw;
    float th[FJ];
#pragma unroll
    for (int j = 0; j < FJ; ++j)
      th[j] = xyz * bw * G0[j] + dx * yzw * G1[0][j] + dy * xzw * G1[1][j] + dz * xyw * G1[2][j] +
              dw * xyz * G1[3][j] + d2x * yzw * G2[0][j] + d2y * xzw * G2[1][j] + d2z * xyw * G2[2][j] +
              d2w * xyz * G2[3][j];
    // one order table at a time (a uniform loop), its lanes adding one contiguous row
#pragma unroll
    for (int k = 0; k <= 4; ++k) {
      if (order != k) continue;
      const bool dense = (g.dense[k] >> l) & 1u;
      const uint32_t row = row4(keys, c, dense, g.T[k], g.Tmask[k]);
      float* dst = grad + g.off[k][l] + (size_t)row * (slots4(k) * F) + slot * F + f0;
#pragma unroll
      for (int j = 0; j < FJ; ++j) atomic_add_f32(dst + FL * j, th[j]);
    }
  }
}

// Lookup-stage export for d = 4: rows of the 16 corners of table `order`, [n][L][16].
__global__ __launch_bounds__(kBlock) void debug_indices4_kernel(const Grid g, int order, int64_t n,
                                                                const float* __restrict__ x,
                                                                int32_t* __restrict__ out) {
  const int64_t p = (int64_t)blockIdx.x * kBlock + threadIdx.x;
  if (p >= n) return;
  float xp[4];
  for (int i = 0; i < 4; ++i) xp[i] = x[p * 4 + i];
  for (int l = 0; l < g.L; ++l) {
    uint32_t base[4];
    float t[4];
    locate<4>(xp, g.N[l], g.Nf[l], base, t);
    const Keys4 keys = keys4(base, g.N[l]);
    const bool dense = (g.dense[order] >> l) & 1u;
    for (int c = 0; c < 16; ++c)
      out[(p * g.L + l) * 16 + c] = (int32_t)row4(keys, c, dense, g.T[order], g.Tmask[order]);
  }
}

// Binned backward for d = 4, count pass: lane j of the workgroup's loop takes point j / 16
// of the tile and its corner j % 16, and histograms that corner's row in every order table
// at each level of the group (once, in fine bins, when the table sizes are equal).
__global__ __launch_bounds__(kBinThreads) void hermite4_count_kernel(const Grid g, const BinPlan bp, int64_t n,
                                                                     int32_t tile, int32_t nblk, int32_t lpg,
                                                                     const float* __restrict__ x,
                                                                     int32_t* __restrict__ counts) {
  extern __shared__ int32_t hist[];
  const int blk = bin_tile_of_block(blockIdx.x, nblk);
  const int l0 = blockIdx.y * lpg, l1 = min(g.L, l0 + lpg);
  const bool fine = bp.fine_shift >= 0;
  const int nh = fine ? bp.fine_bin0[g.L] : bp.nbins;
  for (int i = threadIdx.x; i < nh; i += kBinThreads) hist[i] = 0;
  __syncthreads();
  for (int j = threadIdx.x; j < 16 * tile; j += kBinThreads) {
    const int64_t p = (int64_t)blk * tile + j / 16;
    if (p >= n) break;
    const int c = j % 16;
    float xp[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) xp[i] = x[p * 4 + i];
    for (int l = l0; l < l1; ++l) {
      uint32_t base[4];
      float t[4];
      locate<4>(xp, g.N[l], g.Nf[l], base, t);
      const Keys4 keys = keys4(base, g.N[l]);
      if (fine) {
        const int32_t bin =
            bp.fine_bin0[l] + (int32_t)(row4(keys, c, (g.dense[0] >> l) & 1u, g.T[0], g.Tmask[0]) >> bp.fine_shift);
        if (bp.fine_bin0[l + 1] - bp.fine_bin0[l] <= kFewBins) wave_aggregated_add<false>(hist, bin);
        else atomicAdd(&hist[bin], 1);
        continue;
      }
#pragma unroll
      for (int k = 0; k <= 4; ++k) {
        int32_t bin;
        uint32_t local;
        bin_of(bp, k, l, row4(keys, c, (g.dense[k] >> l) & 1u, g.T[k], g.Tmask[k]), bin, local);
        if (bp.seg_bin0[k * bp.L + l + 1] - bp.seg_bin0[k * bp.L + l] <= kFewBins) wave_aggregated_add<false>(hist, bin);
        else atomicAdd(&hist[bin], 1);
      }
    }
  }
  __syncthreads();
  store_tile_counts(bp, l0, l1, fine, hist, counts + (int64_t)blk * bp.nbins);
}

// Upstream of one point at one level for the d = 4 scatter: G0 value, G1[i] first and G2[i]
// second derivative along axis i (the Laplacian's upstream counts for every axis).
template <int F>
struct Up4 {
  float G0[F], G1[4][F], G2[4][F];
};

template <int F>
__device__ __forceinline__ Up4<F> load_up4(const Grid& g, int64_t p, int l, int d2_mode, const float* __restrict__ gg,
                                          const float* __restrict__ gd, const float* __restrict__ g2) {
  const int64_t LF = (int64_t)g.Lrow * F;
  const int64_t col = (int64_t)l * F;
  Up4<F> u;
  if (gg) load_vec<F>(gg + p * LF + col, u.G0);
  else
#pragma unroll
    for (int f = 0; f < F; ++f) u.G0[f] = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (gd) load_vec<F>(gd + (p * 4 + i) * LF + col, u.G1[i]);
    else
#pragma unroll
      for (int f = 0; f < F; ++f) u.G1[i][f] = 0.0f;
    if (!g2) {
#pragma unroll
      for (int f = 0; f < F; ++f) u.G2[i][f] = 0.0f;
    } else {
      load_vec<F>(g2 + (d2_mode == HASHENC_D2_DIAG ? (p * 4 + i) * LF : p * LF) + col, u.G2[i]);
    }
  }
  return u;
}

// d theta of the coefficient with derivative bits A of one corner: the upstream of every
// output times the product of that corner's per-axis factors for the bits of A (value basis
// on every axis but the differentiated one; the transpose of the forward's contraction).
template <int F, int A>
__device__ __forceinline__ void coef_grad4(const CornerAxis (&ca)[4], const Up4<F>& u, float* v) {
  constexpr int ax = A & 1, ay = (A >> 1) & 1, az = (A >> 2) & 1, aw = (A >> 3) & 1;
  const float bx = ca[0].b[ax], by = ca[1].b[ay], bz = ca[2].b[az], bw = ca[3].b[aw];
  const float xyz = bx * by * bz, xyw = bx * by * bw, xzw = bx * bz * bw, yzw = by * bz * bw;
  const float w0 = xyz * bw;
  const float w1x = ca[0].d[ax] * yzw, w1y = ca[1].d[ay] * xzw, w1z = ca[2].d[az] * xyw, w1w = ca[3].d[aw] * xyz;
  const float w2x = ca[0].d2[ax] * yzw, w2y = ca[1].d2[ay] * xzw, w2z = ca[2].d2[az] * xyw,
              w2w = ca[3].d2[aw] * xyz;
#pragma unroll
  for (int f = 0; f < F; ++f)
    v[f] = w0 * u.G0[f] + w1x * u.G1[0][f] + w1y * u.G1[1][f] + w1z * u.G1[2][f] + w1w * u.G1[3][f] +
           w2x * u.G2[0][f] + w2y * u.G2[1][f] + w2z * u.G2[2][f] + w2w * u.G2[3][f];
}

// One (level, order table K) phase of the d = 4 scatter workgroup (T lanes, 16 per point):
// each lane stages its corner's table-K record {local row, C(4,K) F values} at its slot,
// sorted by bin, then the records are copied out one per lane.
template <int F, int T, int K>
__device__ __forceinline__ void scatter4_table(const Grid& g, const BinPlan& bp, int l, bool on, int c, int np,
                                               int lo_k, int32_t base, const Keys4& keys, const CornerAxis (&ca)[4],
                                               const Up4<F>& u, const BinState* __restrict__ st,
                                               float* __restrict__ vals_out, const HScatterLds<4, F, T>& sh,
                                               uint32_t* vsh, uint32_t nf) {
  constexpr int S = slots4(K);
  constexpr int W = S * F;
  constexpr int R = hermite_rec_width(W);
  constexpr int RS = hermite_stage_width(W);
  const int sg = K * bp.L + l;
  const int32_t b0 = bp.seg_bin0[sg];
  const int nb = bp.seg_bin0[sg + 1] - b0;
  float vmx = 0.0f;  // largest |value| of this lane's record (NaN values aside: nf)
  if (on) {
    float rec[RS];
    [&]<int... Q>(std::integer_sequence<int, Q...>) {
      (coef_grad4<F, alpha4_of_slot(K, Q)>(ca, u, rec + 1 + Q * F), ...);
    }(std::make_integer_sequence<int, S>{});
#pragma unroll
    for (int j = 1; j <= W; ++j) vmx = fmaxf(vmx, fabsf(rec[j]));
    int32_t bin;
    uint32_t local;
    bin_of(bp, K, l, row4(keys, c, (g.dense[K] >> l) & 1u, g.T[K], g.Tmask[K]), bin, local);
    const int i = lo_k + (bin - b0);
    const int32_t slot = nb <= kFewBins ? wave_aggregated_add<true>(sh.lcur + lo_k, bin - b0) : atomicAdd(&sh.lcur[i], 1);
    rec[0] = __uint_as_float(local);
    rec[R] = __int_as_float(sh.delta[i] + slot);  // the record's entry in the segment
#pragma unroll
    for (int j = R + 1; j < RS; ++j) rec[j] = 0.0f;
    store_vec<RS>(sh.st_rec + (int64_t)(slot - base) * RS, rec);
  }
  raise_seg_vmax(vsh, sg, max(__float_as_uint(vmx), nf));
  __syncthreads();
  const int32_t ebase = st->seg_ebase[sg];
  float* vseg = vals_out + st->seg_vbase[sg];
  for (int32_t q = threadIdx.x; q < np * 16; q += T) {
    float v[RS];
    load_vec<RS>(sh.st_rec + (int64_t)q * RS, v);
    float* dst = vseg + (int64_t)(__float_as_int(v[R]) - ebase) * R;
#pragma unroll
    for (int j = 0; j < R; ++j) dst[j] = v[j];
  }
  __syncthreads();
}

// Binned backward for d = 4, scatter pass: 16 lanes per point of a P-point tile, lane c
// owning corner c.  Per level the tile's slot ranges in all of the level's bins are set up at
// once; then per order table each lane computes its corner's record, stages it by bin and the
// workgroup copies the records out as contiguous runs.
template <int F, int P>
__global__ __launch_bounds__(16 * P) void hermite4_scatter_kernel(
    const Grid g, const BinPlan bp, int64_t n, int32_t nblk, int32_t lpg, int d2_mode, const float* __restrict__ x,
    const float* __restrict__ gg, const float* __restrict__ gd, const float* __restrict__ g2,
    const int32_t* __restrict__ counts, const int32_t* __restrict__ totals, const int32_t* __restrict__ bin_start,
    const BinState* __restrict__ st, float* __restrict__ vals_out, uint32_t* __restrict__ vmax) {
  constexpr int T = 16 * P;
  extern __shared__ int32_t lds[];
  const HScatterLds<4, F, T> sh(lds, bp.max_level_bins);
  __shared__ uint32_t vsh[kMaxSeg];  // the workgroup's segment bounds
  for (int i = threadIdx.x; i < kMaxSeg; i += T) vsh[i] = 0u;
  __syncthreads();
  const int blk = bin_tile_of_block(blockIdx.x, nblk);
  const int c = threadIdx.x % 16;
  const int64_t p = (int64_t)blk * P + threadIdx.x / 16;
  const bool on = p < n;
  const int np = (int)min((int64_t)P, n - (int64_t)blk * P);
  float xp[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) xp[i] = on ? x[p * 4 + i] : 0.0f;
  const int l0 = blockIdx.y * lpg, l1 = min(g.L, l0 + lpg);
  for (int l = l0; l < l1; ++l) {
    Up4<F> u;
    uint32_t nf = 0u;  // NaN bound for the level's segments unless its values are finite
    if (on) {
      u = load_up4<F>(g, p, l, d2_mode, gg, gd, g2);
      uint32_t m = 0u;
#pragma unroll
      for (int f = 0; f < F; ++f) {
        m = max(m, abs_bits(u.G0[f]));
#pragma unroll
        for (int i = 0; i < 4; ++i) m = max(m, max(abs_bits(u.G1[i][f]), abs_bits(u.G2[i][f])));
      }
      nf = hermite_nonfinite_floor(m, g.Nf[l], 4);
    }
    int32_t base_k[5];
    hermite_level_bins<4, T>(bp, l, blk, nblk, counts, totals, bin_start, sh.delta, sh.lcur, sh.wsum, base_k);
    Keys4 keys;
    CornerAxis ca[4];
    if (on) {
      uint32_t base[4];
      float t[4];
      locate<4>(xp, g.N[l], g.Nf[l], base, t);
      keys = keys4(base, g.N[l]);
#pragma unroll
      for (int i = 0; i < 4; ++i) ca[i] = corner_axis(t[i], g.Nf[l], g.invN[l], (c >> i) & 1);
    }
    int lo = 0;
    scatter4_table<F, T, 0>(g, bp, l, on, c, np, lo, base_k[0], keys, ca, u, st, vals_out, sh, vsh, nf);
    lo += bp.seg_bin0[l + 1] - bp.seg_bin0[l];
    scatter4_table<F, T, 1>(g, bp, l, on, c, np, lo, base_k[1], keys, ca, u, st, vals_out, sh, vsh, nf);
    lo += bp.seg_bin0[bp.L + l + 1] - bp.seg_bin0[bp.L + l];
    scatter4_table<F, T, 2>(g, bp, l, on, c, np, lo, base_k[2], keys, ca, u, st, vals_out, sh, vsh, nf);
    lo += bp.seg_bin0[2 * bp.L + l + 1] - bp.seg_bin0[2 * bp.L + l];
    scatter4_table<F, T, 3>(g, bp, l, on, c, np, lo, base_k[3], keys, ca, u, st, vals_out, sh, vsh, nf);
    lo += bp.seg_bin0[3 * bp.L + l + 1] - bp.seg_bin0[3 * bp.L + l];
    scatter4_table<F, T, 4>(g, bp, l, on, c, np, lo, base_k[4], keys, ca, u, st, vals_out, sh, vsh, nf);
  }
  __syncthreads();
  publish_seg_vmax(vsh, bp.nseg, vmax);
}

template <int F>
hipError_t launch_bin4(const Grid& g, const BinPlan& bp, const BinWorkspace& w, char* ws, int d2_mode, bool scatter,
                       int64_t n, const float* x, const float* gg, const float* gd, const float* g2, hipStream_t s) {
  const dim3 grid((unsigned)w.nblk, (unsigned)w.lgroups);
  int32_t* counts = reinterpret_cast<int32_t*>(ws + w.counts);
  if (!scatter) {
    const size_t hist = sizeof(int32_t) * (size_t)(bp.fine_shift >= 0 ? bp.fine_bin0[g.L] : bp.nbins);
    hipLaunchKernelGGL(hermite4_count_kernel, grid, dim3(kBinThreads), hist, s, g, bp, n, w.tile, w.nblk, w.lpg, x,
                       counts);
    return hipGetLastError();
  }
  constexpr int P = hermite4_scatter_points(F);
  if (w.tile != P) return hipErrorInvalidValue;
  const size_t lds = hermite_scatter_lds_bytes(bp, 4, F);
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&hermite4_scatter_kernel<F, P>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((hermite4_scatter_kernel<F, P>), grid, dim3(16 * P), lds, s, g, bp, n, w.nblk, w.lpg, d2_mode, x,
                     gg, gd, g2, counts, reinterpret_cast<const int32_t*>(ws + w.totals),
                     reinterpret_cast<const int32_t*>(ws + w.bin_start), reinterpret_cast<const BinState*>(ws + w.state),
                     reinterpret_cast<float*>(ws + w.vals), reinterpret_cast<BinState*>(ws + w.state)->vmax_bits);
  return hipGetLastError();
}

template <int F>
hipError_t launch_fwd4(const Grid& g, int d2_mode, int64_t n, const float* x, const float* params, float* packed,
                       float* gamma, float* dgamma, float* d2gamma, hipStream_t s) {
  const int64_t tiles = (n + kBlock - 1) / kBlock;
  if (tiles * g.L > 0x7fffffff) return hipErrorInvalidValue;
  const dim3 grid((unsigned)(tiles * g.L));
  if constexpr (F <= 2) {
    if (packed) {
      const PackPlan pp = make_pack_plan(g, 4, F);
      hipLaunchKernelGGL((hermite4_pack_kernel<F>), dim3((unsigned)((pp.poff[g.L] / (16 * F) + kBlock - 1) / kBlock)),
                         dim3(kBlock), 0, s, g, pp, params, packed);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      hipLaunchKernelGGL((hermite4_forward_kernel<F, true>), grid, dim3(kBlock), 0, s, g, pp, n, (int32_t)tiles,
                         d2_mode, x, packed, gamma, dgamma, d2gamma);
    } else {
      hipLaunchKernelGGL((hermite4_forward_kernel<F, false>), grid, dim3(kBlock), 0, s, g, PackPlan{}, n,
                         (int32_t)tiles, d2_mode, x, params, gamma, dgamma, d2gamma);
    }
  } else {
    if (packed) return hipErrorInvalidValue;  // F > 2: no packed copy
    hipLaunchKernelGGL((hermite4_forward_kernel<F, false>), grid, dim3(kBlock), 0, s, g, PackPlan{}, n,
                       (int32_t)tiles, d2_mode, x, params, gamma, dgamma, d2gamma);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || g.L == g.Lrow) return e;
  const int RF = g.Lrow * F, AF = g.L * F;
  if (gamma) e = launch_zero_columns(gamma, n, RF, AF, s);
  if (e == hipSuccess && dgamma) e = launch_zero_columns(dgamma, n * 4, RF, AF, s);
  if (e == hipSuccess && d2gamma) e = launch_zero_columns(d2gamma, n * (d2_mode == HASHENC_D2_DIAG ? 4 : 1), RF, AF, s);
  return e;
}

template <int F>
hipError_t launch_bwd4(const Grid& g, int d2_mode, int64_t n, const float* x, const float* gg, const float* gd,
                       const float* g2, float* grad, hipStream_t s) {
  constexpr int PTS = kBlock / h4_lanes<F>();  // points per workgroup
  const int64_t tiles = (n + PTS - 1) / PTS;
  if (tiles * g.L > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL((hermite4_backward_kernel<F>), dim3((unsigned)(tiles * g.L)), dim3(kBlock), 0, s, g, n,
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

bool hermite_packable(const Grid& g, int d) {
  // every table equal to the order-0 one, or a power of two no larger than it (which the
  // order-0 size then is too): the row of a vertex in table k follows from its order-0 row
  for (int k = 1; k <= d; ++k)
    if (g.T[k] != g.T[0] && !(g.Tmask[k] && g.Tmask[0] && g.T[k] < g.T[0])) return false;
  return true;
}

size_t hermite_packed_bytes(const Grid& g, int d, int F) {
  return hermite_packable(g, d) ? sizeof(float) * (size_t)make_pack_plan(g, d, F).poff[g.L] : 0;
}

hipError_t launch_hermite_pack(const Grid& g, int d, int F, const float* params, float* packed, hipStream_t s) {
  HASHENC_DISPATCH_DF(d, F, launch_pack, g, params, packed, s);
}

size_t hermite_stage_bytes(const Grid& g, int d, int F, int d2_mode, int64_t n) {
  const int M = 1 + d + (d2_mode == HASHENC_D2_DIAG ? d : 1);
  return sizeof(float) * (size_t)n * g.L * M * F;
}

hipError_t launch_hermite_forward(const Grid& g, int d, int F, int d2_mode, int64_t n,
                                  const float* x, const float* params, const float* packed, float* stage,
                                  bool to_rows, float* gamma, float* dgamma, float* d2gamma, hipStream_t s) {
  HASHENC_DISPATCH_DF(d, F, launch_fwd, g, d2_mode, n, x, params, packed, stage, to_rows, gamma, dgamma, d2gamma,
                      s);
}

hipError_t launch_hermite_backward(const Grid& g, int d, int F, int d2_mode, int64_t n,
                                   const float* x, const float* g_gamma, const float* g_dgamma,
                                   const float* g_d2gamma, const float* u_levels, float* grad, hipStream_t s) {
  HASHENC_DISPATCH_DF(d, F, launch_bwd, g, d2_mode, n, x, g_gamma, g_dgamma, g_d2gamma, u_levels, grad, s);
}

#define HASHENC_DISPATCH_F4(F, FN, ...)         \
  do {                                          \
    switch (F) {                                \
      case 1: return FN<1>(__VA_ARGS__);        \
      case 2: return FN<2>(__VA_ARGS__);        \
      case 4: return FN<4>(__VA_ARGS__);        \
      case 8: return FN<8>(__VA_ARGS__);        \
    }                                           \
    return hipErrorInvalidValue;                \
  } while (0)

hipError_t launch_debug_indices4(const Grid& g, int order, int64_t n, const float* x, int32_t* out, hipStream_t s) {
  hipLaunchKernelGGL(debug_indices4_kernel, dim3((unsigned)((n + kBlock - 1) / kBlock)), dim3(kBlock), 0, s, g, order,
                     n, x, out);
  return hipGetLastError();
}

size_t hermite4_packed_bytes(const Grid& g, int F) {
  return F <= 2 && hermite_packable(g, 4) ? sizeof(float) * (size_t)make_pack_plan(g, 4, F).poff[g.L] : 0;
}

hipError_t launch_hermite4_forward(const Grid& g, int F, int d2_mode, int64_t n, const float* x,
                                   const float* params, float* packed, float* gamma, float* dgamma, float* d2gamma,
                                   hipStream_t s) {
  HASHENC_DISPATCH_F4(F, launch_fwd4, g, d2_mode, n, x, params, packed, gamma, dgamma, d2gamma, s);
}

hipError_t launch_hermite4_backward(const Grid& g, int F, int d2_mode, int64_t n, const float* x,
                                    const float* g_gamma, const float* g_dgamma, const float* g_d2gamma,
                                    float* grad, hipStream_t s) {
  HASHENC_DISPATCH_F4(F, launch_bwd4, g, d2_mode, n, x, g_gamma, g_dgamma, g_d2gamma, grad, s);
}

hipError_t launch_hermite4_bin(const Grid& g, const BinPlan& bp, const BinWorkspace& w, char* ws, int F,
                               int d2_mode, bool scatter, int64_t n, const float* x, const float* g_gamma,
                               const float* g_dgamma, const float* g_d2gamma, hipStream_t s) {
  switch (F) {  // F = 8 has rows wider than the reduce takes (no binned plan)
    case 1: return launch_bin4<1>(g, bp, w, ws, d2_mode, scatter, n, x, g_gamma, g_dgamma, g_d2gamma, s);
    case 2: return launch_bin4<2>(g, bp, w, ws, d2_mode, scatter, n, x, g_gamma, g_dgamma, g_d2gamma, s);
    case 4: return launch_bin4<4>(g, bp, w, ws, d2_mode, scatter, n, x, g_gamma, g_dgamma, g_d2gamma, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_hermite_bin(const Grid& g, const BinPlan& bp, const BinWorkspace& w, char* ws, int d, int F,
                              int d2_mode, bool scatter, int64_t n, const float* x, const float* g_gamma,
                              const float* g_dgamma, const float* g_d2gamma, const float* u_levels, hipStream_t s) {
  HASHENC_DISPATCH_DF(d, F, launch_bin, g, bp, w, ws, d2_mode, scatter, n, x, g_gamma, g_dgamma, g_d2gamma, u_levels,
                      s);
}

}  // namespace hg
