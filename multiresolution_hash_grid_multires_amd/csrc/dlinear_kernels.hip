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
#include "binned_backward.h"
#include "hashenc_internal.h"
#include "vec_io.h"

namespace hg {
namespace {

// Forward.  Workgroups are ordered level-major: workgroup b handles level b / n_tiles for
// the b % n_tiles-th tile of kBlock points.  Workgroups are dispatched in order, so at any
// moment the whole chip works on one or two levels and each XCD's L2 holds those levels'
// tables (4 MB for a hashed level of 2^19 rows of F = 2) instead of streaming every level's
// table from the Infinity Cache.  x is re-read per level (12 bytes per point, cache hits).
// LM_OUT: write level-major [L][n][F] (whole cache lines per workgroup) instead of the
// point-major [n][L*F] rows, for the workspace path that transposes afterwards.
template <int D, int F, bool LM_OUT>
__global__ __launch_bounds__(kBlock) void dlinear_forward_kernel(const Grid g, int64_t n, int32_t n_tiles,
                                                                 const float* __restrict__ x,
                                                                 const float* __restrict__ params,
                                                                 float* __restrict__ gamma) {
  const int l = blockIdx.x / n_tiles;
  const int64_t p = (int64_t)(blockIdx.x % n_tiles) * kBlock + threadIdx.x;
  if (p >= n) return;
  float xp[D];
#pragma unroll
  for (int i = 0; i < D; ++i) xp[i] = x[p * D + i];
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
  if constexpr (LM_OUT) store_vec<F>(gamma + ((int64_t)l * n + p) * F, acc);
  else store_vec<F>(gamma + p * (int64_t)g.L * F + (int64_t)l * F, acc);
}

// [L][n][F] -> [n][L*F]: one lane per point assembles its output row 4 floats at a time
// from the level-major rows (loads coalesced across lanes) and writes 16-byte pieces, so
// every output line is written whole by one wavefront.
template <int F>
__global__ __launch_bounds__(kBlock) void level_major_to_rows_kernel(int32_t L, int64_t n,
                                                                     const float* __restrict__ lm,
                                                                     float* __restrict__ out) {
  const int64_t p = (int64_t)blockIdx.x * kBlock + threadIdx.x;
  if (p >= n) return;
  const int LF = L * F;
  float* row = out + p * (int64_t)LF;
  for (int c = 0; c < LF; c += 4) {
    float v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int col = c + i;
      v[i] = col < LF ? lm[((int64_t)(col / F) * n + p) * F + col % F] : 0.0f;
    }
    if ((LF & 3) == 0) {  // rows 16-byte aligned
      reinterpret_cast<float4*>(row)[c / 4] = make_float4(v[0], v[1], v[2], v[3]);
    } else {
      for (int i = 0; c + i < LF; ++i) row[c + i] = v[i];
    }
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

// Binned backward, count pass: a workgroup owns a tile of `tile` points (at most 4 per
// lane) and histograms their entries over all bins in LDS.  On pair-mode levels the two
// x-corners of each (y, z) corner pair make one entry (they always share a bin); elsewhere
// each corner is its own entry.
template <int D>
__global__ __launch_bounds__(kBinThreads) void dlinear_count_kernel(const Grid g, const BinPlan bp, int64_t n,
                                                                    int32_t tile, int32_t nblk,
                                                                    const float* __restrict__ x,
                                                                    int32_t* __restrict__ counts) {
  extern __shared__ int32_t hist[];
  const int blk = blockIdx.x;
  for (int i = threadIdx.x; i < bp.nbins; i += kBinThreads) hist[i] = 0;
  __syncthreads();
  const int ppt = tile / kBinThreads;
  const int64_t p0 = (int64_t)blk * tile + threadIdx.x;
  float xp[4][D];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int64_t p = p0 + (int64_t)j * kBinThreads;
#pragma unroll
    for (int i = 0; i < D; ++i) xp[j][i] = (j < ppt && p < n) ? x[p * D + i] : 0.0f;
  }
  for (int l = 0; l < g.L; ++l) {
    const bool dense = (g.dense[0] >> l) & 1u;
    const bool pair = (bp.pair_mask >> l) & 1u;
    const bool few = bp.seg_bin0[l + 1] - bp.seg_bin0[l] <= kFewBins;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t p = p0 + (int64_t)j * kBinThreads;
      if (j >= ppt || p >= n) break;
      uint32_t base[D];
      float t[D];
      locate<D>(xp[j], g.N[l], g.Nf[l], base, t);
      const CellKeys<D> keys = cell_keys<D>(base, g.N[l]);
      [&]<int... Y>(std::integer_sequence<int, Y...>) {
        ((
             [&] {
               int32_t b0, b1;
               uint32_t local;
               bin_of(bp, 0, l, corner_row<D, (Y << 1)>(keys, dense, g.T[0], g.Tmask[0]), b0, local);
               if (few) wave_aggregated_add<false>(hist, b0);
               else atomicAdd(&hist[b0], 1);
               if (!pair) {
                 bin_of(bp, 0, l, corner_row<D, (Y << 1) | 1>(keys, dense, g.T[0], g.Tmask[0]), b1, local);
                 if (few) wave_aggregated_add<false>(hist, b1);
                 else atomicAdd(&hist[b1], 1);
               }
             }()),
         ...);
      }(std::make_integer_sequence<int, 1 << (D - 1)>{});
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < bp.nbins; i += kBinThreads) counts[(int64_t)i * nblk + blk] = hist[i];
}

// Binned backward, scatter pass.  Per level, the tile's pair records are first sorted by bin
// in LDS (a local counting sort seeded with the tile's per-bin counts from the count pass),
// then copied out so that each bin receives one contiguous run: consecutive lanes write
// consecutive records and cache lines are written whole.  Single-corner records (levels
// not in pair mode) are written straight to their slots.
// PRE: the tile's upstream rows (L*F <= 32 floats per point) are read once into registers
// before the level loop; otherwise each level reads its F floats of the row.
template <int D, int F, bool PRE>
__global__ __launch_bounds__(kScatterThreads) void dlinear_scatter_kernel(
    const Grid g, const BinPlan bp, int64_t n, int32_t tile, int32_t nblk, const float* __restrict__ x,
    const float* __restrict__ g_gamma, const int32_t* __restrict__ counts,
    const int32_t* __restrict__ totals, const int32_t* __restrict__ bin_start,
    const BinState* __restrict__ st, float* __restrict__ vals_out) {
  constexpr int NP = 1 << (D - 1);  // x-corner pairs per cell
  constexpr int R = 2 + F;          // floats per record
  extern __shared__ int32_t lds[];
  const int mb = bp.max_seg_bins;
  const int nbins = bp.nbins;
  int32_t* gstart = lds;                 // [nbins] global slot of this tile's run in each bin
  int32_t* bcnt = lds + nbins;           // [nbins] this tile's entries in each bin
  int32_t* lstart = lds + 2 * nbins;     // [mb] start of each bin's run in the staging area
  int32_t* lcur = lstart + mb;           // [mb] slot cursors
  int32_t* scan = lcur + mb;             // [kScatterThreads]
  float* st_rec = reinterpret_cast<float*>(scan + kScatterThreads);          // [tile*NP*R]
  int32_t* st_pos = reinterpret_cast<int32_t*>(st_rec + (int64_t)tile * NP * R);  // [tile*NP]

  const int blk = blockIdx.x;
  const int ppt = tile / kScatterThreads;
  const int64_t p0 = (int64_t)blk * tile + threadIdx.x;
  const int64_t tile_pts = min((int64_t)tile, n - (int64_t)blk * tile);
  for (int i = threadIdx.x; i < nbins; i += kScatterThreads) {
    const int32_t pre = counts[(int64_t)i * nblk + blk];
    const int32_t nxt = blk + 1 < nblk ? counts[(int64_t)i * nblk + blk + 1] : totals[i];
    gstart[i] = bin_start[i] + pre;
    bcnt[i] = nxt - pre;
  }
  __syncthreads();
  constexpr int MAXP = 2;  // points per lane (tile <= 2 * kScatterThreads)
  float xp[MAXP][D];
  const int64_t LF = (int64_t)g.L * F;
  float up[PRE ? MAXP : 1][PRE ? 32 : 1];
#pragma unroll
  for (int j = 0; j < MAXP; ++j) {
    const int64_t p = p0 + (int64_t)j * kScatterThreads;
    const bool on = j < ppt && p < n;
#pragma unroll
    for (int i = 0; i < D; ++i) xp[j][i] = on ? x[p * D + i] : 0.0f;
    if constexpr (PRE) {
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        float4 a = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        if (on && g_gamma && 4 * q < LF) a = reinterpret_cast<const float4*>(g_gamma + p * LF)[q];
        up[j][4 * q] = a.x; up[j][4 * q + 1] = a.y; up[j][4 * q + 2] = a.z; up[j][4 * q + 3] = a.w;
      }
    }
  }
  for (int l = 0; l < g.L; ++l) {
    const int32_t b0 = bp.seg_bin0[l];
    const int nb = bp.seg_bin0[l + 1] - b0;
    // exclusive scan of this tile's counts over the level's bins -> staging starts
    const int per = (nb + kScatterThreads - 1) / kScatterThreads;
    int32_t mysum = 0;
    for (int q = 0; q < per; ++q) {
      const int i = threadIdx.x * per + q;
      if (i < nb) mysum += bcnt[b0 + i];
    }
    scan[threadIdx.x] = mysum;
    __syncthreads();
    for (int off = 1; off < kScatterThreads; off <<= 1) {
      const int32_t v = threadIdx.x >= off ? scan[threadIdx.x - off] : 0;
      __syncthreads();
      scan[threadIdx.x] += v;
      __syncthreads();
    }
    int32_t run = scan[threadIdx.x] - mysum;
    for (int q = 0; q < per; ++q) {
      const int i = threadIdx.x * per + q;
      if (i < nb) {
        lstart[i] = run;
        lcur[i] = run;
        run += bcnt[b0 + i];
      }
    }
    __syncthreads();
    const bool dense = (g.dense[0] >> l) & 1u;
    const bool pair = (bp.pair_mask >> l) & 1u;
    const bool few = nb <= kFewBins;
    const int32_t ebase = st->seg_ebase[l];
    float* vseg = vals_out + st->seg_vbase[l];
#pragma unroll
    for (int j = 0; j < MAXP; ++j) {
      const int64_t p = p0 + (int64_t)j * kScatterThreads;
      if (j >= ppt || p >= n) break;
      uint32_t base[D];
      float t[D];
      locate<D>(xp[j], g.N[l], g.Nf[l], base, t);
      const CellKeys<D> keys = cell_keys<D>(base, g.N[l]);
      float G[F];
      if constexpr (PRE) {
        // register array indexed by the wave-uniform level: select with a small unrolled scan
#pragma unroll
        for (int f = 0; f < F; ++f) {
          float v = 0.0f;
#pragma unroll
          for (int c = f; c < 32; c += F)
            if (c == l * F + f) v = up[j][c];
          G[f] = v;
        }
      } else if (g_gamma) {
        load_vec<F>(g_gamma + p * LF + (int64_t)l * F, G);
      } else {
#pragma unroll
        for (int f = 0; f < F; ++f) G[f] = 0.0f;
      }
      [&]<int... Y>(std::integer_sequence<int, Y...>) {
        ((
             [&] {
               float a = 1.0f;  // weight of the (y, z) corner pair
#pragma unroll
               for (int i = 1; i < D; ++i) a *= ((Y >> (i - 1)) & 1) ? t[i] : 1.0f - t[i];
               float rec[R];
#pragma unroll
               for (int f = 0; f < F; ++f) rec[2 + f] = a * G[f];
               int32_t bn0, bn1;
               uint32_t lo, hi;
               bin_of(bp, 0, l, corner_row<D, (Y << 1)>(keys, dense, g.T[0], g.Tmask[0]), bn0, lo);
               bin_of(bp, 0, l, corner_row<D, (Y << 1) | 1>(keys, dense, g.T[0], g.Tmask[0]), bn1, hi);
               if (pair) {
                 const int i = bn0 - b0;
                 const int32_t lp = few ? wave_aggregated_add<true>(lcur, i) : atomicAdd(&lcur[i], 1);
                 rec[0] = __uint_as_float(lo | (hi << 16));
                 rec[1] = t[0];
#pragma unroll
                 for (int q = 0; q < R; ++q) st_rec[(int64_t)lp * R + q] = rec[q];
                 st_pos[lp] = gstart[bn0] + (lp - lstart[i]);
               } else {
                 // two single-corner records, lower row gets (1 - t) aG
                 const int i0 = bn0 - b0, i1 = bn1 - b0;
                 const int32_t s0 = few ? wave_aggregated_add<true>(lcur, i0) : atomicAdd(&lcur[i0], 1);
                 rec[0] = __uint_as_float(lo | 0xFFFF0000u);
                 rec[1] = t[0];
                 store_vec<R>(vseg + (int64_t)(gstart[bn0] + (s0 - lstart[i0]) - ebase) * R, rec);
                 const int32_t s1 = few ? wave_aggregated_add<true>(lcur, i1) : atomicAdd(&lcur[i1], 1);
                 rec[0] = __uint_as_float(hi | 0xFFFF0000u);
                 rec[1] = 1.0f - t[0];
                 store_vec<R>(vseg + (int64_t)(gstart[bn1] + (s1 - lstart[i1]) - ebase) * R, rec);
               }
             }()),
         ...);
      }(std::make_integer_sequence<int, NP>{});
    }
    __syncthreads();
    if (pair) {
      const int32_t total = (int32_t)(tile_pts * NP);
      for (int32_t q = threadIdx.x; q < total; q += kScatterThreads) {
        float rec[R];
#pragma unroll
        for (int c = 0; c < R; ++c) rec[c] = st_rec[(int64_t)q * R + c];
        store_vec<R>(vseg + (int64_t)(st_pos[q] - ebase) * R, rec);
      }
      __syncthreads();
    }
  }
}

template <int D, int F>
hipError_t launch_bin(const Grid& g, const BinPlan& bp, const BinWorkspace& w, char* ws, bool scatter,
                      int64_t n, const float* x, const float* gg, hipStream_t s) {
  const dim3 grid((unsigned)w.nblk);
  int32_t* counts = reinterpret_cast<int32_t*>(ws + w.counts);
  if (!scatter) {
    hipLaunchKernelGGL((dlinear_count_kernel<D>), grid, dim3(kBinThreads), sizeof(int32_t) * (size_t)bp.nbins, s,
                       g, bp, n, w.tile, w.nblk, x, counts);
    return hipGetLastError();
  }
  const size_t lds = sizeof(int32_t) * (2 * (size_t)bp.nbins + 2 * (size_t)bp.max_seg_bins + kScatterThreads) +
                     (size_t)w.tile * (1 << (D - 1)) * (sizeof(float) * (2 + F) + sizeof(int32_t));
  const int32_t* totals = reinterpret_cast<const int32_t*>(ws + w.totals);
  const int32_t* bin_start = reinterpret_cast<const int32_t*>(ws + w.bin_start);
  const BinState* st = reinterpret_cast<const BinState*>(ws + w.state);
  float* vals = reinterpret_cast<float*>(ws + w.vals);
  if (g.L * F <= 32) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&dlinear_scatter_kernel<D, F, true>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((dlinear_scatter_kernel<D, F, true>), grid, dim3(kScatterThreads), lds, s, g, bp, n, w.tile,
                       w.nblk, x, gg, counts, totals, bin_start, st, vals);
  } else {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&dlinear_scatter_kernel<D, F, false>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((dlinear_scatter_kernel<D, F, false>), grid, dim3(kScatterThreads), lds, s, g, bp, n, w.tile,
                       w.nblk, x, gg, counts, totals, bin_start, st, vals);
  }
  return hipGetLastError();
}

template <int D, int F>
hipError_t launch_fwd(const Grid& g, int64_t n, const float* x, const float* params, float* gamma,
                      float* scratch, hipStream_t s) {
  const int64_t tiles = (n + kBlock - 1) / kBlock;
  if (tiles * g.L > 0x7fffffff) return hipErrorInvalidValue;
  const dim3 grid((unsigned)(tiles * g.L));
  if (!scratch) {
    hipLaunchKernelGGL((dlinear_forward_kernel<D, F, false>), grid, dim3(kBlock), 0, s, g, n, (int32_t)tiles, x,
                       params, gamma);
    return hipGetLastError();
  }
  hipLaunchKernelGGL((dlinear_forward_kernel<D, F, true>), grid, dim3(kBlock), 0, s, g, n, (int32_t)tiles, x,
                     params, scratch);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((level_major_to_rows_kernel<F>), dim3((unsigned)tiles), dim3(kBlock), 0, s, g.L, n, scratch,
                     gamma);
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
                                  const float* params, float* gamma, float* scratch, hipStream_t s) {
  HASHENC_DISPATCH_DF(d, F, launch_fwd, g, n, x, params, gamma, scratch, s);
}

hipError_t launch_dlinear_backward(const Grid& g, int d, int F, int64_t n, const float* x,
                                   const float* g_gamma, float* grad, hipStream_t s) {
  HASHENC_DISPATCH_DF(d, F, launch_bwd, g, n, x, g_gamma, grad, s);
}

hipError_t launch_dlinear_bin(const Grid& g, const BinPlan& bp, const BinWorkspace& w, char* ws, int d, int F,
                              bool scatter, int64_t n, const float* x, const float* g_gamma, hipStream_t s) {
  HASHENC_DISPATCH_DF(d, F, launch_bin, g, bp, w, ws, scatter, n, x, g_gamma, s);
}

}  // namespace hg
