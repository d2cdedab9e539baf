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
template <int D, int F>
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
  store_vec<F>(gamma + p * (int64_t)g.L * F + (int64_t)l * F, acc);
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
// lane) and histograms their corner contributions over all bins in LDS.
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
    const bool few = bp.seg_bin0[l + 1] - bp.seg_bin0[l] <= kFewBins;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t p = p0 + (int64_t)j * kBinThreads;
      if (j >= ppt || p >= n) break;
      uint32_t base[D];
      float t[D];
      locate<D>(xp[j], g.N[l], g.Nf[l], base, t);
      const CellKeys<D> keys = cell_keys<D>(base, g.N[l]);
      [&]<int... C>(std::integer_sequence<int, C...>) {
        ((
             [&] {
               int32_t bin;
               uint32_t local;
               bin_of(bp, 0, l, corner_row<D, C>(keys, dense, g.T[0], g.Tmask[0]), bin, local);
               if (few) wave_aggregated_add<false>(hist, bin);
               else atomicAdd(&hist[bin], 1);
             }()),
         ...);
      }(std::make_integer_sequence<int, 1 << D>{});
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < bp.nbins; i += kBinThreads) counts[(int64_t)i * nblk + blk] = hist[i];
}

// Binned backward, scatter pass.  Per level, the tile's entries are first sorted by bin in
// LDS (a local counting sort seeded with the tile's per-bin counts from the count pass),
// then copied out so that each bin receives one contiguous run: consecutive lanes write
// consecutive rows / values and every cache line is written whole.
// PRE: the tile's upstream rows (L*F <= 32 floats per point) are read once into registers
// before the level loop; otherwise each level reads its F floats of the row.
template <int D, int F, bool PRE>
__global__ __launch_bounds__(kScatterThreads) void dlinear_scatter_kernel(
    const Grid g, const BinPlan bp, int64_t n, int32_t tile, int32_t nblk, const float* __restrict__ x,
    const float* __restrict__ g_gamma, const int32_t* __restrict__ counts,
    const int32_t* __restrict__ totals, const int32_t* __restrict__ bin_start,
    const BinState* __restrict__ st, uint16_t* __restrict__ rows_out, float* __restrict__ vals_out) {
  constexpr int NC = 1 << D;
  extern __shared__ int32_t lds[];
  const int mb = bp.max_seg_bins;
  const int nbins = bp.nbins;
  int32_t* gstart = lds;                 // [nbins] global position of this tile's run in each bin
  int32_t* bcnt = lds + nbins;           // [nbins] this tile's entries in each bin
  int32_t* lstart = lds + 2 * nbins;     // [mb] start of each bin's run in the staging area
  int32_t* lcur = lstart + mb;           // [mb] staging cursors
  int32_t* scan = lcur + mb;             // [kScatterThreads]
  float* st_val = reinterpret_cast<float*>(scan + kScatterThreads);                     // [tile*NC*F]
  int32_t* st_pos = reinterpret_cast<int32_t*>(st_val + (int64_t)tile * NC * F);    // [tile*NC]
  uint16_t* st_row = reinterpret_cast<uint16_t*>(st_pos + (int64_t)tile * NC);      // [tile*NC]

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
    // this tile's count and global start in each bin of the level; exclusive scan of counts
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
    const bool few = nb <= kFewBins;
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
      [&]<int... C>(std::integer_sequence<int, C...>) {
        ((
             [&] {
               int32_t bin;
               uint32_t local;
               bin_of(bp, 0, l, corner_row<D, C>(keys, dense, g.T[0], g.Tmask[0]), bin, local);
               const int i = bin - b0;
               const int32_t lp = few ? wave_aggregated_add<true>(lcur, i) : atomicAdd(&lcur[i], 1);
               float w = 1.0f;
#pragma unroll
               for (int a = 0; a < D; ++a) w *= ((C >> a) & 1) ? t[a] : 1.0f - t[a];
               st_row[lp] = (uint16_t)local;
               st_pos[lp] = gstart[bin] + (lp - lstart[i]);
#pragma unroll
               for (int f = 0; f < F; ++f) st_val[(int64_t)lp * F + f] = w * G[f];
             }()),
         ...);
      }(std::make_integer_sequence<int, NC>{});
    }
    __syncthreads();
    const int32_t ebase = st->seg_ebase[l];
    float* vseg = vals_out + st->seg_vbase[l];
    const int32_t total = (int32_t)(tile_pts * NC);
    for (int32_t q = threadIdx.x; q < total; q += kScatterThreads) {
      const int32_t gp = st_pos[q];
      rows_out[gp] = st_row[q];
      float v[F];
#pragma unroll
      for (int f = 0; f < F; ++f) v[f] = st_val[(int64_t)q * F + f];
      store_vec<F>(vseg + (int64_t)(gp - ebase) * F, v);
    }
    __syncthreads();
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
                     (size_t)w.tile * (1 << D) * (sizeof(float) * F + sizeof(int32_t) + sizeof(uint16_t));
  const int32_t* totals = reinterpret_cast<const int32_t*>(ws + w.totals);
  const int32_t* bin_start = reinterpret_cast<const int32_t*>(ws + w.bin_start);
  const BinState* st = reinterpret_cast<const BinState*>(ws + w.state);
  uint16_t* rows = reinterpret_cast<uint16_t*>(ws + w.rows);
  float* vals = reinterpret_cast<float*>(ws + w.vals);
  if (g.L * F <= 32) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&dlinear_scatter_kernel<D, F, true>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((dlinear_scatter_kernel<D, F, true>), grid, dim3(kScatterThreads), lds, s, g, bp, n, w.tile,
                       w.nblk, x, gg, counts, totals, bin_start, st, rows, vals);
  } else {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&dlinear_scatter_kernel<D, F, false>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((dlinear_scatter_kernel<D, F, false>), grid, dim3(kScatterThreads), lds, s, g, bp, n, w.tile,
                       w.nblk, x, gg, counts, totals, bin_start, st, rows, vals);
  }
  return hipGetLastError();
}

template <int D, int F>
hipError_t launch_fwd(const Grid& g, int64_t n, const float* x, const float* params, float* gamma,
                      hipStream_t s) {
  const int64_t tiles = (n + kBlock - 1) / kBlock;
  if (tiles * g.L > 0x7fffffff) return hipErrorInvalidValue;
  const dim3 grid((unsigned)(tiles * g.L));
  hipLaunchKernelGGL((dlinear_forward_kernel<D, F>), grid, dim3(kBlock), 0, s, g, n, (int32_t)tiles, x, params,
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
                                  const float* params, float* gamma, hipStream_t s) {
  HASHENC_DISPATCH_DF(d, F, launch_fwd, g, n, x, params, gamma, s);
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
