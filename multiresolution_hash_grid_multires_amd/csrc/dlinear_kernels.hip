// Instant-NGP d-linear hash-grid encoding: forward gather + interpolation and backward
// scatter-add, gfx950.
//
// Method: Instant-NGP explainer (nxrte.com), encoding pipeline steps 1-4 (per level, the
// 2^d vertices around x, table lookup, d-linear interpolation, concatenation over levels);
// Instant-NGP news article (antipu.com.cn), efficiency paragraph (no control flow, all
// levels looked up independently) and adaptivity paragraph (colliding gradients combine:
// here they sum).
//
// Mapping: the level loop is wave-uniform so the per-level block description stays in
// scalar registers; the corner gathers of a level are independent loads issued back to
// back; x-adjacent corners usually share a cache line, which the forward exploits by giving
// the two x-corners of a pair to neighbouring lanes.
#include "binned_backward.h"
#include "hashenc_internal.h"
#include "vec_io.h"

namespace hg {
namespace {

// Forward.  Workgroups are ordered by pass: workgroup b handles pass b / n_tiles for the
// b % n_tiles-th tile of points, a pass being one level or a run of consecutive small levels
// whose tables together fit kFwdPassBytes.  Workgroups are dispatched in order, so at any
// moment the whole chip works on one or two passes and each XCD's L2 holds those tables (4 MB
// for a hashed level of 2^19 rows of F = 2) instead of streaming every level's table from
// the Infinity Cache.  x is re-read per pass (12 bytes per point).
// LM_OUT: write level-major [L][n][F] (whole cache lines per workgroup) instead of the
// point-major [n][L*F] rows; without it every level is one pass.
constexpr int64_t kFwdPassBytes = int64_t(3) << 20;

struct FwdPlan {
  int32_t n_pass;
  uint8_t first[kMaxLevels];  // levels [first, last] of a pass
  uint8_t last[kMaxLevels];
};

FwdPlan make_fwd_plan(const Grid& g, int d, int F, bool group, int first = 0) {
  FwdPlan fp;
  fp.n_pass = 0;
  int64_t group_bytes = 0;
  for (int l = first; l < g.L; ++l) {
    int64_t rows = g.T[0];
    if ((g.dense[0] >> l) & 1u) {
      rows = 1;
      for (int i = 0; i < d; ++i) rows *= (int64_t)g.N[l] + 1;
    }
    const int64_t bytes = rows * F * (int64_t)sizeof(float);
    if (group && fp.n_pass > 0 && group_bytes + bytes <= kFwdPassBytes) {
      fp.last[fp.n_pass - 1] = (uint8_t)l;
      group_bytes += bytes;
      continue;
    }
    fp.first[fp.n_pass] = fp.last[fp.n_pass] = (uint8_t)l;
    ++fp.n_pass;
    group_bytes = bytes;
  }
  return fp;
}

// Coarse levels from LDS.  The leading dense levels whose tables fit in LDS together
// (kFwdLdsBytes) are interpolated by one persistent workgroup per CU that copies those
// tables into LDS once and walks its share of the points: these levels then issue no L2
// request per point, and the L2 request rate is what bounds the gather (four line requests
// per point and level).
constexpr int64_t kFwdLdsBytes = 144 * 1024;
constexpr int kFwdLdsThreads = 1024;

int fwd_lds_levels(const Grid& g, int d, int F) {
  int64_t bytes = 0;
  int c = 0;
  for (int l = 0; l < g.L; ++l) {
    if (!((g.dense[0] >> l) & 1u)) break;
    int64_t rows = 1;
    for (int i = 0; i < d; ++i) rows *= (int64_t)g.N[l] + 1;
    if (bytes + rows * F * (int64_t)sizeof(float) > kFwdLdsBytes) break;
    bytes += rows * F * (int64_t)sizeof(float);
    ++c;
  }
  return c;
}

// Levels 0 .. Lc-1 (dense, contiguous in the parameter array) into the level-major staging.
// Two lanes per point as in the L2 gather; both lanes of a point run the same iterations.
template <int D, int F>
__global__ __launch_bounds__(kFwdLdsThreads) void dlinear_forward_lds_kernel(const Grid g, int32_t Lc,
                                                                          int32_t nfloats, int64_t n,
                                                                          const float* __restrict__ x,
                                                                          const float* __restrict__ params,
                                                                          float* __restrict__ stage) {
  extern __shared__ float tab[];
  // table copy in 16-byte pieces, four loads in flight per thread (table 0 level 0 starts at
  // the 16-byte aligned start of the parameters)
  {
    const float4* src4 = reinterpret_cast<const float4*>(params + g.off[0][0]);
    float4* tab4 = reinterpret_cast<float4*>(tab);
    const int n4 = nfloats >> 2;
    for (int i = threadIdx.x; i < n4; i += 4 * kFwdLdsThreads) {
      const int i1 = i + kFwdLdsThreads, i2 = i + 2 * kFwdLdsThreads, i3 = i + 3 * kFwdLdsThreads;
      const float4 a0 = src4[i];
      const float4 a1 = src4[min(i1, n4 - 1)];
      const float4 a2 = src4[min(i2, n4 - 1)];
      const float4 a3 = src4[min(i3, n4 - 1)];
      tab4[i] = a0;
      if (i1 < n4) tab4[i1] = a1;
      if (i2 < n4) tab4[i2] = a2;
      if (i3 < n4) tab4[i3] = a3;
    }
    for (int i = 4 * n4 + threadIdx.x; i < nfloats; i += kFwdLdsThreads) tab[i] = params[g.off[0][0] + i];
  }
  __syncthreads();
  constexpr int PTS = kFwdLdsThreads / 2;
  const int c0 = threadIdx.x & 1;
  const int64_t stride = (int64_t)gridDim.x * PTS;
  int64_t p = (int64_t)blockIdx.x * PTS + (threadIdx.x >> 1);
  float xn[D];  // the next point's coordinates, loaded one iteration ahead
#pragma unroll
  for (int i = 0; i < D; ++i) xn[i] = p < n ? x[p * D + i] : 0.0f;
  for (; p < n; p += stride) {
    float xp[D];
#pragma unroll
    for (int i = 0; i < D; ++i) {
      xp[i] = xn[i];
      xn[i] = p + stride < n ? x[(p + stride) * D + i] : 0.0f;
    }
    int32_t loff = 0;  // the level's table in LDS
    for (int l = 0; l < Lc; ++l) {
      uint32_t base[D];
      float t[D];
      locate<D>(xp, g.N[l], g.Nf[l], base, t);
      const CellKeys<D> keys = cell_keys<D>(base, g.N[l]);
      constexpr int NP = 1 << (D - 1);
      float acc[F];
#pragma unroll
      for (int f = 0; f < F; ++f) acc[f] = 0.0f;
      const float wx = c0 ? t[0] : 1.0f - t[0];
      [&]<int... Y>(std::integer_sequence<int, Y...>) {
        ((
             [&] {
               const uint32_t r = c0 ? corner_row<D, (Y << 1) | 1>(keys, true, g.T[0], g.Tmask[0])
                                     : corner_row<D, (Y << 1)>(keys, true, g.T[0], g.Tmask[0]);
               float w = wx;
#pragma unroll
               for (int i = 1; i < D; ++i) w *= ((Y >> (i - 1)) & 1) ? t[i] : 1.0f - t[i];
#pragma unroll
               for (int f = 0; f < F; ++f) acc[f] = fmaf(w, tab[loff + (int32_t)r * F + f], acc[f]);
             }()),
         ...);
      }(std::make_integer_sequence<int, NP>{});
#pragma unroll
      for (int f = 0; f < F; ++f) acc[f] = add_lane_pair(acc[f]);
      if (c0 == 0) store_vec<F>(stage + ((int64_t)l * n + p) * F, acc);
      int32_t rows = 1;
#pragma unroll
      for (int i = 0; i < D; ++i) rows *= g.N[l] + 1;
      loff += rows * F;
    }
  }
}

// Two lanes per point: lane c0 gathers the 2^(d-1) corners with x-bit c0, so the two corners
// of every x-pair -- adjacent rows on dense levels, rows differing in the low bits on hashed
// levels -- are read by neighbouring lanes of one load instruction and share one L2 request
// whenever they share a cache line.  The lane sums meet through one cross-lane add.
// CNT: also histogram the binned backward's entries of these points over the pass's bins
// (the count pass, from the corner rows the gather computes anyway) and add the workgroup's
// histogram to counts[tile][bin] (ctile points per backward tile, a multiple of the
// workgroup's points).  On pair-mode levels the two x-corners of a pair make one entry and
// share its bin, so each lane counts the pairs whose y/z index has its parity; elsewhere each
// lane counts its own corners.
constexpr int kFwdCntBins = 512;  // LDS counters of one pass's bins (a pass with more counts in the backward)

template <int D, int F, bool LM_OUT, bool CNT>
__global__ __launch_bounds__(kBlock) void dlinear_forward_kernel(const Grid g, const FwdPlan fp, int64_t n,
                                                                 int32_t n_tiles, const float* __restrict__ x,
                                                                 const float* __restrict__ params,
                                                                 float* __restrict__ gamma, const BinPlan bp,
                                                                 int32_t ctile, int32_t* __restrict__ counts) {
  constexpr int PTS = kBlock / 2;  // points per workgroup
  const int pass = blockIdx.x / n_tiles;
  const int l0 = fp.first[pass], l1 = fp.last[pass];
  const int c0 = threadIdx.x & 1;
  const int64_t p = (int64_t)(blockIdx.x % n_tiles) * PTS + (threadIdx.x >> 1);
  [[maybe_unused]] __shared__ int32_t hist[CNT ? kFwdCntBins : 1];
  [[maybe_unused]] int32_t pb0 = 0, pb1 = 0;
  if constexpr (CNT) {
    pb0 = bp.seg_bin0[l0];
    pb1 = bp.seg_bin0[l1 + 1];
    for (int i = threadIdx.x; i < pb1 - pb0; i += kBlock) hist[i] = 0;
    __syncthreads();
  } else {
    if (p >= n) return;  // both lanes of a point leave together
  }
  const bool on = p < n;
  float xp[D];
#pragma unroll
  for (int i = 0; i < D; ++i) xp[i] = x[(on ? p : n - 1) * D + i];
  for (int l = l0; l <= l1; ++l) {
    uint32_t base[D];
    float t[D];
    locate<D>(xp, g.N[l], g.Nf[l], base, t);
    const CellKeys<D> keys = cell_keys<D>(base, g.N[l]);
    const bool dense = (g.dense[0] >> l) & 1u;
    const float* tab = params + g.off[0][l];
    constexpr int NP = 1 << (D - 1);
    float rows[NP][F];
    [[maybe_unused]] uint32_t rr[NP];
    // issue every gather of the level before using any of them
    [&]<int... Y>(std::integer_sequence<int, Y...>) {
      ((
           [&] {
             const uint32_t r = c0 ? corner_row<D, (Y << 1) | 1>(keys, dense, g.T[0], g.Tmask[0])
                                   : corner_row<D, (Y << 1)>(keys, dense, g.T[0], g.Tmask[0]);
             load_vec<F>(tab + (size_t)r * F, rows[Y]);
             if constexpr (CNT) rr[Y] = r;
           }()),
       ...);
    }(std::make_integer_sequence<int, NP>{});
    if constexpr (CNT) {
      if (on) {
        const bool pair = (bp.pair_mask >> l) & 1u;
        const bool few = bp.seg_bin0[l + 1] - bp.seg_bin0[l] <= kFewBins;
#pragma unroll
        for (int y = 0; y < NP; ++y) {
          if (pair && (y & 1) != c0) continue;
          int32_t b;
          uint32_t local;
          bin_of(bp, 0, l, rr[y], b, local);
          if (few) wave_aggregated_add<false>(hist, b - pb0);
          else atomicAdd(&hist[b - pb0], 1);
        }
      }
    }
    float acc[F];
#pragma unroll
    for (int f = 0; f < F; ++f) acc[f] = 0.0f;
    const float wx = c0 ? t[0] : 1.0f - t[0];
#pragma unroll
    for (int y = 0; y < NP; ++y) {
      float w = wx;
#pragma unroll
      for (int i = 1; i < D; ++i) w *= ((y >> (i - 1)) & 1) ? t[i] : 1.0f - t[i];
#pragma unroll
      for (int f = 0; f < F; ++f) acc[f] = fmaf(w, rows[y][f], acc[f]);
    }
#pragma unroll
    for (int f = 0; f < F; ++f) acc[f] = add_lane_pair(acc[f]);
    if (c0 == 0 && on) {
      if constexpr (LM_OUT) store_vec<F>(gamma + ((int64_t)l * n + p) * F, acc);
      else store_vec<F>(gamma + p * (int64_t)g.Lrow * F + (int64_t)l * F, acc);
    }
  }
  if constexpr (CNT) {
    __syncthreads();
    const int64_t row = (int64_t)(blockIdx.x % n_tiles) * PTS / ctile;
    for (int i = threadIdx.x; i < pb1 - pb0; i += kBlock)
      if (hist[i] != 0) atomicAdd(&counts[row * bp.nbins + pb0 + i], hist[i]);
  }
}

// [L][n][F] -> [n][Lrow*F] through LDS.  A workgroup owns P consecutive points: it reads
// the P*F contiguous floats of each level (coalesced runs; 16-byte loads, four in flight per
// lane before the first LDS write, when every run is 16-byte aligned), parks them in LDS as
// P rows of L*F (pitch L*F + 1 keeps the scattered LDS writes free of bank conflicts) and
// writes the P*Lrow*F contiguous output floats as 16-byte pieces, so every output line is
// written whole.  Columns of the inactive levels L..Lrow-1 are written as zeros.
template <int F>
__global__ __launch_bounds__(kBlock) void level_major_to_rows_kernel(int32_t L, int32_t Lrow, int64_t n, int32_t P,
                                                                     const float* __restrict__ lm,
                                                                     float* __restrict__ out) {
  extern __shared__ float tile[];
  const int AF = L * F;     // active columns (held in LDS)
  const int LF = Lrow * F;  // output row
  const int pitch = AF + 1;
  const int64_t p0 = (int64_t)blockIdx.x * P;
  const int np = (int)min((int64_t)P, n - p0);
  const int per_level = np * F;
  if (((n * F) & 3) == 0 && (per_level & 3) == 0 && ((P * F) & 3) == 0) {
    constexpr int U = 4;
    const int q_per = per_level >> 2;  // 16-byte pieces per level
    const int total = L * q_per;
    for (int i0 = threadIdx.x; i0 < total; i0 += U * kBlock) {
      float4 v[U];
      int lv[U], rv[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int i = i0 + u * kBlock;
        lv[u] = i / q_per;
        rv[u] = 4 * (i - lv[u] * q_per);  // float index inside the level's run
        if (i < total) v[u] = *reinterpret_cast<const float4*>(lm + ((int64_t)lv[u] * n + p0) * F + rv[u]);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (i0 + u * kBlock >= total) break;
        const float e[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
        for (int k = 0; k < 4; ++k) tile[((rv[u] + k) / F) * pitch + lv[u] * F + (rv[u] + k) % F] = e[k];
      }
    }
  } else {
    for (int i = threadIdx.x; i < L * per_level; i += kBlock) {
      const int l = i / per_level, r = i - l * per_level;
      tile[(r / F) * pitch + l * F + r % F] = lm[((int64_t)l * n + p0) * F + r];
    }
  }
  __syncthreads();
  float* dst = out + p0 * LF;
  if ((LF & 3) == 0) {  // every row, hence the block's output, is 16-byte aligned
    const int q4 = LF >> 2;  // 16-byte pieces per row
    for (int q = threadIdx.x; q < np * q4; q += kBlock) {
      const int pt = q / q4, c = 4 * (q - pt * q4);
      float v[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) v[k] = c + k < AF ? tile[pt * pitch + c + k] : 0.0f;
      reinterpret_cast<float4*>(dst)[q] = make_float4(v[0], v[1], v[2], v[3]);
    }
  } else {
    const int total = np * LF;
    for (int e = threadIdx.x; e < total; e += kBlock) {
      const int c = e % LF;
      dst[e] = c < AF ? tile[(e / LF) * pitch + c] : 0.0f;
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
// u_lm: the upstream level-major ([L][n][F]) instead of the rows of g_gamma, or NULL.
template <int D, int F>
__global__ __launch_bounds__(kBlock) void dlinear_backward_kernel(const Grid g, int64_t n,
                                                                  const float* __restrict__ x,
                                                                  const float* __restrict__ g_gamma,
                                                                  const float* __restrict__ u_lm,
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
  const int64_t LF = (int64_t)g.Lrow * F;
  const float* up = u_lm ? u_lm + p * F + f : g_gamma + p * LF + f;
  const int64_t lstride = u_lm ? n * F : F;  // floats between a point's levels
  for (int l = 0; l < g.L; ++l) {
    const float G = up[(int64_t)l * lstride];
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

// Binned backward, count pass: a workgroup of TPB lanes owns a tile of `tile` = 2 TPB points
// (two per lane) and one group of lpg levels (blockIdx.y), and histograms their entries over
// that group's bins in LDS.  On pair-mode levels the two x-corners of each (y, z) corner pair
// make one entry (they always share a bin); elsewhere each corner is its own entry.
// zero_rest: also zero the tile's counters of every later bin (whose levels the counting
// forward then adds with atomics).
template <int D, int TPB>
__global__ __launch_bounds__(TPB) void dlinear_count_kernel(const Grid g, const BinPlan bp, int64_t n, int32_t tile,
                                                            int32_t nblk, int32_t lpg, const float* __restrict__ x,
                                                            int32_t* __restrict__ counts, int32_t zero_rest) {
  extern __shared__ int32_t hist[];
  const int blk = bin_tile_of_block(blockIdx.x, nblk);
  const int l0 = blockIdx.y * lpg, l1 = min(g.L, l0 + lpg);
  const int32_t gb0 = bp.seg_bin0[l0], gb1 = bp.seg_bin0[l1];
  for (int i = gb0 + threadIdx.x; i < gb1; i += TPB) hist[i] = 0;
  __syncthreads();
  constexpr int PPT = 2;  // points per lane
  const int64_t p0 = (int64_t)blk * tile + threadIdx.x;
  // both points' coordinates in flight at once (lanes past the end re-read the last point and
  // skip it below): a guarded load per coordinate would wait for each before the next
  float xp[PPT][D];
#pragma unroll
  for (int j = 0; j < PPT; ++j) {
    const int64_t p = min(p0 + (int64_t)j * TPB, n - 1);
#pragma unroll
    for (int i = 0; i < D; ++i) xp[j][i] = x[p * D + i];
  }
  for (int l = l0; l < l1; ++l) {
    const bool dense = (g.dense[0] >> l) & 1u;
    const bool pair = (bp.pair_mask >> l) & 1u;
    const bool few = bp.seg_bin0[l + 1] - bp.seg_bin0[l] <= kFewBins;
#pragma unroll
    for (int j = 0; j < PPT; ++j) {
      const int64_t p = p0 + (int64_t)j * TPB;
      if (p >= n) break;
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
  const int32_t ge = zero_rest ? bp.nbins : gb1;
  for (int i = gb0 + threadIdx.x; i < ge; i += TPB) counts[(int64_t)blk * bp.nbins + i] = i < gb1 ? hist[i] : 0;
}

// G = up[l*F .. l*F + F) for a wave-uniform l < 32 / F: per feature, a tournament over the
// 32 / F candidates on the bits of l (15 selects for F = 2), with compile-time register
// indices only, since indexing the register array by l can demote it to scratch.
template <int F>
__device__ __forceinline__ void pick_group(const float (&up)[32], int l, float (&G)[F]) {
  constexpr int K = 32 / F;
#pragma unroll
  for (int f = 0; f < F; ++f) {
    float c[K / 2 > 0 ? K / 2 : 1];
    const bool top = (l & (K / 2)) != 0;
#pragma unroll
    for (int j = 0; j < K / 2; ++j) c[j] = top ? up[(j + K / 2) * F + f] : up[j * F + f];
#pragma unroll
    for (int half = K / 4; half >= 1; half /= 2) {
      const bool hi = (l & half) != 0;
#pragma unroll
      for (int j = 0; j < half; ++j) c[j] = hi ? c[j + half] : c[j];
    }
    G[f] = c[0];
  }
}

// Binned backward, scatter pass.  One lane per point (TPB = tile).  At the start the workgroup turns the
// tile's per-bin counts (from the count pass) into an exclusive prefix over all bins, which
// is both each bin's slot range in the LDS staging area (relative to the level's first bin)
// and its cursor.  Per level, the tile's pair records are sorted by bin in LDS and then
// copied out so that each bin receives one contiguous run: consecutive lanes write
// consecutive records and cache lines are written whole.  Single-corner records (levels
// not in pair mode) are written straight to their slots.
// PRE: the workgroup's part of the point's upstream row (lpg*F <= 32 floats, a multiple of 4,
// from column l0*F) is read once into registers before the level loop; otherwise each level
// reads its F floats of the row, or of the level-major upstream u_lm when given.
template <int D, int F, bool PRE, int TPB>
__global__ __launch_bounds__(TPB) void dlinear_scatter_kernel(
    const Grid g, const BinPlan bp, int64_t n, int32_t tile, int32_t nblk, int32_t lpg, const float* __restrict__ x,
    const float* __restrict__ g_gamma, const float* __restrict__ u_lm, const int32_t* __restrict__ counts,
    const int32_t* __restrict__ totals, const int32_t* __restrict__ bin_start,
    const BinState* __restrict__ st, float* __restrict__ vals_out, uint32_t* __restrict__ vmax) {
  constexpr int NP = 1 << (D - 1);  // x-corner pairs per cell
  constexpr int R = 2 + F;          // floats per record
  extern __shared__ int32_t lds[];
  const int nbins = bp.nbins;
  // A record given slot s of bin b (s counts from the bin's first slot in the tile's
  // exclusive prefix) goes to entry delta[b] + s: delta is the bin's global start for this
  // tile minus that first slot.
  int32_t* delta = lds;                   // [nbins]
  int32_t* lcur = lds + nbins;            // [nbins] slot cursors: the tile's exclusive prefix
  int32_t* wsum = lds + 2 * nbins;        // [TPB / 64]
  int32_t* lbase = wsum + TPB / 64;  // [kMaxLevels] first staging slot of each level
  // staged records start 16-byte aligned so each record moves with the widest LDS access
  float* st_rec = reinterpret_cast<float*>(lds + ((2 * nbins + TPB / 64 + kMaxLevels + 3) & ~3));
  int32_t* st_pos = reinterpret_cast<int32_t*>(st_rec + (int64_t)tile * NP * R);  // [tile*NP]

  __shared__ uint32_t vsh[kMaxSeg];  // the workgroup's segment (= level) bounds
  for (int i = threadIdx.x; i < kMaxSeg; i += TPB) vsh[i] = 0u;
  const int blk = bin_tile_of_block(blockIdx.x, nblk);
  const int64_t p = (int64_t)blk * tile + threadIdx.x;
  const bool on = p < n;
  const int np = (int)min((int64_t)tile, n - (int64_t)blk * tile);
  // Every store below lands inside the chunk's entries and staging even when the counts do
  // not describe these points (counts left by a counting forward on other x): per level a
  // tile has np * NP pair records (2 np NP single ones) whatever x is, so only the bins of
  // mismatched records are wrong; the guards keep them in bounds (the gradient is then wrong).
  const int32_t etot = bin_start[nbins];
  // this workgroup's levels and their bins (all of them unless the levels are split)
  const int l0 = blockIdx.y * lpg, l1 = min(g.L, l0 + lpg);
  const int32_t gb0 = bp.seg_bin0[l0], gb1 = bp.seg_bin0[l1];
  for (int i = gb0 + threadIdx.x; i < gb1; i += TPB) {
    const int32_t pre = counts[(int64_t)blk * nbins + i];
    const int32_t nxt = blk + 1 < nblk ? counts[(int64_t)(blk + 1) * nbins + i] : totals[i];
    delta[i] = bin_start[i] + pre;
    lcur[i] = nxt - pre;
  }
  __syncthreads();
  block_exclusive_scan<TPB>(lcur + gb0, gb1 - gb0, wsum);
  for (int i = gb0 + threadIdx.x; i < gb1; i += TPB) delta[i] -= lcur[i];
  for (int i = l0 + threadIdx.x; i < l1; i += TPB) lbase[i] = lcur[bp.seg_bin0[i]];
  float xp[D];
#pragma unroll
  for (int i = 0; i < D; ++i) xp[i] = on ? x[p * D + i] : 0.0f;
  const int64_t LF = (int64_t)g.Lrow * F;
  float up[PRE ? 32 : 1];
  if constexpr (PRE) {
    const int gf = (l1 - l0) * F;  // floats of this workgroup's levels
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      float4 a = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
      if (on && g_gamma && 4 * q < gf) a = reinterpret_cast<const float4*>(g_gamma + p * LF + (int64_t)l0 * F)[q];
      up[4 * q] = a.x; up[4 * q + 1] = a.y; up[4 * q + 2] = a.z; up[4 * q + 3] = a.w;
    }
  }
  __syncthreads();
  for (int l = l0; l < l1; ++l) {
    const int32_t b0 = bp.seg_bin0[l];
    const int nb = bp.seg_bin0[l + 1] - b0;
    const int32_t lb = lbase[l];  // staging slots of this level start here
    const bool dense = (g.dense[0] >> l) & 1u;
    const bool pair = (bp.pair_mask >> l) & 1u;
    const bool few = nb <= kFewBins;
    const int32_t ebase = st->seg_ebase[l];
    float* vseg = vals_out + st->seg_vbase[l];
    // bound on the values the level's records add to rows: each is t aG or (1 - t) aG with a
    // weight a <= 1, so max |G| bounds them
    uint32_t vm = 0u;
    if (on) {
      uint32_t base[D];
      float t[D];
      locate<D>(xp, g.N[l], g.Nf[l], base, t);
      const CellKeys<D> keys = cell_keys<D>(base, g.N[l]);
      float G[F];
      if constexpr (PRE) {
        // register array indexed by the wave-uniform level: select with a small unrolled scan
#pragma unroll
        for (int f = 0; f < F; ++f) {
          float v = 0.0f;
#pragma unroll
          for (int c = f; c < 32; c += F)
            if (c == (l - l0) * F + f) v = up[c];
          G[f] = v;
        }
      } else if (u_lm) {
        load_vec<F>(u_lm + ((int64_t)l * n + p) * F, G);  // level-major: coalesced per level
      } else if (g_gamma) {
        load_vec<F>(g_gamma + p * LF + (int64_t)l * F, G);
      } else {
#pragma unroll
        for (int f = 0; f < F; ++f) G[f] = 0.0f;
      }
#pragma unroll
      for (int f = 0; f < F; ++f) vm = max(vm, abs_bits(G[f]));
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
                 const int32_t s0 = few ? wave_aggregated_add<true>(lcur, bn0) : atomicAdd(&lcur[bn0], 1);
                 const int32_t lp = s0 - lb;
                 rec[0] = __uint_as_float(lo | (hi << 16));
                 rec[1] = t[0];
                 if ((uint32_t)lp < (uint32_t)(np * NP)) {
                   store_vec<R>(st_rec + (int64_t)lp * R, rec);
                   st_pos[lp] = delta[bn0] + s0;
                 }
               } else {
                 // two single-corner records, lower row gets (1 - t) aG
                 const int32_t s0 = few ? wave_aggregated_add<true>(lcur, bn0) : atomicAdd(&lcur[bn0], 1);
                 rec[0] = __uint_as_float(lo | 0xFFFF0000u);
                 rec[1] = t[0];
                 const int32_t e0 = delta[bn0] + s0;
                 if ((uint32_t)e0 < (uint32_t)etot) store_vec<R>(vseg + (int64_t)(e0 - ebase) * R, rec);
                 const int32_t s1 = few ? wave_aggregated_add<true>(lcur, bn1) : atomicAdd(&lcur[bn1], 1);
                 rec[0] = __uint_as_float(hi | 0xFFFF0000u);
                 rec[1] = 1.0f - t[0];
                 const int32_t e1 = delta[bn1] + s1;
                 if ((uint32_t)e1 < (uint32_t)etot) store_vec<R>(vseg + (int64_t)(e1 - ebase) * R, rec);
               }
             }()),
         ...);
      }(std::make_integer_sequence<int, NP>{});
    }
    raise_seg_vmax(vsh, l, vm);
    if (pair) {  // uniform over the workgroup
      __syncthreads();
      const int32_t total = np * NP;
      for (int32_t q = threadIdx.x; q < total; q += TPB) {
        float rec[R];
        load_vec<R>(st_rec + (int64_t)q * R, rec);
        const int32_t e = st_pos[q];
        if ((uint32_t)e < (uint32_t)etot) store_vec<R>(vseg + (int64_t)(e - ebase) * R, rec);
      }
      __syncthreads();
    }
  }
  __syncthreads();
  publish_seg_vmax(vsh, bp.nseg, vmax);
}

template <int D, int F, int TPB>
hipError_t launch_bin_tile(const Grid& g, const BinPlan& bp, const BinWorkspace& w, char* ws, bool scatter,
                           int64_t n, const float* x, const float* gg, const float* u_lm, hipStream_t s) {
  const dim3 grid((unsigned)w.nblk, (unsigned)w.lgroups);
  int32_t* counts = reinterpret_cast<int32_t*>(ws + w.counts);
  if (!scatter) {  // two points per count lane
    if (w.tile != TPB) return hipErrorInvalidValue;
    hipLaunchKernelGGL((dlinear_count_kernel<D, TPB / 2>), grid, dim3(TPB / 2), sizeof(int32_t) * (size_t)bp.nbins,
                       s, g, bp, n, w.tile, w.nblk, w.lpg, x, counts, 0);
    return hipGetLastError();
  }
  const size_t lds = dlinear_scatter_lds_bytes(bp, D, F, w.tile);
  const int32_t* totals = reinterpret_cast<const int32_t*>(ws + w.totals);
  const int32_t* bin_start = reinterpret_cast<const int32_t*>(ws + w.bin_start);
  const BinState* st = reinterpret_cast<const BinState*>(ws + w.state);
  float* vals = reinterpret_cast<float*>(ws + w.vals);
  uint32_t* vmax = reinterpret_cast<BinState*>(ws + w.state)->vmax_bits;
  // PRE reads the group's part of the row as 16-byte pieces: rows and groups of a multiple of
  // 4 floats only, so that every piece is aligned and inside the row
  if (!u_lm && w.lpg * F <= 32 && (w.lpg * F) % 4 == 0 && (g.Lrow * F) % 4 == 0) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&dlinear_scatter_kernel<D, F, true, TPB>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((dlinear_scatter_kernel<D, F, true, TPB>), grid, dim3(TPB), lds, s, g, bp, n, w.tile, w.nblk,
                       w.lpg, x, gg, nullptr, counts, totals, bin_start, st, vals, vmax);
  } else {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&dlinear_scatter_kernel<D, F, false, TPB>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((dlinear_scatter_kernel<D, F, false, TPB>), grid, dim3(TPB), lds, s, g, bp, n, w.tile,
                       w.nblk, w.lpg, x, gg, u_lm, counts, totals, bin_start, st, vals, vmax);
  }
  return hipGetLastError();
}

template <int D, int F>
hipError_t launch_bin(const Grid& g, const BinPlan& bp, const BinWorkspace& w, char* ws, bool scatter,
                      int64_t n, const float* x, const float* gg, const float* u_lm, hipStream_t s) {
  if (w.tile == kScatterTileLarge)
    return launch_bin_tile<D, F, kScatterTileLarge>(g, bp, w, ws, scatter, n, x, gg, u_lm, s);
  if (w.tile == kScatterTileSmall)
    return launch_bin_tile<D, F, kScatterTileSmall>(g, bp, w, ws, scatter, n, x, gg, u_lm, s);
  return hipErrorInvalidValue;
}

// The counting forward's backward workspace: plan, layout and base (all NULL: no counting).
struct FwdCounts {
  const BinPlan* bp;
  const BinWorkspace* w;
  char* ws;
};

template <int D, int F>
hipError_t launch_fwd(const Grid& g, int64_t n, const float* x, const float* params, float* gamma,
                      float* scratch, hipStream_t s, const FwdCounts& cnt) {
  const int64_t tiles = (n + kBlock / 2 - 1) / (kBlock / 2);  // two lanes per point
  // with the level-major staging, the leading dense levels that fit in LDS go to the LDS kernel
  const int Lc = scratch ? fwd_lds_levels(g, D, F) : 0;
  const FwdPlan fp = make_fwd_plan(g, D, F, scratch != nullptr, Lc);
  if (tiles * fp.n_pass > 0x7fffffff) return hipErrorInvalidValue;
  const dim3 grid((unsigned)(tiles * fp.n_pass));
  BinPlan nobp;
  nobp.nbins = 0;
  if (!scratch) {
    hipLaunchKernelGGL((dlinear_forward_kernel<D, F, false, false>), grid, dim3(kBlock), 0, s, g, fp, n,
                       (int32_t)tiles, x, params, gamma, nobp, 0, nullptr);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || g.L == g.Lrow) return e;
    return launch_zero_columns(gamma, n, g.Lrow * F, g.L * F, s);
  }
  hipError_t e = hipSuccess;
  int32_t* counts = cnt.ws ? reinterpret_cast<int32_t*>(cnt.ws + cnt.w->counts) : nullptr;
  if (counts && n > 0) {
    // the LDS kernel's levels 0 .. Lc-1 by the count kernel, which also zeroes every later
    // counter of its tile for the forward's atomics
    const BinWorkspace& w = *cnt.w;
    const int tpb = w.tile / 2;
    const size_t hist = sizeof(int32_t) * (size_t)cnt.bp->nbins;
    if (tpb == kScatterTileLarge / 2)
      hipLaunchKernelGGL((dlinear_count_kernel<D, kScatterTileLarge / 2>), dim3((unsigned)w.nblk, 1), dim3(tpb), hist,
                         s, g, *cnt.bp, n, w.tile, w.nblk, (int32_t)Lc, x, counts, 1);
    else if (tpb == kScatterTileSmall / 2)
      hipLaunchKernelGGL((dlinear_count_kernel<D, kScatterTileSmall / 2>), dim3((unsigned)w.nblk, 1), dim3(tpb), hist,
                         s, g, *cnt.bp, n, w.tile, w.nblk, (int32_t)Lc, x, counts, 1);
    else
      return hipErrorInvalidValue;
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (Lc > 0 && n > 0) {
    int32_t nfl = 0;
    for (int l = 0; l < Lc; ++l) {
      int32_t rows = 1;
      for (int i = 0; i < D; ++i) rows *= g.N[l] + 1;
      nfl += rows * F;
    }
    const size_t lds = sizeof(float) * (size_t)nfl;
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(&dlinear_forward_lds_kernel<D, F>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    const int64_t blocks = std::min<int64_t>(256, (n + kFwdLdsThreads / 2 - 1) / (kFwdLdsThreads / 2));
    hipLaunchKernelGGL((dlinear_forward_lds_kernel<D, F>), dim3((unsigned)blocks), dim3(kFwdLdsThreads), lds, s, g,
                       (int32_t)Lc, nfl, n, x, params, scratch);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (fp.n_pass > 0) {
    if (counts)
      hipLaunchKernelGGL((dlinear_forward_kernel<D, F, true, true>), grid, dim3(kBlock), 0, s, g, fp, n,
                         (int32_t)tiles, x, params, scratch, *cnt.bp, cnt.w->tile, counts);
    else
      hipLaunchKernelGGL((dlinear_forward_kernel<D, F, true, false>), grid, dim3(kBlock), 0, s, g, fp, n,
                         (int32_t)tiles, x, params, scratch, nobp, 0, nullptr);
    e = hipGetLastError();
  }
  if (e != hipSuccess || !gamma) return e;  // no gamma: the level-major staging is the output
  const int32_t P = g.L * F <= 128 ? 64 : 32;  // LDS tile at most 32 x 257 floats
  const size_t lds = sizeof(float) * (size_t)P * (g.L * F + 1);
  hipLaunchKernelGGL((level_major_to_rows_kernel<F>), dim3((unsigned)((n + P - 1) / P)), dim3(kBlock), lds, s, g.L,
                     g.Lrow, n, P, scratch, gamma);
  return hipGetLastError();
}

template <int D, int F>
hipError_t launch_bwd(const Grid& g, int64_t n, const float* x, const float* gg, const float* u_lm, float* grad,
                      hipStream_t s) {
  const int64_t lanes = n * 2 * F;
  const dim3 grid((unsigned)((lanes + kBlock - 1) / kBlock));
  hipLaunchKernelGGL((dlinear_backward_kernel<D, F>), grid, dim3(kBlock), 0, s, g, n, x, gg, u_lm, grad);
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

size_t dlinear_forward_workspace_bytes(const Grid& g, int d, int F, int64_t n) {
  (void)d;
  return sizeof(float) * (size_t)n * g.L * F;
}

hipError_t launch_dlinear_forward(const Grid& g, int d, int F, int64_t n, const float* x,
                                  const float* params, float* gamma, float* scratch, hipStream_t s) {
  const FwdCounts none{nullptr, nullptr, nullptr};
  HASHENC_DISPATCH_DF(d, F, launch_fwd, g, n, x, params, gamma, scratch, s, none);
}

bool dlinear_forward_counts(const Grid& g, int d, int F) {
  if (!binned_fits(g, d, F, false)) return false;
  BinPlan bp;
  make_bin_plan(g, d, F, false, bp);
  const int Lc = fwd_lds_levels(g, d, F);
  const FwdPlan fp = make_fwd_plan(g, d, F, true, Lc);
  for (int i = 0; i < fp.n_pass; ++i)
    if (bp.seg_bin0[fp.last[i] + 1] - bp.seg_bin0[fp.first[i]] > kFwdCntBins) return false;
  return true;
}

hipError_t launch_dlinear_forward_counting(const Grid& g, int d, int F, int64_t n, const float* x,
                                           const float* params, float* gamma, float* scratch, void* bws,
                                           hipStream_t s) {
  if (n > bin_chunk_points(g, d, false)) return hipErrorInvalidValue;  // one chunk of the backward
  BinPlan bp;
  make_bin_plan(g, d, F, false, bp);
  const BinWorkspace w = bin_workspace_for(g, bp, d, F, false, n);
  const FwdCounts cnt{&bp, &w, static_cast<char*>(bws)};
  HASHENC_DISPATCH_DF(d, F, launch_fwd, g, n, x, params, gamma, scratch, s, cnt);
}

hipError_t launch_dlinear_backward(const Grid& g, int d, int F, int64_t n, const float* x,
                                   const float* g_gamma, const float* u_levels, float* grad, hipStream_t s) {
  HASHENC_DISPATCH_DF(d, F, launch_bwd, g, n, x, g_gamma, u_levels, grad, s);
}

hipError_t launch_dlinear_bin(const Grid& g, const BinPlan& bp, const BinWorkspace& w, char* ws, int d, int F,
                              bool scatter, int64_t n, const float* x, const float* g_gamma,
                              const float* u_levels, hipStream_t s) {
  HASHENC_DISPATCH_DF(d, F, launch_bin, g, bp, w, ws, scatter, n, x, g_gamma, u_levels, s);
}

}  // namespace hg
