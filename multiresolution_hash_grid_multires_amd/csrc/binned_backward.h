// Binned backward: plan, workspace layout and device helpers shared by the generic stages
// (scan, plan, reduce) and the interpolant-specific count / scatter kernels.
#pragma once

#include "hashenc_internal.h"

namespace hg {

constexpr int kMaxBinTables = 5;                  // order tables of the binned backward (d <= 4)
constexpr int kMaxSeg = kMaxBinTables * kMaxLevels;  // segment s = table k * L + level l
constexpr int kBinLdsValues = 16384;              // 128 KB fp64 LDS accumulator per work item
constexpr int kBinLdsValuesSmall = 2048;          // 16 KB accumulator for grids with small bins
constexpr int kBinThreads = 256;
constexpr int kBinItemEntries = 1 << 18;          // entries per reduce work item (at most)
constexpr int kBinItemMin = 1 << 12;              // ... and at least, when bins are split

// Entries per reduce work item for a chunk of `entries` entries: about 512 items, so small
// problems still spread over every CU, between kBinItemMin and kBinItemEntries.
inline int32_t bin_item_entries(int64_t entries) {
  int64_t e = entries / 512;
  if (e < kBinItemMin) e = kBinItemMin;
  if (e > kBinItemEntries) e = kBinItemEntries;
  return (int32_t)e;
}
constexpr int kReduceThreads = 1024;
constexpr int kBinReduceBlocks = 256;             // persistent reduce workgroups (1 per CU)
// d-linear scatter workgroup = tile: one point per lane.  Larger tiles give each bin longer
// runs per tile (whole lines written); the larger size is used when its LDS staging fits.
constexpr int kScatterTileLarge = 1024;
constexpr int kScatterTileSmall = 512;
constexpr size_t kMaxScatterLds = 150 * 1024;     // of the 160 KB LDS of a gfx950 CU
// Below this many entries per bin on average the reduce walks its items in a static order
// (all items short: the per-item round trips, not balance, set the time).
constexpr int64_t kSparseBinEntries = 4096;

// Small, by-value plan: bins are (segment, chunk of rows) in segment order.  A chunk has
// 2^cshift rows, except on dense d-linear segments in pair mode, where it holds whole
// x-lines (seg_chunk rows, not a power of two) so that x-neighbour rows never straddle.
//
// Entries of d-linear segments are records {uint32 rows, float t, float aG[F]}: rows packs
// the chunk-local row of the x-corner pair's lower (c0 = 0) corner in the low 16 bits and
// the upper corner's in the high 16 bits (0xFFFF: a single corner); the lower row receives
// (1 - t) * aG and the upper t * aG.  Entries of Hermite segments are {uint32 local row,
// float v[W]} (hermite_rec_width(W) floats).  Either way the row index travels
// as the bits of the record's first float, so every entry is written and read as one
// contiguous record.
struct BinPlan {
  int32_t d, L, ntab, nseg, nbins;
  int32_t records;              // 1: d-linear records (2 + F floats); 0: Hermite (1 + W floats)
  int32_t max_seg_bins;         // most bins of any one segment
  int32_t max_level_bins;       // most bins of the segments of any one level (all tables)
  int32_t width[kMaxTables];    // floats per row of table k
  int32_t cshift[kMaxTables];   // log2 rows per chunk of table k (power-of-two chunks)
  uint32_t pair_mask;           // d-linear: bit l set = level l uses x-corner pair records
  // Hermite with equal table sizes: every order table maps a vertex to the same row, so the
  // count pass histograms rows once per level in chunks of 2^fine_shift rows (the narrowest
  // chunk) and derives each table's bin counts by summing consecutive fine bins.  -1: off.
  int32_t fine_shift;
  int32_t fine_bin0[kMaxLevels + 1];
  int32_t seg_chunk[kMaxSeg];   // rows per chunk of segment s
  int32_t seg_bin0[kMaxSeg + 1];
};

// Floats per Hermite record of a W-wide row: the row word and the W values.
__host__ __device__ constexpr int hermite_rec_width(int W) { return W + 1; }
// Floats per record in the scatter's LDS staging: the record, its entry index and padding to
// a whole number of 16-byte words, so a record moves with 16-byte LDS accesses.
__host__ __device__ constexpr int hermite_stage_width(int W) { return (hermite_rec_width(W) + 1 + 3) & ~3; }
// Value floats of every segment start on a 128-byte boundary.
constexpr int64_t kSegAlignFloats = 32;

struct WorkItem {
  int32_t bin, seg, begin, end, split;
};

// Device-side results of the plan stage.
struct BinState {
  int32_t n_items;
  int32_t next_item;
  // Per segment s: an upper bound on |v| over every value the chunk's records of segment s
  // add to a row, as fp32 bits (non-negative floats order like their bit patterns; inf and
  // NaN lie above every finite bound).  Zeroed by the plan stage, raised by the scatter, read
  // by the reduce to pick each work item's fixed-point scale.
  uint32_t vmax_bits[kMaxSeg];
  int32_t seg_ebase[kMaxSeg];   // first entry of segment s
  int64_t seg_vbase[kMaxSeg];   // first value float of segment s
};

// |v| as its fp32 bit pattern: the unsigned maximum of these is the bits of max |v|, with
// NaN (and inf) above every finite value, which a float max would drop.
__device__ __forceinline__ uint32_t abs_bits(float v) { return __float_as_uint(v) & 0x7fffffffu; }

// Bound on |value| of a Hermite record per unit of upstream: every record value is
// sum_o u_o * dO_o/dtheta over the level's outputs o (gamma, d first derivatives, the d
// second derivatives of the diagonal or their sum), and per axis the cubic Hermite factors
// are at most 1 (value; a derivative slot carries Delta x = 1/N), 1.5 N (first derivative)
// and 6 N^2 (second derivative), so |value| <= max|u| (1 + 1.5 d N + 6 d N^2); doubled to
// cover the fp32 rounding of the factor chains.  While this bound is finite no value
// overflows, so the largest value written (which a float max over the values finds, NaN
// aside) is a finite bound; where it is not, the level's segments get a NaN bound.
__device__ __forceinline__ float hermite_value_bound(float N, int d) {
  return 2.0f * (1.0f + 1.5f * (float)d * N + 6.0f * (float)d * N * N);
}
// 0, or NaN bits when max|u| (as abs_bits) times the level's bound is not finite
__device__ __forceinline__ uint32_t hermite_nonfinite_floor(uint32_t ubits, float N, int d) {
  return __uint_as_float(ubits) * hermite_value_bound(N, d) < __builtin_inff() ? 0u : 0x7fc00000u;
}

// Largest m over the wavefront (all 64 lanes active), in every lane: DPP row shifts build
// each 16-lane row's running max, two row broadcasts carry it across rows, lane 63 ends with
// the whole wavefront's.  VALU only -- a chain of cross-lane LDS permutes costs a round trip
// per step, which the scatter's wavefronts cannot hide.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t m) {
  int v = (int)m;
  v = (int)max((uint32_t)v, (uint32_t)__builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, true));  // row_shr:1
  v = (int)max((uint32_t)v, (uint32_t)__builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, true));  // row_shr:2
  v = (int)max((uint32_t)v, (uint32_t)__builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, true));  // row_shr:4
  v = (int)max((uint32_t)v, (uint32_t)__builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, true));  // row_shr:8
  v = (int)max((uint32_t)v, (uint32_t)__builtin_amdgcn_update_dpp(v, v, 0x142, 0xa, 0xf, false));  // row_bcast:15
  v = (int)max((uint32_t)v, (uint32_t)__builtin_amdgcn_update_dpp(v, v, 0x143, 0xc, 0xf, false));  // row_bcast:31
  return (uint32_t)__builtin_amdgcn_readlane(v, 63);
}

// Segment bounds of a scatter workgroup: raised per wavefront in LDS (vsh[kMaxSeg], zeroed
// before the workgroup's first barrier), added to the chunk's bounds once per workgroup.
// Every lane of the wavefront calls raise_seg_vmax.
__device__ __forceinline__ void raise_seg_vmax(uint32_t* vsh, int s, uint32_t m) {
  m = wave_max_u32(m);
  if (__lane_id() == 0 && m != 0u) atomicMax(&vsh[s], m);
}
// after a barrier that follows the last raise_seg_vmax
__device__ __forceinline__ void publish_seg_vmax(const uint32_t* vsh, int nseg, uint32_t* vmax) {
  for (int i = (int)threadIdx.x; i < nseg; i += (int)blockDim.x)
    if (vsh[i] != 0u) atomicMax(&vmax[i], vsh[i]);
}

struct BinWorkspace {
  int32_t tile;   // points per count / scatter workgroup
  int32_t nblk;
  // Levels are split over lgroups workgroups per tile (lpg levels each) when there are too
  // few tiles to fill the chip: a workgroup's levels run one after the other, so a small
  // batch would otherwise wait on the per-level chain of a few workgroups.
  int32_t lgroups, lpg;
  int64_t max_items;
  int32_t item_entries;  // entries per reduce work item
  size_t counts, totals, seg_sums, state, bin_start, items, vals, ups, total;
};

__host__ __device__ inline int64_t seg_rows(const Grid& g, int d, int k, int l) {
  if ((g.dense[k] >> l) & 1u) {
    int64_t r = 1;
    for (int i = 0; i < d; ++i) r *= (int64_t)g.N[l] + 1;
    return r;
  }
  return (int64_t)g.T[k];
}

// Add 1 to hist[bin] for every active lane; lanes of the wavefront that share a bin are
// combined first (one LDS atomic per distinct bin).  With RTN the lane's own slot is
// returned: the counter's old value plus its rank among the lanes sharing the bin.  Used
// where a level has few bins, so that a wavefront's lanes would otherwise serialise on one
// LDS address.
template <bool RTN>
__device__ __forceinline__ int32_t wave_aggregated_add(int32_t* hist, int32_t bin) {
  const int lane = (int)__lane_id();
  int32_t result = 0;
  uint64_t todo = __ballot(1);
  while (todo) {
    const int leader = __ffsll((unsigned long long)todo) - 1;
    const int32_t b = __shfl(bin, leader);
    const uint64_t same = __ballot(bin == b) & todo;
    int32_t base = 0;
    if (lane == leader) base = atomicAdd(&hist[b], (int32_t)__popcll(same));
    if constexpr (RTN) {
      base = __shfl(base, leader);
      if (bin == b) result = base + (int32_t)__popcll(same & ((uint64_t(1) << lane) - 1));
    }
    todo &= ~same;
  }
  return result;
}

// Tile handled by workgroup b of an nblk-workgroup count or scatter launch.  Workgroups are
// dealt round-robin to the 8 XCDs (b % 8), so this hands each XCD a contiguous range of
// tiles: the runs that neighbouring tiles write into one bin are adjacent in memory, and
// partially written cache lines at run boundaries then meet in one XCD's L2.
__device__ __forceinline__ int bin_tile_of_block(int b, int nblk) {
  const int q = nblk / 8;
  if (b >= 8 * q) return b;  // the last nblk % 8 tiles, in order
  return (b % 8) * q + b / 8;
}

// Exclusive prefix sum of v[0..n) in place over the whole workgroup (T threads, each
// scanning a run of consecutive elements); wsum holds T / 64 partial sums.
template <int T>
__device__ inline void block_exclusive_scan(int32_t* v, int n, int32_t* wsum) {
  const int per = (n + T - 1) / T;
  const int lo = threadIdx.x * per;
  const int hi = min(n, lo + per);
  int32_t own = 0;
  for (int i = lo; i < hi; ++i) own += v[i];
  // inclusive scan of the per-thread sums inside the wavefront
  const int lane = (int)__lane_id();
  int32_t inc = own;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int32_t u = __shfl_up(inc, off, 64);
    if (lane >= off) inc += u;
  }
  const int wave = threadIdx.x / 64;
  if (lane == 63) wsum[wave] = inc;
  __syncthreads();
  int32_t before = 0;
  for (int w = 0; w < wave; ++w) before += wsum[w];
  int32_t run = before + inc - own;
  for (int i = lo; i < hi; ++i) {
    const int32_t c = v[i];
    v[i] = run;
    run += c;
  }
  __syncthreads();
}

// Levels with at most this many bins use the wavefront-aggregated counters (with more, one
// LDS atomic per lane measured faster: at 16 the aggregation loop cost the config-3 count
// and scatter 25 us and the config-4 count and scatter 127 us).
constexpr int kFewBins = 4;

// Bin of a row of segment (k, l) and its row inside the chunk.
__device__ __forceinline__ void bin_of(const BinPlan& bp, int k, int l, uint32_t row, int32_t& bin,
                                       uint32_t& local) {
  const int s = k * bp.L + l;
  const uint32_t C = (uint32_t)bp.seg_chunk[s];
  if (C & (C - 1u)) {  // whole x-lines of a dense level
    const uint32_t q = row / C;
    bin = bp.seg_bin0[s] + (int32_t)q;
    local = row - q * C;
  } else {
    const int cs = bp.cshift[k];
    bin = bp.seg_bin0[s] + (int32_t)(row >> cs);
    local = row & ((1u << cs) - 1u);
  }
}

int bin_cshift_for_width(int W);
void make_bin_plan(const Grid& g, int d, int F, bool hermite, BinPlan& bp);
int bin_tile_points(const BinPlan& bp, int d, int F, bool hermite);
// Points (= threads) of a Hermite scatter workgroup: its LDS staging holds one order table's
// records for every corner of the tile.
constexpr int hermite_scatter_points(int F) { return F <= 2 ? 512 : F == 4 ? 128 : 64; }
// d = 4: a scatter workgroup has one lane per (point, corner), 16 lanes per point; its LDS
// staging holds one order table's records (at most 6F values) for every lane.
constexpr int hermite4_scatter_points(int F) { return F <= 2 ? 64 : 32; }
size_t hermite_scatter_lds_bytes(const BinPlan& bp, int d, int F);
// LDS of the d-linear scatter workgroup: two per-bin arrays, the per-level staging bases and
// the pair-record staging.
size_t dlinear_scatter_lds_bytes(const BinPlan& bp, int d, int F, int tile);
BinWorkspace bin_workspace_layout(const BinPlan& bp, int64_t chunk_points, int64_t entries_per_point,
                                  int64_t floats_per_point, int tile);
// Stages 2-3 (after the interpolant's count kernel) and stage 5 (after its scatter kernel).
hipError_t run_bin_middle(const BinPlan& bp, const BinWorkspace& w, char* ws, hipStream_t s);
// entries: the chunk's entry count (or a bound on it), which picks the reduce's item order
hipError_t run_bin_reduce(const Grid& g, const BinPlan& bp, const BinWorkspace& w, char* ws,
                          float* grad, int64_t entries, hipStream_t s);

// Interpolant-specific count / scatter launches (d-linear and Hermite kernel files).
// d-linear count / scatter; u_levels: the chunk's upstream level-major ([L][n][F]) or NULL
// to read the rows of g_gamma
hipError_t launch_dlinear_bin(const Grid& g, const BinPlan& bp, const BinWorkspace& w, char* ws,
                              int d, int F, bool scatter, int64_t n, const float* x,
                              const float* g_gamma, const float* u_levels, hipStream_t s);
// d = 4 Hermite count / scatter (upstream read from the row-major arrays)
hipError_t launch_hermite4_bin(const Grid& g, const BinPlan& bp, const BinWorkspace& w, char* ws, int F,
                               int d2_mode, bool scatter, int64_t n, const float* x, const float* g_gamma,
                               const float* g_dgamma, const float* g_d2gamma, hipStream_t s);
// Hermite count / scatter; u_levels: the chunk's upstream already level-major
// ([L][n][M][F], as the forward's staging) or NULL to rearrange g_gamma / g_dgamma / g_d2gamma
hipError_t launch_hermite_bin(const Grid& g, const BinPlan& bp, const BinWorkspace& w, char* ws,
                              int d, int F, int d2_mode, bool scatter, int64_t n, const float* x,
                              const float* g_gamma, const float* g_dgamma, const float* g_d2gamma,
                              const float* u_levels, hipStream_t s);

constexpr int32_t kMaxBins = 16384;
constexpr int64_t kBinChunkPoints = int64_t(1) << 21;  // points per pass of the binned backward
// Entry indices (bin starts, work-item ranges, per-tile slots) are int32: a chunk holds at
// most this many entries, which leaves room for one work item past the last entry.
constexpr int64_t kMaxChunkEntries = (int64_t(1) << 31) - (int64_t(1) << 20);

// Entries per point at most (every corner its own entry; Hermite: one per order table).
inline int64_t bin_entries_per_point(int d, int L, bool hermite) {
  return (int64_t)L * (1 << d) * (hermite ? d + 1 : 1);
}
// Points per pass of the binned backward: kBinChunkPoints, fewer when the chunk's entries
// would not fit the int32 indices (L = 32 Hermite 3D reaches 2^31 entries at 2^21 points);
// a multiple of 1024 so every tile size divides it.
inline int64_t bin_chunk_points(const Grid& g, int d, bool hermite) {
  const int64_t cap = (kMaxChunkEntries / bin_entries_per_point(d, g.L, hermite)) & ~int64_t(1023);
  return cap < kBinChunkPoints ? cap : kBinChunkPoints;
}

// Whether this configuration's bins and staging fit the LDS budgets of the binned path.
bool binned_fits(const Grid& g, int d, int F, bool hermite);

// Whole binned backward over n points, in chunks that fit the workspace.
size_t binned_backward_workspace_bytes(const Grid& g, int d, int F, bool hermite, int64_t n);
// u_levels (else NULL): upstream already level-major for all n points (Hermite [L][n][M][F],
// d-linear [L][n][F]; n at most one internal chunk); then the row-major upstream pointers are
// ignored.
// max_chunk > 0 lowers the points per pass below bin_chunk_points (a workspace sized for
// max_chunk points then suffices).
// counted: the chunk's counts are already in the workspace (left by the counting d-linear
// forward on the same x; n at most one chunk), so the count pass is skipped.
hipError_t run_binned_backward(const Grid& g, int d, int F, bool hermite, int d2_mode, int64_t n,
                               const float* x, const float* g_gamma, const float* g_dgamma,
                               const float* g_d2gamma, const float* u_levels, float* grad, void* workspace,
                               hipStream_t s, int64_t max_chunk = 0, bool counted = false);
// Workspace layout of one chunk of chunk_points points.
BinWorkspace bin_workspace_for(const Grid& g, const BinPlan& bp, int d, int F, bool hermite, int64_t chunk_points);

// Counting d-linear forward: the workspace forward (level-major staging in scratch, then rows
// in gamma) that also writes the binned backward's per-tile counts of these n points (at most
// one chunk) into the backward workspace bws, so that run_binned_backward(..., counted) on
// the same x skips its count pass.  dlinear_forward_counts: whether this configuration's
// forward passes can count (each pass's bins fit the forward's LDS counters).
bool dlinear_forward_counts(const Grid& g, int d, int F);
hipError_t launch_dlinear_forward_counting(const Grid& g, int d, int F, int64_t n, const float* x,
                                           const float* params, float* gamma, float* scratch, void* bws,
                                           hipStream_t s);

}  // namespace hg
