// Binned backward: the scatter-add dL/dtheta += sum over (point, level, corner) without
// global atomics on the hot part, gfx950.
//
// Why: fp32 global atomics on this part run at ~21 G requests/s whatever the footprint, so
// a backward issuing one request per corner row is bounded far below HBM bandwidth.  Here
// the contributions are instead routed to the workgroup that owns their rows:
//   1. count   per point tile, histogram of contributions over bins (table, level, chunk
//              of rows small enough to accumulate in LDS)
//   2. scan    per bin, exclusive prefix over point tiles (and the bin totals); the counts
//              are stored tile-major, counts[tile][bin], so every tile writes and reads
//              its own row contiguously
//   3. plan    exclusive scan over bins, per-segment bases, work items (bin, entry range)
//   4. scatter recompute the contributions and write compact entries (local row, values)
//              to their bin's range
//   5. reduce  one workgroup per work item accumulates its entries into an LDS copy of the
//              chunk and adds it to the gradient (plain read-modify-write when the bin is a
//              single item, atomics only when a large bin was split across items)
// Steps 1 and 4 are interpolant-specific (d-linear, Hermite kernel files); 2, 3 and 5 live
// here.  Within one call the chunks of points run back to back on the stream.
#include "binned_backward.h"
#include "vec_io.h"

namespace hg {

namespace {

// counts[tile][bin] -> exclusive prefix over tiles in place; totals[bin] = sum.  The tiles
// are cut into kScanSegs consecutive segments, one per wavefront of a (64-bin group,
// segment group) workgroup; a lane owns one bin, so every row access is one coalesced
// 256-byte run.  First pass: segment sums; second pass: each wavefront adds the sums of the
// segments before its own and rewrites its rows as running prefixes.
constexpr int kScanWavesPerBlock = 4;
constexpr int kScanSegs = 16 * kScanWavesPerBlock;

__device__ __forceinline__ void scan_segment(int nblk, int& r0, int& r1, int& seg) {
  const int rows = (nblk + kScanSegs - 1) / kScanSegs;
  seg = blockIdx.y * kScanWavesPerBlock + (int)(threadIdx.x >> 6);
  r0 = seg * rows;
  r1 = min(nblk, r0 + rows);
}

__global__ __launch_bounds__(64 * kScanWavesPerBlock) void bin_scan_sums_kernel(const int32_t* __restrict__ counts,
                                                                               int32_t nblk, int32_t nbins,
                                                                               int32_t* __restrict__ seg_sums) {
  const int bin = blockIdx.x * 64 + (int)(threadIdx.x & 63);
  if (bin >= nbins) return;
  int r0, r1, seg;
  scan_segment(nblk, r0, r1, seg);
  int32_t s = 0;
#pragma unroll 8
  for (int r = r0; r < r1; ++r) s += counts[(int64_t)r * nbins + bin];
  seg_sums[(int64_t)seg * nbins + bin] = s;
}

__global__ __launch_bounds__(64 * kScanWavesPerBlock) void bin_scan_apply_kernel(int32_t* __restrict__ counts,
                                                                                int32_t nblk, int32_t nbins,
                                                                                const int32_t* __restrict__ seg_sums,
                                                                                int32_t* __restrict__ totals) {
  const int bin = blockIdx.x * 64 + (int)(threadIdx.x & 63);
  if (bin >= nbins) return;
  int r0, r1, seg;
  scan_segment(nblk, r0, r1, seg);
  int32_t run = 0;
  {
    int32_t part[8] = {0, 0, 0, 0, 0, 0, 0, 0};  // eight loads in flight
    int j = 0;
    for (; j + 8 <= seg; j += 8)
#pragma unroll
      for (int u = 0; u < 8; ++u) part[u] += seg_sums[(int64_t)(j + u) * nbins + bin];
    for (; j < seg; ++j) part[0] += seg_sums[(int64_t)j * nbins + bin];
#pragma unroll
    for (int u = 0; u < 8; ++u) run += part[u];
  }
  if (seg == kScanSegs - 1) totals[bin] = run + seg_sums[(int64_t)seg * nbins + bin];
  // eight rows' loads in flight before their stores (a store between two loads of the same
  // array would otherwise hold every load back until the one before it returns)
  int r = r0;
  for (; r + 8 <= r1; r += 8) {
    int32_t c[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) c[u] = counts[(int64_t)(r + u) * nbins + bin];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      counts[(int64_t)(r + u) * nbins + bin] = run;
      run += c[u];
    }
  }
  for (; r < r1; ++r) {
    const int32_t c = counts[(int64_t)r * nbins + bin];
    counts[(int64_t)r * nbins + bin] = run;
    run += c;
  }
}

__global__ __launch_bounds__(1024) void bin_plan_kernel(const BinPlan bp, const int32_t* __restrict__ totals,
                                                        int32_t* __restrict__ bin_start,
                                                        WorkItem* __restrict__ items,
                                                        BinState* __restrict__ st, int32_t emax) {
  // One workgroup: bin_start = exclusive scan of totals; work items; segment bases.  The
  // totals are staged in LDS by coalesced loads (four in flight per thread), and the first
  // entry of every segment is kept in LDS for the segment bases.
  __shared__ int32_t part[1024];
  __shared__ int32_t ipart[1024];
  __shared__ int32_t seg0[kMaxSeg + 1];
  __shared__ int32_t seg_first[kMaxSeg];
  __shared__ int32_t tot_sh[kMaxBins];
  const int t = threadIdx.x;
  for (int i = t; i <= bp.nseg; i += 1024) seg0[i] = bp.seg_bin0[i];
  const int nb = bp.nbins;
  for (int i0 = t; i0 < nb; i0 += 4 * 1024) {
    int32_t v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = i0 + u * 1024 < nb ? totals[i0 + u * 1024] : 0;
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (i0 + u * 1024 < nb) tot_sh[i0 + u * 1024] = v[u];
  }
  __syncthreads();
  const int per = (nb + 1023) / 1024;
  const int b0 = t * per;
  int32_t s = 0, si = 0;
  for (int i = 0; i < per; ++i) {
    const int b = b0 + i;
    if (b < nb) {
      const int32_t tot = tot_sh[b];
      s += tot;
      si += (tot + emax - 1) / emax;
    }
  }
  part[t] = s;
  ipart[t] = si;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const int32_t v = t >= off ? part[t - off] : 0;
    const int32_t vi = t >= off ? ipart[t - off] : 0;
    __syncthreads();
    part[t] += v;
    ipart[t] += vi;
    __syncthreads();
  }
  int32_t run = part[t] - s;
  int32_t irun = ipart[t] - si;
  int sg = 0;
  for (int i = 0; i < per; ++i) {
    const int b = b0 + i;
    if (b < nb) {
      const int32_t tot = tot_sh[b];
      bin_start[b] = run;
      while (sg + 1 < bp.nseg && seg0[sg + 1] <= b) ++sg;  // segment owning bin b
      if (seg0[sg] == b) seg_first[sg] = run;  // every segment has at least one bin
      const int32_t nit = (tot + emax - 1) / emax;
      for (int j = 0; j < nit; ++j) {
        WorkItem w;
        w.bin = b;
        w.seg = sg;
        w.begin = run + j * emax;
        w.end = min(run + tot, run + (j + 1) * emax);
        w.split = nit > 1 ? 1 : 0;
        items[irun + j] = w;
      }
      run += tot;
      irun += nit;
    }
  }
  if (t == 1023) {
    bin_start[nb] = part[1023];
    st->n_items = ipart[1023];
    st->next_item = 0;
  }
  __syncthreads();
  if (t == 0) {
    int64_t vb = 0;
    for (int g = 0; g < bp.nseg; ++g) {
      const int32_t e0 = seg_first[g];
      const int32_t e1 = g + 1 < bp.nseg ? seg_first[g + 1] : part[1023];
      st->seg_ebase[g] = e0;
      st->seg_vbase[g] = vb;
      vb += (int64_t)(e1 - e0) * (bp.records ? 2 + bp.width[0] : hermite_rec_width(bp.width[g / bp.L]));
      vb = (vb + kSegAlignFloats - 1) / kSegAlignFloats * kSegAlignFloats;
    }
  }
}

// Accumulate entries [begin, end) of one segment (a chunk-local row stored as the bits of
// the first float, then the row's W values) into the LDS chunk: each thread keeps U entries
// (about 32 value registers) in flight before its LDS atomics.  acc holds the chunk
// component-major (acc[j * plane + row]) so that the W components of one row fall in
// different LDS banks' rotation and a wavefront's random rows spread over all banks.
template <int W>
__device__ __forceinline__ void accumulate_entries(double* __restrict__ acc, int plane,
                                                   const float* __restrict__ vseg, int32_t ebase,
                                                   int32_t begin, int32_t end) {
  constexpr int R = hermite_rec_width(W);
  constexpr int U = W >= 32 ? 1 : 32 / W > 8 ? 8 : 32 / W;
  const int T = blockDim.x;
  for (int32_t e0 = begin + (int32_t)threadIdx.x; e0 < end; e0 += T * U) {
    int r[U];
    float rec[U][R];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int32_t e = e0 + u * T;
      if (e < end) {
        load_vec_nt<R>(vseg + (int64_t)(e - ebase) * R, rec[u]);
        r[u] = (int)__float_as_uint(rec[u][0]);
      } else {
        r[u] = -1;
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (r[u] >= 0)
#pragma unroll
        for (int j = 0; j < W; ++j) atomicAdd(&acc[j * plane + r[u]], (double)rec[u][1 + j]);
  }
}

// d-linear records {rows, t, aG[F]}: the lower row gets (1 - t) aG, the upper (if any) t aG.
template <int F>
__device__ __forceinline__ void accumulate_records(double* __restrict__ acc, int plane,
                                                   const float* __restrict__ vseg, int32_t ebase,
                                                   int32_t begin, int32_t end) {
  constexpr int R = 2 + F;
  constexpr int U = 32 / R > 8 ? 8 : (32 / R < 1 ? 1 : 32 / R);
  const int T = blockDim.x;
  for (int32_t e0 = begin + (int32_t)threadIdx.x; e0 < end; e0 += T * U) {
    float rec[U][R];
    bool on[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int32_t e = e0 + u * T;
      on[u] = e < end;
      if (on[u]) load_vec_nt<R>(vseg + (int64_t)(e - ebase) * R, rec[u]);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (!on[u]) continue;
      const uint32_t rows = __float_as_uint(rec[u][0]);
      const int lo = (int)(rows & 0xFFFFu), hi = (int)(rows >> 16);
      const double t = rec[u][1];
#pragma unroll
      for (int f = 0; f < F; ++f) {
        const double a = rec[u][2 + f];
        atomicAdd(&acc[f * plane + lo], (1.0 - t) * a);
        if (hi != 0xFFFF) atomicAdd(&acc[f * plane + hi], t * a);
      }
    }
  }
}

__global__ __launch_bounds__(kReduceThreads) void bin_reduce_kernel(const Grid g, const BinPlan bp,
                                                                    BinState* __restrict__ st,
                                                                    const WorkItem* __restrict__ items,
                                                                    const float* __restrict__ vals,
                                                                    float* __restrict__ grad) {
  // fp64 accumulator: LDS fp64 atomics run several times faster than fp32 ones on gfx950
  // and the chunk sum is exact to far below the fp32 result precision.
  __shared__ double acc[kBinLdsValues];
  __shared__ int item_sh;
  const int n_items = st->n_items;
  for (;;) {
    if (threadIdx.x == 0) item_sh = atomicAdd(&st->next_item, 1);
    __syncthreads();
    const int it = item_sh;
    __syncthreads();
    if (it >= n_items) break;
    const WorkItem w = items[it];
    const int sg = __builtin_amdgcn_readfirstlane(w.seg);
    const int k = sg / bp.L, l = sg % bp.L;
    const int W = bp.width[k];
    const int64_t C = bp.seg_chunk[sg];
    const int64_t chunk = __builtin_amdgcn_readfirstlane(w.bin) - bp.seg_bin0[sg];
    const int64_t row0 = chunk * C;
    const int64_t rem = seg_rows(g, bp.d, k, l) - row0;
    const int64_t nrows = rem < C ? rem : C;
    const int nfl = (int)(nrows * W);
    for (int i = threadIdx.x; i < nfl; i += kReduceThreads) acc[i] = 0.0;
    __syncthreads();
    // values of entry e of segment sg start at vseg + (e - ebase) * W
    const float* vseg = vals + st->seg_vbase[sg];
    const int32_t eb = st->seg_ebase[sg];
    const int plane = (int)nrows;
    if (bp.records) {
      switch (W) {
        case 1: accumulate_records<1>(acc, plane, vseg, eb, w.begin, w.end); break;
        case 2: accumulate_records<2>(acc, plane, vseg, eb, w.begin, w.end); break;
        case 4: accumulate_records<4>(acc, plane, vseg, eb, w.begin, w.end); break;
        default: accumulate_records<8>(acc, plane, vseg, eb, w.begin, w.end); break;
      }
    } else switch (W) {
      case 1: accumulate_entries<1>(acc, plane, vseg, eb, w.begin, w.end); break;
      case 2: accumulate_entries<2>(acc, plane, vseg, eb, w.begin, w.end); break;
      case 3: accumulate_entries<3>(acc, plane, vseg, eb, w.begin, w.end); break;
      case 4: accumulate_entries<4>(acc, plane, vseg, eb, w.begin, w.end); break;
      case 6: accumulate_entries<6>(acc, plane, vseg, eb, w.begin, w.end); break;
      case 8: accumulate_entries<8>(acc, plane, vseg, eb, w.begin, w.end); break;
      case 12: accumulate_entries<12>(acc, plane, vseg, eb, w.begin, w.end); break;
      case 16: accumulate_entries<16>(acc, plane, vseg, eb, w.begin, w.end); break;
      default: accumulate_entries<24>(acc, plane, vseg, eb, w.begin, w.end); break;
    }
    __syncthreads();
    // flush: element i of the chunk is row i / W, component i % W
    float* dst = grad + g.off[k][l] + row0 * W;
    if (w.split) {
      for (int i = threadIdx.x; i < nfl; i += kReduceThreads) {
        const float a = (float)acc[(i % W) * plane + i / W];
        if (a != 0.0f) atomic_add_f32(dst + i, a);
      }
    } else {
      for (int i = threadIdx.x; i < nfl; i += kReduceThreads) dst[i] += (float)acc[(i % W) * plane + i / W];
    }
    __syncthreads();
  }
}

// Workspace bound: every corner its own entry (single records on d-linear segments).
int64_t entries_per_point(int d, int L, bool hermite) {
  return (int64_t)L * (1 << d) * (hermite ? d + 1 : 1);
}

int64_t floats_per_point(const BinPlan& bp, int d) {
  if (bp.records) return (int64_t)bp.L * (1 << d) * (2 + bp.width[0]);
  int64_t w = 0;
  for (int k = 0; k < bp.ntab; ++k) w += hermite_rec_width(bp.width[k]);
  return (int64_t)bp.L * (1 << d) * w;
}

}  // namespace

int bin_cshift_for_width(int W) {
  int c = 0;
  while (((int64_t)2 << c) * W <= kBinLdsValues) ++c;
  return c;  // largest c with (1 << c) * W <= kBinLdsValues
}

void make_bin_plan(const Grid& g, int d, int F, bool hermite, BinPlan& bp) {
  bp.d = d;
  bp.L = g.L;
  bp.ntab = hermite ? d + 1 : 1;
  bp.nseg = bp.ntab * g.L;
  bp.records = hermite ? 0 : 1;
  bp.pair_mask = 0;
  for (int k = 0; k < kMaxTables; ++k) { bp.width[k] = 0; bp.cshift[k] = 0; }
  int32_t bin = 0;
  bp.max_seg_bins = 0;
  for (int k = 0; k < bp.ntab; ++k) {
    const int W = hermite ? (k == 0 || k == d ? F : (d == 3 ? 3 * F : 2 * F)) : F;
    bp.width[k] = W;
    bp.cshift[k] = bin_cshift_for_width(W);
    const int64_t C = (int64_t)1 << bp.cshift[k];
    for (int l = 0; l < g.L; ++l) {
      const int s = k * g.L + l;
      const int64_t rows = seg_rows(g, d, k, l);
      int64_t chunk = C;
      if (!hermite) {
        const bool dense = (g.dense[k] >> l) & 1u;
        const int64_t line = (int64_t)g.N[l] + 1;
        if (dense && line <= C) {
          chunk = C / line * line;  // whole x-lines: x-neighbours share a chunk
          bp.pair_mask |= 1u << l;
        } else if (!dense && g.Tmask[k] != 0 && 2 * (int64_t)g.N[l] <= C) {
          // XOR-adjacent rows differ below bit log2(2 N) <= cshift: same chunk
          bp.pair_mask |= 1u << l;
        }
      }
      bp.seg_chunk[s] = (int32_t)chunk;
      bp.seg_bin0[s] = bin;
      const int32_t nb = (int32_t)((rows + chunk - 1) / chunk);
      if (nb > bp.max_seg_bins) bp.max_seg_bins = nb;
      bin += nb;
    }
  }
  bp.seg_bin0[bp.nseg] = bin;
  bp.nbins = bin;
  bp.max_level_bins = 0;
  for (int l = 0; l < g.L; ++l) {
    int32_t lb = 0;
    for (int k = 0; k < bp.ntab; ++k) lb += bp.seg_bin0[k * g.L + l + 1] - bp.seg_bin0[k * g.L + l];
    if (lb > bp.max_level_bins) bp.max_level_bins = lb;
  }
  bp.fine_shift = -1;
  if (hermite) {
    bool uniform = true;
    int fine = bp.cshift[0];
    for (int k = 1; k < bp.ntab; ++k) {
      uniform = uniform && g.T[k] == g.T[0];
      if (bp.cshift[k] < fine) fine = bp.cshift[k];
    }
    if (uniform) {
      bp.fine_shift = fine;
      int32_t fb = 0;
      for (int l = 0; l < g.L; ++l) {
        bp.fine_bin0[l] = fb;
        fb += (int32_t)((seg_rows(g, d, 0, l) + ((int64_t)1 << fine) - 1) >> fine);
      }
      bp.fine_bin0[g.L] = fb;
    }
  }
}

int bin_tile_points(const BinPlan& bp, int d, int F, bool hermite) {
  // one point per scatter lane
  if (hermite) return hermite_scatter_points(F);
  return dlinear_scatter_lds_bytes(bp, d, F, kScatterTileLarge) <= kMaxScatterLds ? kScatterTileLarge
                                                                                 : kScatterTileSmall;
}

size_t hermite_scatter_lds_bytes(const BinPlan& bp, int d, int F) {
  const int P = hermite_scatter_points(F);
  const int smax = hermite_stage_width((d == 3 ? 3 : 2) * F);  // widest order table's staged record
  return sizeof(int32_t) * (2 * (size_t)bp.max_level_bins + P / 64 + 3) + (size_t)P * (1 << d) * sizeof(float) * smax;
}

size_t dlinear_scatter_lds_bytes(const BinPlan& bp, int d, int F, int tile) {
  return sizeof(int32_t) * (2 * (size_t)bp.nbins + tile / 64 + kMaxLevels + 3) +
         (size_t)tile * (1 << (d - 1)) * (sizeof(float) * (2 + F) + sizeof(int32_t));
}

BinWorkspace bin_workspace_layout(const BinPlan& bp, int64_t chunk_points, int64_t epp, int64_t fpp, int tile) {
  BinWorkspace w;
  auto al = [](size_t b) { return (b + 255) & ~size_t(255); };
  w.tile = tile;
  w.nblk = (int32_t)((chunk_points + tile - 1) / tile);
  const int64_t entries = chunk_points * epp;
  w.item_entries = bin_item_entries(entries);
  // bins split into items of item_entries: at most entries / item_entries <= max(512,
  // entries / kBinItemEntries) extra items, a bound that only grows with the chunk
  w.max_items = bp.nbins + 514 + entries / kBinItemEntries;
  size_t off = 0;
  w.counts = off; off += al(sizeof(int32_t) * (size_t)bp.nbins * w.nblk);
  w.totals = off; off += al(sizeof(int32_t) * (size_t)bp.nbins);
  w.seg_sums = off; off += al(sizeof(int32_t) * (size_t)bp.nbins * kScanSegs);
  w.state = off; off += al(sizeof(BinState));
  w.bin_start = off; off += al(sizeof(int32_t) * (size_t)(bp.nbins + 1));
  w.items = off; off += al(sizeof(WorkItem) * (size_t)w.max_items);
  w.vals = off; off += al(sizeof(float) * (size_t)(chunk_points * fpp + bp.nseg * kSegAlignFloats));
  // Hermite: the chunk's upstream rearranged level-major, [L][point][1 + 2d][F] at most
  w.ups = off; off += al(bp.records ? 0 : sizeof(float) * (size_t)chunk_points * bp.L * (1 + 2 * bp.d) * bp.width[0]);
  w.total = off;
  return w;
}

hipError_t run_bin_middle(const BinPlan& bp, const BinWorkspace& w, char* ws, hipStream_t s) {
  int32_t* counts = reinterpret_cast<int32_t*>(ws + w.counts);
  int32_t* totals = reinterpret_cast<int32_t*>(ws + w.totals);
  int32_t* seg_sums = reinterpret_cast<int32_t*>(ws + w.seg_sums);
  const dim3 sgrid((unsigned)((bp.nbins + 63) / 64), kScanSegs / kScanWavesPerBlock);
  hipLaunchKernelGGL(bin_scan_sums_kernel, sgrid, dim3(64 * kScanWavesPerBlock), 0, s, counts, w.nblk, bp.nbins,
                     seg_sums);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(bin_scan_apply_kernel, sgrid, dim3(64 * kScanWavesPerBlock), 0, s, counts, w.nblk, bp.nbins,
                     seg_sums, totals);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(bin_plan_kernel, dim3(1), dim3(1024), 0, s, bp, totals,
                     reinterpret_cast<int32_t*>(ws + w.bin_start), reinterpret_cast<WorkItem*>(ws + w.items),
                     reinterpret_cast<BinState*>(ws + w.state), w.item_entries);
  return hipGetLastError();
}

hipError_t run_bin_reduce(const Grid& g, const BinPlan& bp, const BinWorkspace& w, char* ws, float* grad,
                          hipStream_t s) {
  hipLaunchKernelGGL(bin_reduce_kernel, dim3(kBinReduceBlocks), dim3(kReduceThreads), 0, s, g, bp,
                     reinterpret_cast<BinState*>(ws + w.state), reinterpret_cast<const WorkItem*>(ws + w.items),
                     reinterpret_cast<const float*>(ws + w.vals),
                     grad);
  return hipGetLastError();
}

bool binned_fits(const Grid& g, int d, int F, bool hermite) {
  BinPlan bp;
  make_bin_plan(g, d, F, hermite, bp);
  const int32_t count_bins = bp.fine_shift >= 0 ? bp.fine_bin0[g.L] : bp.nbins;
  if (bp.nbins > kMaxBins || count_bins > kMaxBins) return false;  // LDS counters of the count pass
  if (hermite) return hermite_scatter_lds_bytes(bp, d, F) <= kMaxScatterLds;
  const int tile = bin_tile_points(bp, d, F, hermite);
  return dlinear_scatter_lds_bytes(bp, d, F, tile) <= kMaxScatterLds;
}

size_t binned_backward_workspace_bytes(const Grid& g, int d, int F, bool hermite, int64_t n) {
  BinPlan bp;
  make_bin_plan(g, d, F, hermite, bp);
  const int64_t c = n < kBinChunkPoints ? n : kBinChunkPoints;
  return bin_workspace_layout(bp, c, entries_per_point(d, g.L, hermite), floats_per_point(bp, d),
                              bin_tile_points(bp, d, F, hermite)).total;
}

hipError_t run_binned_backward(const Grid& g, int d, int F, bool hermite, int d2_mode, int64_t n,
                               const float* x, const float* g_gamma, const float* g_dgamma,
                               const float* g_d2gamma, const float* u_levels, float* grad, void* workspace,
                               hipStream_t s) {
  BinPlan bp;
  make_bin_plan(g, d, F, hermite, bp);
  if (u_levels && n > kBinChunkPoints) return hipErrorInvalidValue;  // one chunk only
  char* ws = static_cast<char*>(workspace);
  const int64_t LF = (int64_t)g.Lrow * F;  // upstream row stride
  for (int64_t p0 = 0; p0 < n; p0 += kBinChunkPoints) {
    const int64_t c = (n - p0) < kBinChunkPoints ? (n - p0) : kBinChunkPoints;
    const BinWorkspace w = bin_workspace_layout(bp, c, entries_per_point(d, g.L, hermite), floats_per_point(bp, d),
                                                bin_tile_points(bp, d, F, hermite));
    const float* xc = x + p0 * d;
    const float* gg = g_gamma ? g_gamma + p0 * LF : nullptr;
    const float* gd = g_dgamma ? g_dgamma + p0 * d * LF : nullptr;
    const float* g2 = g_d2gamma ? g_d2gamma + p0 * (d2_mode == HASHENC_D2_DIAG ? d : 1) * LF : nullptr;
    for (int pass = 0; pass < 2; ++pass) {
      hipError_t e = hermite ? launch_hermite_bin(g, bp, w, ws, d, F, d2_mode, pass == 1, c, xc, gg, gd, g2,
                                                  u_levels, s)
                             : launch_dlinear_bin(g, bp, w, ws, d, F, pass == 1, c, xc, gg, u_levels, s);
      if (e != hipSuccess) return e;
      if (pass == 0) {
        e = run_bin_middle(bp, w, ws, s);
        if (e != hipSuccess) return e;
      }
    }
    hipError_t e = run_bin_reduce(g, bp, w, ws, grad, s);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace hg
