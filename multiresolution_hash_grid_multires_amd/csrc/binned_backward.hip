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
#include <algorithm>

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

// The same scan in one pass when there are at most kScanOneRows tiles: a 1024-lane workgroup
// per 64 bins, its 16 wavefronts taking consecutive runs of at most 16 tiles each, held in
// registers between the segment sums (exchanged through LDS) and the rewrite.  Small batches
// have few tiles, and there the second launch and its round trips are a visible share.
constexpr int kScanOneWaves = 16;
constexpr int kScanOneRowsPerWave = 16;
constexpr int kScanOneRows = kScanOneWaves * kScanOneRowsPerWave;

__global__ __launch_bounds__(64 * kScanOneWaves) void bin_scan_one_pass_kernel(int32_t* __restrict__ counts,
                                                                             int32_t nblk, int32_t nbins,
                                                                             int32_t* __restrict__ totals) {
  __shared__ int32_t wsum[kScanOneWaves][64];
  const int lane = (int)(threadIdx.x & 63), wave = (int)(threadIdx.x >> 6);
  const int bin = blockIdx.x * 64 + lane;
  const int per = (nblk + kScanOneWaves - 1) / kScanOneWaves;  // <= kScanOneRowsPerWave
  const int r0 = min(nblk, wave * per), r1 = min(nblk, r0 + per);
  const bool on = bin < nbins;
  int32_t c[kScanOneRowsPerWave];
  int32_t s = 0;
#pragma unroll
  for (int u = 0; u < kScanOneRowsPerWave; ++u) {
    c[u] = (on && r0 + u < r1) ? counts[(int64_t)(r0 + u) * nbins + bin] : 0;
    s += c[u];
  }
  wsum[wave][lane] = s;
  __syncthreads();
  int32_t run = 0;
  for (int w = 0; w < wave; ++w) run += wsum[w][lane];
  if (on && wave == kScanOneWaves - 1) totals[bin] = run + s;
#pragma unroll
  for (int u = 0; u < kScanOneRowsPerWave; ++u) {
    if (on && r0 + u < r1) counts[(int64_t)(r0 + u) * nbins + bin] = run;
    run += c[u];
  }
}

__global__ __launch_bounds__(1024) void bin_plan_kernel(const BinPlan bp, const int32_t* __restrict__ totals,
                                                        int32_t* __restrict__ bin_start,
                                                        WorkItem* __restrict__ items,
                                                        BinState* __restrict__ st, int32_t emax) {
  // One workgroup: bin_start = exclusive scan of totals; work items; segment bases.  The
  // totals are staged in LDS by coalesced loads (four in flight per thread), and the first
  // entry of every segment is kept in LDS for the segment bases.
  __shared__ int32_t part[16];   // per-wavefront totals
  __shared__ int32_t ipart[16];
  __shared__ int32_t seg0[kMaxSeg + 1];
  __shared__ int32_t seg_first[kMaxSeg + 1];
  __shared__ int32_t tot_sh[kMaxBins];
  const int t = threadIdx.x;
  if (t < kMaxSeg) st->vmax_bits[t] = 0u;  // raised by the scatter that follows
  for (int i = t; i <= bp.nseg; i += 1024) seg0[i] = bp.seg_bin0[i];
  const int nb = bp.nbins;
  {
    constexpr int U = kMaxBins / 1024;  // every load in flight before the first LDS store
    int32_t v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = t + u * 1024 < nb ? totals[t + u * 1024] : 0;
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (t + u * 1024 < nb) tot_sh[t + u * 1024] = v[u];
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
  // inclusive scans of (s, si) over the workgroup: within each wavefront by shuffles, then
  // the 16 wavefront totals (two barriers in all, where a scan over LDS took twenty)
  int32_t inc = s, inci = si;
  const int lane = t & 63, wv = t >> 6;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int32_t a = __shfl_up(inc, off, 64), ai = __shfl_up(inci, off, 64);
    if (lane >= off) {
      inc += a;
      inci += ai;
    }
  }
  if (lane == 63) {
    part[wv] = inc;
    ipart[wv] = inci;
  }
  __syncthreads();
  int32_t before = 0, beforei = 0;
  for (int w = 0; w < wv; ++w) {
    before += part[w];
    beforei += ipart[w];
  }
  int32_t run = before + inc - s;
  int32_t irun = beforei + inci - si;
  // segment owning bin b0 (the last with seg0 <= b0; seg0[0] = 0) by bisection, then walked
  // forward over this thread's few bins
  int sg = 0;
  for (int hi = bp.nseg - 1; sg < hi;) {
    const int mid = (sg + hi + 1) >> 1;
    if (seg0[mid] <= b0) sg = mid;
    else hi = mid - 1;
  }
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
    bin_start[nb] = run;
    st->n_items = irun;
    st->next_item = 0;
    seg_first[bp.nseg] = run;  // the entry count closes the last segment
  }
  __syncthreads();
  // segment bases: the value floats of each segment rounded up to whole 128-byte lines,
  // prefix-summed by the first wavefront (a few consecutive segments per lane, then a scan)
  if (t < 64) {
    constexpr int SPL = (kMaxSeg + 63) / 64;
    int64_t sz[SPL];
    int64_t own = 0;
#pragma unroll
    for (int j = 0; j < SPL; ++j) {
      const int g = t * SPL + j;
      sz[j] = 0;
      if (g < bp.nseg) {
        sz[j] = (int64_t)(seg_first[g + 1] - seg_first[g]) *
                (bp.records ? 2 + bp.width[0] : hermite_rec_width(bp.width[g / bp.L]));
        sz[j] = (sz[j] + kSegAlignFloats - 1) / kSegAlignFloats * kSegAlignFloats;
      }
      own += sz[j];
    }
    int64_t incv = own;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int64_t a = __shfl_up(incv, off, 64);
      if (lane >= off) incv += a;
    }
    int64_t vb = incv - own;
#pragma unroll
    for (int j = 0; j < SPL; ++j) {
      const int g = t * SPL + j;
      if (g < bp.nseg) {
        st->seg_ebase[g] = seg_first[g];
        st->seg_vbase[g] = vb;
      }
      vb += sz[j];
    }
  }
}

// The LDS accumulator holds 64-bit words: fp64 sums, or (the usual case) fixed-point sums.
// Fixed point: every value v a work item adds is rounded once to the integer nearest v * 2^S,
// where 2^S puts the bound on |v| of the item's segment (from BinState::vmax_bits) at 2^43,
// and the integers are summed exactly with 64-bit LDS integer adds -- which run about 1.8x
// faster than fp64 LDS adds on gfx950 (random rows of a 128 KB accumulator: 2.6 against
// 1.45 T lane-operations/s) and make the sum independent of the order of the records.  A work
// item holds at most 2^18 entries and each entry adds at most one value to a given (row,
// component), so every sum stays below 2^61 in magnitude; the rounding error of each value is
// at most 2^-44 of the bound.  The bound is per segment (order table and level), and is the
// largest value actually written where the weights do not bound it tightly (Hermite: the
// values of levels and tables differ by many orders of magnitude -- the second derivatives
// carry N_l^2, each derivative order of a table 1/N_l -- and a record's basis factors can be
// arbitrarily small); d-linear: max |upstream|, which the largest of a point's 2^d corner
// weights (at least 2^-d) brings within 2^d of its values.  An item whose bound is not
// finite (inf or NaN upstream) is summed in fp64 instead.
struct FixedScale {
  double s;    // 2^S
  double inv;  // 2^-S
};

// round(v * 2^S) for |v * 2^S| < 2^51: adding 1.5 * 2^52 leaves the rounded integer in the
// low mantissa bits of a double whose exponent is fixed (one fused multiply-add, one rounding).
__device__ __forceinline__ int64_t to_fixed(double v, double s) {
  constexpr double kMagic = 6755399441055744.0;  // 1.5 * 2^52
  return __double_as_longlong(__builtin_fma(v, s, kMagic)) - __double_as_longlong(kMagic);
}

template <bool FX>
__device__ __forceinline__ void acc_add(uint64_t* acc, int i, double v, const FixedScale& fs) {
  if constexpr (FX) atomicAdd((unsigned long long*)&acc[i], (unsigned long long)to_fixed(v, fs.s));
  else atomicAdd(reinterpret_cast<double*>(acc) + i, v);
}

template <bool FX>
__device__ __forceinline__ float acc_value(const uint64_t* acc, int i, const FixedScale& fs) {
  if constexpr (FX) return (float)((double)(int64_t)acc[i] * fs.inv);
  else return (float)__longlong_as_double((long long)acc[i]);
}

// Accumulate entries [begin, end) of one segment (a chunk-local row stored as the bits of
// the first float, then the row's W values) into the LDS chunk: each thread keeps U entries
// (about 32 value registers) in flight before its LDS adds.  acc holds the chunk
// component-major (acc[j * plane + row]) so that the W components of one row fall in
// different LDS banks' rotation and a wavefront's random rows spread over all banks.  Only
// entries inside the item are loaded: the small items of small batches would otherwise
// issue many loads per useful one.
template <int W, bool FX>
__device__ __forceinline__ void accumulate_entries(uint64_t* __restrict__ acc, int plane,
                                                   const float* __restrict__ vseg, int32_t ebase,
                                                   int32_t begin, int32_t end, const FixedScale& fs) {
  constexpr int R = hermite_rec_width(W);
  // the fp64 fallback (non-finite bounds only) keeps one entry in flight: its registers would
  // otherwise set the whole kernel's allocation
  constexpr int U = !FX ? 1 : W >= 32 ? 1 : 32 / W > 8 ? 8 : 32 / W;
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
        for (int j = 0; j < W; ++j) acc_add<FX>(acc, j * plane + r[u], (double)rec[u][1 + j], fs);
  }
}

// d-linear records {rows, t, aG[F]}: the lower row gets (1 - t) aG, the upper (if any) t aG.
template <int F, bool FX>
__device__ __forceinline__ void accumulate_records(uint64_t* __restrict__ acc, int plane,
                                                   const float* __restrict__ vseg, int32_t ebase,
                                                   int32_t begin, int32_t end, const FixedScale& fs) {
  constexpr int R = 2 + F;
  constexpr int U = !FX ? 1 : 32 / R > 8 ? 8 : (32 / R < 1 ? 1 : 32 / R);
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
        acc_add<FX>(acc, f * plane + lo, (1.0 - t) * a, fs);
        if (hi != 0xFFFF) acc_add<FX>(acc, f * plane + hi, t * a, fs);
      }
    }
  }
}

constexpr int kFlushBatch = 16;  // gradient values per thread in flight in the reduce's flush (at most)

// Flush of one chunk of the LDS accumulator into the gradient: element i of the chunk is row
// i / W, component i % W (component-major planes of `plane` values).  Each value is read and
// set back to zero, so the accumulator is all zeros again when the next item starts.  Rows no
// entry touched keep their gradient: no read-modify-write for them (a bin of a small batch
// touches few of its rows).  FB gradient loads per thread are in flight before their stores:
// one read-modify-write round trip per batch rather than one per value.  A bin split over
// several items (split) adds its part with atomics instead.  i / W is taken as the truncation
// of (i + 1/2) / W in fp32: that quotient lies at least 1/(2W) from an integer, and its
// rounding error, below (i + 1/2) / W * 2^-23, stays smaller for every i < 2^22 (a chunk holds
// at most kBinLdsValues = 16384 values), so the truncation is exact.
template <int FB, int THREADS, bool FX>
__device__ __forceinline__ void flush_chunk(uint64_t* __restrict__ acc, int W, int plane, int nfl,
                                            float* __restrict__ dst, bool split, const FixedScale& fs) {
  const float rw = 1.0f / (float)W;
  auto slot = [&](int i) {
    const int q = (int)(((float)i + 0.5f) * rw);
    return (i - q * W) * plane + q;
  };
  if (split) {
    for (int i = threadIdx.x; i < nfl; i += THREADS) {
      const int a_i = slot(i);
      const float a = acc_value<FX>(acc, a_i, fs);
      acc[a_i] = 0u;
      if (a != 0.0f) atomic_add_f32(dst + i, a);
    }
    return;
  }
  for (int i0 = threadIdx.x; i0 < nfl; i0 += THREADS * FB) {
    float a[FB], gv[FB];
#pragma unroll
    for (int u = 0; u < FB; ++u) {
      const int i = i0 + u * THREADS;
      a[u] = 0.0f;
      if (i < nfl) {
        const int a_i = slot(i);
        a[u] = acc_value<FX>(acc, a_i, fs);
        acc[a_i] = 0u;
      }
    }
#pragma unroll
    for (int u = 0; u < FB; ++u)
      if (a[u] != 0.0f) gv[u] = dst[i0 + u * THREADS];
#pragma unroll
    for (int u = 0; u < FB; ++u)
      if (a[u] != 0.0f) dst[i0 + u * THREADS] = gv[u] + a[u];
  }
}

// One work item: accumulate its entries into the LDS chunk and flush the chunk into the
// gradient.  The claim of the next item (dynamic order) is issued between the two.  The
// kernel is compiled for one set of record widths (REC: d-linear records of W0 features;
// else Hermite entries of the widths W0, W1, W2, 0 = none): a kernel holding every width's
// loop gets the register allocation of the widest and spills the others' addresses.
template <bool FX, bool REC, int W0, int W1, int W2>
__device__ __forceinline__ void accumulate_item(uint64_t* __restrict__ acc, int W, int plane,
                                                const float* __restrict__ vseg, int32_t eb, const WorkItem& w,
                                                const FixedScale& fs) {
  if constexpr (REC) {
    accumulate_records<W0, FX>(acc, plane, vseg, eb, w.begin, w.end, fs);
  } else {
    if (W == W0) accumulate_entries<W0, FX>(acc, plane, vseg, eb, w.begin, w.end, fs);
    if constexpr (W1 > 0)
      if (W == W1) accumulate_entries<W1, FX>(acc, plane, vseg, eb, w.begin, w.end, fs);
    if constexpr (W2 > 0)
      if (W == W2) accumulate_entries<W2, FX>(acc, plane, vseg, eb, w.begin, w.end, fs);
  }
}

template <int ACC, int THREADS, bool FX, bool REC, int W0, int W1, int W2>
__device__ __forceinline__ void reduce_item(uint64_t* __restrict__ acc, const BinPlan& bp, int W, int plane, int nfl,
                                            const float* __restrict__ vseg, int32_t eb, const WorkItem& w,
                                            float* __restrict__ dst, const FixedScale& fs, bool claim,
                                            int32_t* __restrict__ ctr_ptr, int& claimed) {
  accumulate_item<FX, REC, W0, W1, W2>(acc, W, plane, vseg, eb, w, fs);
  if (claim && threadIdx.x == 0) {
    // the counter's (global) address through a register the compiler cannot see into:
    // otherwise the one-lane atomic becomes a wavefront-aggregated one whose result is read
    // back (and waited for) at once
    using global_i32 = __attribute__((address_space(1))) int32_t;
    global_i32* ctr = (global_i32*)ctr_ptr;
    __asm__ volatile("" : "+v"(ctr));
    claimed = __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  constexpr int FB = ACC / THREADS < kFlushBatch ? ACC / THREADS : kFlushBatch;
  flush_chunk<FB, THREADS, FX>(acc, W, plane, nfl, dst, w.split, fs);
}

// ACC fp64 accumulator values and THREADS lanes per workgroup: the 128 KB accumulator (one
// 1024-lane workgroup per CU) for bins of up to 16384 values, and a 16 KB one (eight 256-lane
// workgroups per CU) for the small bins of small grids, whose work items are short enough that
// the per-item latency (fetch, zero, flush) rather than the records sets the time.
template <int ACC, int THREADS, bool REC, int W0, int W1, int W2>
__global__ __launch_bounds__(THREADS) void bin_reduce_kernel(const Grid g, const BinPlan bp,
                                                                    BinState* __restrict__ st,
                                                                    const WorkItem* __restrict__ items,
                                                                    const float* __restrict__ vals,
                                                                    float* __restrict__ grad, int static_items) {
  // 64-bit accumulator words (fixed point, or fp64 for a chunk with a non-finite bound): LDS
  // 64-bit adds run several times faster than fp32 ones (ds_add_f32) on gfx950.
  // component planes of nrows + 1 values (odd for even nrows), so that the W components of a
  // row fall in different LDS banks when the flush reads them side by side
  __shared__ uint64_t acc[ACC + 32];
  __shared__ int item_sh[2];
  __shared__ int64_t vbase_sh[kMaxSeg];  // the segments' value and entry bases, read once
  __shared__ int32_t ebase_sh[kMaxSeg];
  __shared__ WorkItem next_sh[2];
  __shared__ uint32_t vmax_sh[kMaxSeg];
  for (int i = threadIdx.x; i < bp.nseg; i += THREADS) {
    vbase_sh[i] = st->seg_vbase[i];
    ebase_sh[i] = st->seg_ebase[i];
  }
  for (int i = threadIdx.x; i < bp.nseg; i += THREADS) vmax_sh[i] = st->vmax_bits[i];
  // zeroed once: every flush leaves the accumulator zero again
  for (int i = threadIdx.x; i < ACC + 32; i += THREADS) acc[i] = 0u;
  const int n_items = st->n_items;
  // Workgroup b takes item b first.  Dynamic order (static_items == 0): later items come
  // from a counter (which starts after the first gridDim.x items), claimed once the current
  // item's entries are accumulated: the claiming thread keeps the index in a register until
  // the flush is done, so the claim's round trip overlaps the flush's instead of holding the
  // barrier before it, and no item is held back during the long part.  Static order (small
  // batches, whose items are all short): workgroup b takes items b, b + gridDim.x, ..., and
  // each next item's descriptor is loaded while the current item runs.  Two slots, so a new
  // index or descriptor never overwrites the one others are still reading.
  int it = blockIdx.x;
  int slot = 0;
  if (threadIdx.x < 5 && it < n_items)
    reinterpret_cast<int*>(&next_sh[0])[threadIdx.x] = reinterpret_cast<const int*>(items + it)[threadIdx.x];
  __syncthreads();
  while (it < n_items) {
    const WorkItem w = next_sh[slot];
    // static order: the next descriptor, in a register of five lanes until the flush is done
    const int nxt = it + (int)gridDim.x;
    int pre = 0;
    if (static_items && threadIdx.x < 5 && nxt < n_items) {
      // a global vector load through a register the compiler cannot see into (not a scalar
      // or flat load): its wait comes at the use after the flush, not at the barriers between
      using global_ci32 = const __attribute__((address_space(1))) int32_t;
      global_ci32* src = (global_ci32*)(reinterpret_cast<const int32_t*>(items + nxt) + threadIdx.x);
      __asm__ volatile("" : "+v"(src));
      pre = *src;
    }
    const int sg = __builtin_amdgcn_readfirstlane(w.seg);
    const int k = sg / bp.L, l = sg % bp.L;
    const int W = bp.width[k];
    const int64_t C = bp.seg_chunk[sg];
    const int64_t chunk = __builtin_amdgcn_readfirstlane(w.bin) - bp.seg_bin0[sg];
    const int64_t row0 = chunk * C;
    const int64_t rem = seg_rows(g, bp.d, k, l) - row0;
    const int64_t nrows = rem < C ? rem : C;
    const int nfl = (int)(nrows * W);
    const int plane = (int)nrows + 1;
    // values of entry e of segment sg start at vseg + (e - ebase) * W
    const float* vseg = vals + vbase_sh[sg];
    const int32_t eb = ebase_sh[sg];
    int claimed = 0;  // counter value, the item index less gridDim.x
    float* dst = grad + g.off[k][l] + row0 * W;
    // the segment's value bound: 2^S puts it at 2^43 (a zero bound: every value is zero)
    const uint32_t vb = vmax_sh[sg];
    const bool fixed = vb < 0x7f800000u;
    FixedScale fs;
    {
      int e = 0;
      (void)frexpf(__uint_as_float(vb), &e);  // bound < 2^e
      fs.s = ldexp(1.0, 43 - e);
      fs.inv = ldexp(1.0, e - 43);
    }
    if (fixed)
      reduce_item<ACC, THREADS, true, REC, W0, W1, W2>(acc, bp, W, plane, nfl, vseg, eb, w, dst, fs, !static_items,
                                                       &st->next_item, claimed);
    else
      reduce_item<ACC, THREADS, false, REC, W0, W1, W2>(acc, bp, W, plane, nfl, vseg, eb, w, dst, fs, !static_items,
                                                        &st->next_item, claimed);
    if (static_items) {
      if (threadIdx.x < 5 && nxt < n_items) reinterpret_cast<int*>(&next_sh[slot ^ 1])[threadIdx.x] = pre;
      __syncthreads();
      it = nxt;
    } else {
      if (threadIdx.x == 0) item_sh[slot] = (int)gridDim.x + claimed;
      __syncthreads();
      it = item_sh[slot];
      if (threadIdx.x < 5 && it < n_items)
        reinterpret_cast<int*>(&next_sh[slot ^ 1])[threadIdx.x] = reinterpret_cast<const int*>(items + it)[threadIdx.x];
      __syncthreads();
    }
    slot ^= 1;
  }
}

// Workspace bound: every corner its own entry (single records on d-linear segments).
int64_t entries_per_point(int d, int L, bool hermite) { return bin_entries_per_point(d, L, hermite); }

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
  // Rows per bin: what the LDS accumulator holds at the table's width, but at most about
  // 1/512 of all rows, so that a small configuration still has a few hundred bins -- enough
  // to spread the reduce over the CUs without splitting bins into several work items, each of
  // which would accumulate and flush the whole chunk.  d-linear pair records keep the chunks
  // they need (whole x-lines of dense levels, 2N rows of hashed ones).
  int64_t all_rows = 0;
  for (int k = 0; k < bp.ntab; ++k)
    for (int l = 0; l < g.L; ++l) all_rows += seg_rows(g, d, k, l);
  int cap = 8;
  while ((int64_t(2) << cap) <= all_rows / 512) ++cap;
  if (!hermite)
    for (int l = 0; l < g.L; ++l) {
      const bool dense = (g.dense[0] >> l) & 1u;
      const int64_t need = dense ? (int64_t)g.N[l] + 1 : 2 * (int64_t)g.N[l];
      while ((int64_t(1) << cap) < need && cap < 30) ++cap;
    }
  for (int k = 0; k < bp.ntab; ++k) {
    int W = F;  // Hermite: C(d, k) slots of F floats
    if (hermite)
      for (int i = 1; i <= k; ++i) W = W * (d - k + i) / i;
    bp.width[k] = W;
    bp.cshift[k] = std::min(bin_cshift_for_width(W), cap);
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
  if (hermite) return d == 4 ? hermite4_scatter_points(F) : hermite_scatter_points(F);
  return dlinear_scatter_lds_bytes(bp, d, F, kScatterTileLarge) <= kMaxScatterLds ? kScatterTileLarge
                                                                                 : kScatterTileSmall;
}

size_t hermite_scatter_lds_bytes(const BinPlan& bp, int d, int F) {
  if (d == 4)  // one staged record of the widest table (6F values) per lane, 16 lanes a point
    return sizeof(int32_t) * (2 * (size_t)bp.max_level_bins + 16 * hermite4_scatter_points(F) / 64 + 3) +
           (size_t)16 * hermite4_scatter_points(F) * sizeof(float) * hermite_stage_width(6 * F);
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
  // about 512 count / scatter workgroups at least, when the levels allow (more groups re-read
  // the points and repeat the per-workgroup set-up: at 2^18 points of the 16-level d-linear
  // grid, 4 groups were slower than 1)
  int32_t groups = (int32_t)std::min<int64_t>(bp.L, (512 + w.nblk - 1) / w.nblk);
  w.lpg = (bp.L + groups - 1) / groups;
  w.lgroups = (bp.L + w.lpg - 1) / w.lpg;
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
  w.ups = off;
  off += al(bp.records || bp.d == 4 ? 0 : sizeof(float) * (size_t)chunk_points * bp.L * (1 + 2 * bp.d) * bp.width[0]);
  w.total = off;
  return w;
}

hipError_t run_bin_middle(const BinPlan& bp, const BinWorkspace& w, char* ws, hipStream_t s) {
  int32_t* counts = reinterpret_cast<int32_t*>(ws + w.counts);
  int32_t* totals = reinterpret_cast<int32_t*>(ws + w.totals);
  int32_t* seg_sums = reinterpret_cast<int32_t*>(ws + w.seg_sums);
  hipError_t e;
  if (w.nblk <= kScanOneRows) {
    hipLaunchKernelGGL(bin_scan_one_pass_kernel, dim3((unsigned)((bp.nbins + 63) / 64)), dim3(64 * kScanOneWaves), 0,
                       s, counts, w.nblk, bp.nbins, totals);
  } else {
    const dim3 sgrid((unsigned)((bp.nbins + 63) / 64), kScanSegs / kScanWavesPerBlock);
    hipLaunchKernelGGL(bin_scan_sums_kernel, sgrid, dim3(64 * kScanWavesPerBlock), 0, s, counts, w.nblk, bp.nbins,
                       seg_sums);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(bin_scan_apply_kernel, sgrid, dim3(64 * kScanWavesPerBlock), 0, s, counts, w.nblk, bp.nbins,
                       seg_sums, totals);
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(bin_plan_kernel, dim3(1), dim3(1024), 0, s, bp, totals,
                     reinterpret_cast<int32_t*>(ws + w.bin_start), reinterpret_cast<WorkItem*>(ws + w.items),
                     reinterpret_cast<BinState*>(ws + w.state), w.item_entries);
  return hipGetLastError();
}

hipError_t run_bin_reduce(const Grid& g, const BinPlan& bp, const BinWorkspace& w, char* ws, float* grad,
                          int64_t entries, hipStream_t s) {
  // small batches (few entries per bin): static item order with the next descriptor loaded
  // ahead, since every item is short and the per-item round trips set the time
  const int static_items = entries < (int64_t)bp.nbins * kSparseBinEntries ? 1 : 0;
  // the largest chunk of any table, in values: the small accumulator when it fits
  int64_t chunk_values = 0;
  for (int k = 0; k < bp.ntab; ++k) chunk_values = std::max<int64_t>(chunk_values, (int64_t)bp.width[k] << bp.cshift[k]);
  const bool small = chunk_values <= kBinLdsValuesSmall;
  // the plan's record widths select the kernel: d-linear F; Hermite F with 2F (d = 2),
  // 3F (d = 3) or 4F and 6F (d = 4)
  const int F = bp.width[0];
  const int code = bp.records ? F : bp.d * 100 + F;
  switch (code) {
#define HG_REDUCE(C, REC, W0, W1, W2)                                                                       \
  case C:                                                                                                   \
    if (small)                                                                                              \
      hipLaunchKernelGGL((bin_reduce_kernel<kBinLdsValuesSmall, 256, REC, W0, W1, W2>),                     \
                         dim3(kBinReduceBlocks * 8), dim3(256), 0, s, g, bp, reinterpret_cast<BinState*>(ws + w.state), \
                         reinterpret_cast<const WorkItem*>(ws + w.items), reinterpret_cast<const float*>(ws + w.vals), \
                         grad, static_items);                                                               \
    else                                                                                                    \
      hipLaunchKernelGGL((bin_reduce_kernel<kBinLdsValues, kReduceThreads, REC, W0, W1, W2>),               \
                         dim3(kBinReduceBlocks), dim3(kReduceThreads), 0, s, g, bp,                         \
                         reinterpret_cast<BinState*>(ws + w.state), reinterpret_cast<const WorkItem*>(ws + w.items), \
                         reinterpret_cast<const float*>(ws + w.vals), grad, static_items);                   \
    return hipGetLastError();
    HG_REDUCE(1, true, 1, 0, 0)
    HG_REDUCE(2, true, 2, 0, 0)
    HG_REDUCE(4, true, 4, 0, 0)
    HG_REDUCE(8, true, 8, 0, 0)
    HG_REDUCE(201, false, 1, 2, 0)
    HG_REDUCE(202, false, 2, 4, 0)
    HG_REDUCE(204, false, 4, 8, 0)
    HG_REDUCE(208, false, 8, 16, 0)
    HG_REDUCE(301, false, 1, 3, 0)
    HG_REDUCE(302, false, 2, 6, 0)
    HG_REDUCE(304, false, 4, 12, 0)
    HG_REDUCE(308, false, 8, 24, 0)
    HG_REDUCE(401, false, 1, 4, 6)
    HG_REDUCE(402, false, 2, 8, 12)
    HG_REDUCE(404, false, 4, 16, 24)
#undef HG_REDUCE
    default:
      return hipErrorInvalidValue;
  }
}

bool binned_fits(const Grid& g, int d, int F, bool hermite) {
  BinPlan bp;
  make_bin_plan(g, d, F, hermite, bp);
  const int32_t count_bins = bp.fine_shift >= 0 ? bp.fine_bin0[g.L] : bp.nbins;
  if (bp.nbins > kMaxBins || count_bins > kMaxBins) return false;  // LDS counters of the count pass
  for (int k = 0; k < bp.ntab; ++k)
    if (bp.width[k] > 24) return false;  // the reduce's widest record
  if (hermite) return hermite_scatter_lds_bytes(bp, d, F) <= kMaxScatterLds;
  const int tile = bin_tile_points(bp, d, F, hermite);
  return dlinear_scatter_lds_bytes(bp, d, F, tile) <= kMaxScatterLds;
}

size_t binned_backward_workspace_bytes(const Grid& g, int d, int F, bool hermite, int64_t n) {
  BinPlan bp;
  make_bin_plan(g, d, F, hermite, bp);
  const int64_t cmax = bin_chunk_points(g, d, hermite);
  const int64_t c = n < cmax ? n : cmax;
  return bin_workspace_layout(bp, c, entries_per_point(d, g.L, hermite), floats_per_point(bp, d),
                              bin_tile_points(bp, d, F, hermite)).total;
}

BinWorkspace bin_workspace_for(const Grid& g, const BinPlan& bp, int d, int F, bool hermite, int64_t chunk_points) {
  return bin_workspace_layout(bp, chunk_points, entries_per_point(d, g.L, hermite), floats_per_point(bp, d),
                              bin_tile_points(bp, d, F, hermite));
}

hipError_t run_binned_backward(const Grid& g, int d, int F, bool hermite, int d2_mode, int64_t n,
                               const float* x, const float* g_gamma, const float* g_dgamma,
                               const float* g_d2gamma, const float* u_levels, float* grad, void* workspace,
                               hipStream_t s, int64_t max_chunk, bool counted) {
  BinPlan bp;
  make_bin_plan(g, d, F, hermite, bp);
  int64_t cmax = bin_chunk_points(g, d, hermite);
  if (max_chunk > 0 && max_chunk < cmax) cmax = max_chunk;
  if ((u_levels || counted) && n > cmax) return hipErrorInvalidValue;  // one chunk only
  char* ws = static_cast<char*>(workspace);
  const int64_t LF = (int64_t)g.Lrow * F;  // upstream row stride
  for (int64_t p0 = 0; p0 < n; p0 += cmax) {
    const int64_t c = (n - p0) < cmax ? (n - p0) : cmax;
    const BinWorkspace w = bin_workspace_for(g, bp, d, F, hermite, c);
    const float* xc = x + p0 * d;
    const float* gg = g_gamma ? g_gamma + p0 * LF : nullptr;
    const float* gd = g_dgamma ? g_dgamma + p0 * d * LF : nullptr;
    const float* g2 = g_d2gamma ? g_d2gamma + p0 * (d2_mode == HASHENC_D2_DIAG ? d : 1) * LF : nullptr;
    for (int pass = counted ? 1 : 0; pass < 2; ++pass) {
      if (counted && pass == 1) {  // the counting forward left this chunk's counts
        hipError_t e = run_bin_middle(bp, w, ws, s);
        if (e != hipSuccess) return e;
      }
      hipError_t e = !hermite ? launch_dlinear_bin(g, bp, w, ws, d, F, pass == 1, c, xc, gg, u_levels, s)
                     : d == 4 ? launch_hermite4_bin(g, bp, w, ws, F, d2_mode, pass == 1, c, xc, gg, gd, g2, s)
                              : launch_hermite_bin(g, bp, w, ws, d, F, d2_mode, pass == 1, c, xc, gg, gd, g2,
                                                   u_levels, s);
      if (e != hipSuccess) return e;
      if (pass == 0) {
        e = run_bin_middle(bp, w, ws, s);
        if (e != hipSuccess) return e;
      }
    }
    hipError_t e = run_bin_reduce(g, bp, w, ws, grad, c * entries_per_point(d, g.L, hermite), s);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace hg
