// Diagnostic kernels: export of the lookup stage (corner rows per point and level), a plain
// streaming copy used to calibrate bandwidth figures, and a cache-resident read that gives
// the L2 ceiling the gather kernels are compared with.
#include "hashenc_internal.h"

namespace hg {
namespace {

template <int D>
__global__ __launch_bounds__(kBlock) void debug_indices_kernel(const Grid g, int order, int64_t n,
                                                               const float* __restrict__ x,
                                                               int32_t* __restrict__ out) {
  const int64_t p = (int64_t)blockIdx.x * kBlock + threadIdx.x;
  if (p >= n) return;
  float xp[D];
  for (int i = 0; i < D; ++i) xp[i] = x[p * D + i];
  for (int l = 0; l < g.L; ++l) {
    uint32_t base[D];
    float t[D];
    locate<D>(xp, g.N[l], g.Nf[l], base, t);
    const CellKeys<D> keys = cell_keys<D>(base, g.N[l]);
    const bool dense = (g.dense[order] >> l) & 1u;
    for (int c = 0; c < (1 << D); ++c)
      out[(p * g.L + l) * (1 << D) + c] =
          (int32_t)corner_row_rt<D>(keys, c, dense, g.T[order], g.Tmask[order]);
  }
}

// Streaming copy tuned for HBM: a workgroup moves whole 16 KB pieces, each lane four 16-byte
// loads in flight before its four stores, with the non-temporal cache policy on both sides
// (nothing is reused).  Of the variants measured on MI355X over 4 GiB (one or four loads per
// lane, temporal or not, 1024..8192 workgroups, eight loads per lane) this one was fastest:
// 5.44 TB/s of read + write against 4.83 TB/s for one plain load per lane.
constexpr int kCopyUnroll = 4;
constexpr int64_t kCopyPiece = (int64_t)kBlock * kCopyUnroll;  // float4 per workgroup piece
constexpr int kCopyBlocks = 4096;
typedef float copy_f4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kBlock) void copy_kernel(const copy_f4* __restrict__ src,
                                                      copy_f4* __restrict__ dst, int64_t n4) {
  const int64_t pieces = n4 / kCopyPiece;
  for (int64_t c = blockIdx.x; c < pieces; c += gridDim.x) {
    const int64_t base = c * kCopyPiece + threadIdx.x;
    copy_f4 v[kCopyUnroll];
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) v[u] = __builtin_nontemporal_load(src + base + u * kBlock);
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) __builtin_nontemporal_store(v[u], dst + base + u * kBlock);
  }
  // the float4 past the last whole piece
  for (int64_t i = pieces * kCopyPiece + (int64_t)blockIdx.x * kBlock + threadIdx.x; i < n4;
       i += (int64_t)gridDim.x * kBlock)
    dst[i] = src[i];
}

__global__ void copy_tail_kernel(const float* __restrict__ src, float* __restrict__ dst,
                                 int64_t begin, int64_t n) {
  const int64_t i = begin + threadIdx.x;
  if (i < n) dst[i] = src[i];
}

// L2-resident read.  The buffer is cut into kXcds equal slices; workgroup b reads slice
// b % kXcds, the slice of the XCD it is dispatched to (workgroups go round-robin to the
// XCDs), so after the first pass every read is served by that XCD's L2.  A CU holds 8
// workgroups that each walk their own part of the slice: at 3 MB per slice that is about
// 96 KB per CU per pass, more than the 32 KB vector L1, so the cyclic walk misses L1.  The
// sum is stored only if it takes a value that a buffer of ones cannot give, which keeps the
// loads without writing anything.
constexpr int kXcds = 8;
constexpr int kCacheReadBlocks = kXcds * 256;

__global__ __launch_bounds__(kBlock) void cache_read_kernel(const float4* __restrict__ buf, int64_t slice4,
                                                            int32_t reps, float* __restrict__ out) {
  const int xcd = blockIdx.x % kXcds;
  const int64_t j = blockIdx.x / kXcds;
  const int64_t stride = (int64_t)(kCacheReadBlocks / kXcds) * kBlock;
  const float4* s = buf + xcd * slice4;
  float acc = 0.0f;
  for (int r = 0; r < reps; ++r) {
    for (int64_t i = j * kBlock + threadIdx.x; i < slice4; i += stride) {
      const float4 v = s[i];
      acc += (v.x + v.y) + (v.z + v.w);
    }
  }
  if (acc == -1.0f) out[0] = acc;
}

}  // namespace

hipError_t launch_debug_indices(const Grid& g, int d, int order, int64_t n, const float* x,
                                int32_t* out, hipStream_t s) {
  const dim3 grid((unsigned)((n + kBlock - 1) / kBlock));
  if (d == 2)
    hipLaunchKernelGGL(debug_indices_kernel<2>, grid, dim3(kBlock), 0, s, g, order, n, x, out);
  else if (d == 3)
    hipLaunchKernelGGL(debug_indices_kernel<3>, grid, dim3(kBlock), 0, s, g, order, n, x, out);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_copy(const float* src, float* dst, int64_t n, hipStream_t s) {
  const int64_t n4 = n / 4;
  if (n4 > 0) {
    int64_t blocks = (n4 + kCopyPiece - 1) / kCopyPiece;
    if (blocks > kCopyBlocks) blocks = kCopyBlocks;  // grid-stride over the pieces
    hipLaunchKernelGGL(copy_kernel, dim3((unsigned)blocks), dim3(kBlock), 0, s,
                       reinterpret_cast<const copy_f4*>(src), reinterpret_cast<copy_f4*>(dst), n4);
  }
  if (n % 4) hipLaunchKernelGGL(copy_tail_kernel, dim3(1), dim3(4), 0, s, src, dst, n4 * 4, n);
  return hipGetLastError();
}

int64_t cache_read_granule() { return 4 * kXcds; }

hipError_t launch_cache_read(const float* buf, int64_t n, int32_t reps, float* out, hipStream_t s) {
  const int64_t slice4 = n / (4 * kXcds);
  hipLaunchKernelGGL(cache_read_kernel, dim3(kCacheReadBlocks), dim3(kBlock), 0, s,
                     reinterpret_cast<const float4*>(buf), slice4, reps, out);
  return hipGetLastError();
}

}  // namespace hg
