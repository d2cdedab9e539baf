// Coarse-to-fine level activation (Hermite-NGP reading notes, section 方法详解, key design
// 3): the kernels compute only the active levels; the point-major outputs written directly
// by the forward kernels get their inactive levels' columns cleared here.
#include "hashenc_internal.h"

namespace hg {
namespace {

// Grid-stride over the rows x w floats of the cleared columns, w = row_floats - from:
// consecutive threads write consecutive floats of a row's cleared run.
__global__ __launch_bounds__(kBlock) void zero_columns_kernel(float* __restrict__ out, int64_t rows,
                                                              int32_t row_floats, int32_t from) {
  const int32_t w = row_floats - from;
  const int64_t total = rows * w;
  const int64_t stride = (int64_t)gridDim.x * kBlock;
  for (int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x; i < total; i += stride) {
    const int64_t r = i / w;
    out[r * row_floats + from + (i - r * w)] = 0.0f;
  }
}

}  // namespace

hipError_t launch_zero_columns(float* out, int64_t rows, int32_t row_floats, int32_t from, hipStream_t s) {
  if (from < 0 || from > row_floats) return hipErrorInvalidValue;
  const int64_t total = rows * (int64_t)(row_floats - from);
  if (total == 0) return hipSuccess;
  int64_t blocks = (total + kBlock - 1) / kBlock;
  if (blocks > 256 * 64) blocks = 256 * 64;  // grid-stride: 64 workgroups per CU
  hipLaunchKernelGGL(zero_columns_kernel, dim3((unsigned)blocks), dim3(kBlock), 0, s, out, rows, row_floats, from);
  return hipGetLastError();
}

}  // namespace hg
