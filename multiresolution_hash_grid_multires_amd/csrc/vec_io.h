// Vector loads and stores of F consecutive floats (F = 1, 2, 3, 4, 6, 8) with the widest
// naturally aligned access the layout guarantees: rows of F = 2 are 8-byte aligned,
// F = 4 and 8 rows 16-byte aligned; widths 3 and 6 occur for Hermite order tables.
#pragma once

#include <hip/hip_runtime.h>

#include <utility>

namespace hg {

template <int W>
__device__ __forceinline__ void load_vec(const float* __restrict__ p, float (&v)[W]) {
  if constexpr (W % 4 == 0) {
#pragma unroll
    for (int j = 0; j < W / 4; ++j) {
      const float4 a = reinterpret_cast<const float4*>(p)[j];
      v[4 * j] = a.x; v[4 * j + 1] = a.y; v[4 * j + 2] = a.z; v[4 * j + 3] = a.w;
    }
  } else if constexpr (W % 2 == 0) {
#pragma unroll
    for (int j = 0; j < W / 2; ++j) {
      const float2 a = reinterpret_cast<const float2*>(p)[j];
      v[2 * j] = a.x; v[2 * j + 1] = a.y;
    }
  } else {
#pragma unroll
    for (int j = 0; j < W; ++j) v[j] = p[j];
  }
}

// Load W floats into v[off .. off+W) of a larger array.
template <int W, int N>
__device__ __forceinline__ void load_vec_at(const float* __restrict__ p, float (&v)[N], int off) {
  float tmp[W];
  load_vec<W>(p, tmp);
#pragma unroll
  for (int j = 0; j < W; ++j) v[off + j] = tmp[j];
}

template <int W>
__device__ __forceinline__ void store_vec(float* __restrict__ p, const float (&v)[W]) {
  if constexpr (W % 4 == 0) {
#pragma unroll
    for (int j = 0; j < W / 4; ++j)
      reinterpret_cast<float4*>(p)[j] = make_float4(v[4 * j], v[4 * j + 1], v[4 * j + 2], v[4 * j + 3]);
  } else if constexpr (W % 2 == 0) {
#pragma unroll
    for (int j = 0; j < W / 2; ++j)
      reinterpret_cast<float2*>(p)[j] = make_float2(v[2 * j], v[2 * j + 1]);
  } else {
#pragma unroll
    for (int j = 0; j < W; ++j) p[j] = v[j];
  }
}

// Non-temporal variants (the "nt" cache policy): for streams written or read exactly once,
// so they do not displace table lines from the caches.
typedef float float2_nt __attribute__((ext_vector_type(2)));
typedef float float4_nt __attribute__((ext_vector_type(4)));

template <int W>
__device__ __forceinline__ void store_vec_nt(float* __restrict__ p, const float (&v)[W]) {
  if constexpr (W % 4 == 0) {
#pragma unroll
    for (int j = 0; j < W / 4; ++j) {
      float4_nt a = {v[4 * j], v[4 * j + 1], v[4 * j + 2], v[4 * j + 3]};
      __builtin_nontemporal_store(a, reinterpret_cast<float4_nt*>(p) + j);
    }
  } else if constexpr (W % 2 == 0) {
#pragma unroll
    for (int j = 0; j < W / 2; ++j) {
      float2_nt a = {v[2 * j], v[2 * j + 1]};
      __builtin_nontemporal_store(a, reinterpret_cast<float2_nt*>(p) + j);
    }
  } else {
#pragma unroll
    for (int j = 0; j < W; ++j) __builtin_nontemporal_store(v[j], p + j);
  }
}

template <int W>
__device__ __forceinline__ void load_vec_nt(const float* __restrict__ p, float (&v)[W]) {
  if constexpr (W % 4 == 0) {
#pragma unroll
    for (int j = 0; j < W / 4; ++j) {
      const float4_nt a = __builtin_nontemporal_load(reinterpret_cast<const float4_nt*>(p) + j);
      v[4 * j] = a.x; v[4 * j + 1] = a.y; v[4 * j + 2] = a.z; v[4 * j + 3] = a.w;
    }
  } else if constexpr (W % 2 == 0) {
#pragma unroll
    for (int j = 0; j < W / 2; ++j) {
      const float2_nt a = __builtin_nontemporal_load(reinterpret_cast<const float2_nt*>(p) + j);
      v[2 * j] = a.x; v[2 * j + 1] = a.y;
    }
  } else {
#pragma unroll
    for (int j = 0; j < W; ++j) v[j] = __builtin_nontemporal_load(p + j);
  }
}

}  // namespace hg
