// Device helpers for the memory-bound row kernels (LayerNorm, softmax,
// cross-entropy, reductions): wave64 reductions and bounds-checked float4
// access. Every reduction here combines lanes in a fixed butterfly order,
// so results do not depend on scheduling (bitwise reproducible).
#pragma once

#include "common.hpp"

namespace tt {

typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// float4 at columns c..c+3 of row r (row-major, leading dimension ld);
// columns >= cols read as 0. VEC: the row start is 16-byte aligned.
template <bool VEC>
__device__ __forceinline__ f32x4 ld4(const float* __restrict__ p, int64_t ld, int64_t r, int c, int cols) {
  const float* q = p + r * ld + c;
  if (VEC && c + 3 < cols) return *reinterpret_cast<const f32x4*>(q);
  f32x4 v = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < 4; ++i)
    if (c + i < cols) v[i] = q[i];
  return v;
}

// ld4 for data read once (a streaming sweep): the 16-byte load is
// non-temporal
template <bool VEC>
__device__ __forceinline__ f32x4 ld4_nt(const float* __restrict__ p, int64_t ld, int64_t r, int c, int cols) {
  const float* q = p + r * ld + c;
  if (VEC && c + 3 < cols) return __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(q));
  f32x4 v = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < 4; ++i)
    if (c + i < cols) v[i] = q[i];
  return v;
}

template <bool VEC>
__device__ __forceinline__ void st4(float* __restrict__ p, int64_t ld, int64_t r, int c, int cols, f32x4 v) {
  float* q = p + r * ld + c;
  if (VEC && c + 3 < cols) {
    *reinterpret_cast<f32x4*>(q) = v;
    return;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
    if (c + i < cols) q[i] = v[i];
}

// gamma/bias vectors (contiguous)
template <bool VEC>
__device__ __forceinline__ f32x4 ldv4(const float* __restrict__ p, int c, int cols) {
  return ld4<VEC>(p, 0, 0, c, cols);
}

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

}  // namespace tt
