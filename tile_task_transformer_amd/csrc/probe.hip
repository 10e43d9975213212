// On-chip peak probe: back-to-back fp32 matrix-core instructions with no
// memory traffic, the ceiling the GEMM and attention kernels are measured
// against on the running device (the published MI355X fp32 matrix peak is
// 256 CUs x 4 SIMDs x 2.4 GHz x 64 flop/clk = 157.3 TFLOP/s).
#include "common.hpp"

namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));

// Each wave keeps four independent 32x32 accumulators so that consecutive
// v_mfma_f32_32x32x2_f32 never wait on each other's result; every lane
// stores the sum of its accumulators, so nothing is dead code.
__global__ __launch_bounds__(256) void mfma_probe(int iters, float* __restrict__ out) {
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  const float a = 1e-3f * (float)(threadIdx.x & 7), b = 1e-3f;
  for (int i = 0; i < iters; ++i) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x2f32(b, a, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x2f32(a, a, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x2f32(b, b, c3, 0, 0, 0);
  }
  float s = 0.f;
  for (int j = 0; j < 16; ++j) s += c0[j] + c1[j] + c2[j] + c3[j];
  out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

}  // namespace

extern "C" int tt_probe_mfma_f32(void* stream, int64_t blocks, int64_t iters, float* out, double* flops) {
  if (blocks < 1 || blocks > 65535 || iters < 1 || iters > (1 << 24))
    return tt::fail(TT_ERR_ARG, "tt_probe_mfma_f32: blocks must be 1..65535 and iters 1..2^24");
  if (!out) return tt::fail(TT_ERR_ARG, "tt_probe_mfma_f32: null output");
  if (flops) *flops = (double)blocks * 4.0 /* waves */ * (double)iters * 4.0 /* chains */ * 4096.0;
  hipLaunchKernelGGL(mfma_probe, dim3((unsigned)blocks), dim3(256), 0, tt::as_stream(stream), (int)iters, out);
  return tt::launch_status("tt_probe_mfma_f32");
}

// ---- HBM probes: the practical bandwidth of plain streams on the running
// device, the ceiling the memory-bound kernels are measured against beside
// the published 8 TB/s. Grid-stride over 16-byte elements with four loads
// in flight per thread; read (every element summed, one sum per thread
// written), write (a constant stored) and copy (1:1 read and write), the
// loads and stores optionally non-temporal.

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

template <int MODE, bool NT>
__global__ __launch_bounds__(256) void hbm_probe(const f32x4* __restrict__ src, f32x4* __restrict__ dst, int64_t n4,
                                                 float* __restrict__ red) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  auto put = [&](int64_t k, f32x4 v) {
    if (NT) __builtin_nontemporal_store(v, dst + k);
    else dst[k] = v;
  };
  auto get = [&](int64_t k) -> f32x4 {
    if (NT) return __builtin_nontemporal_load(src + k);
    return src[k];
  };
  if (MODE == TT_PROBE_READ) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (; i + 3 * stride < n4; i += 4 * stride) {
      const f32x4 v0 = get(i), v1 = get(i + stride), v2 = get(i + 2 * stride), v3 = get(i + 3 * stride);
      acc += (v0 + v1) + (v2 + v3);
    }
    for (; i < n4; i += stride) acc += get(i);
    red[(int64_t)blockIdx.x * 256 + threadIdx.x] = acc[0] + acc[1] + acc[2] + acc[3];
  } else if (MODE == TT_PROBE_WRITE) {
    const f32x4 v = {1.f, 2.f, 3.f, (float)blockIdx.x};
    for (; i < n4; i += stride) put(i, v);
  } else {
    for (; i + 3 * stride < n4; i += 4 * stride) {
      const f32x4 v0 = get(i), v1 = get(i + stride), v2 = get(i + 2 * stride), v3 = get(i + 3 * stride);
      put(i, v0);
      put(i + stride, v1);
      put(i + 2 * stride, v2);
      put(i + 3 * stride, v3);
    }
    for (; i < n4; i += stride) put(i, get(i));
  }
}

}  // namespace

extern "C" int tt_probe_hbm(void* stream, int mode, const float* src, float* dst, int64_t n, int64_t blocks,
                            double* bytes) {
  const int kind = mode & 3;
  const bool nt = (mode & TT_PROBE_NONTEMPORAL) != 0;
  if ((mode & ~(3 | TT_PROBE_NONTEMPORAL)) || kind > TT_PROBE_COPY)
    return tt::fail(TT_ERR_ARG, "tt_probe_hbm: unknown mode %d", mode);
  if (n < 0 || n % 4 || blocks < 1 || blocks > 65535)
    return tt::fail(TT_ERR_ARG, "tt_probe_hbm: n must be a multiple of 4 and blocks 1..65535");
  if ((kind != TT_PROBE_WRITE && !src) || !dst) return tt::fail(TT_ERR_ARG, "tt_probe_hbm: null buffer");
  if ((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst)) & 15)
    return tt::fail(TT_ERR_ARG, "tt_probe_hbm: buffers must be 16-byte aligned");
  if (bytes) *bytes = (double)n * 4.0 * (kind == TT_PROBE_COPY ? 2.0 : 1.0);
  hipStream_t s = tt::as_stream(stream);
  const dim3 grid((unsigned)blocks), block(256);
  const f32x4* a = reinterpret_cast<const f32x4*>(src);
  f32x4* b = reinterpret_cast<f32x4*>(dst);
  if (kind == TT_PROBE_READ && nt) hipLaunchKernelGGL((hbm_probe<TT_PROBE_READ, true>), grid, block, 0, s, a, b, n / 4, dst);
  else if (kind == TT_PROBE_READ) hipLaunchKernelGGL((hbm_probe<TT_PROBE_READ, false>), grid, block, 0, s, a, b, n / 4, dst);
  else if (kind == TT_PROBE_WRITE && nt) hipLaunchKernelGGL((hbm_probe<TT_PROBE_WRITE, true>), grid, block, 0, s, a, b, n / 4, dst);
  else if (kind == TT_PROBE_WRITE) hipLaunchKernelGGL((hbm_probe<TT_PROBE_WRITE, false>), grid, block, 0, s, a, b, n / 4, dst);
  else if (nt) hipLaunchKernelGGL((hbm_probe<TT_PROBE_COPY, true>), grid, block, 0, s, a, b, n / 4, dst);
  else hipLaunchKernelGGL((hbm_probe<TT_PROBE_COPY, false>), grid, block, 0, s, a, b, n / 4, dst);
  return tt::launch_status("tt_probe_hbm");
}
