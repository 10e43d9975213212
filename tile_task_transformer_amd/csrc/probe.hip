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
