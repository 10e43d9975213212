// tile_gemm: fp32 GEMM on the CDNA4 matrix cores (v_mfma_f32_32x32x2_f32).
//
// The linear layers and the tied LM head of the GPT2 step are dense
// contractions, so their tile tasks run on MFMA in true fp32 (no xf32/TF32).
//
// Work decomposition (one launch = one tile task):
//   * a workgroup of 256 threads (4 wave64s, 2x2) computes a BM x BN block of
//     C; each wave owns a (BM/2) x (BN/2) sub-block made of 32x32 MFMA tiles
//     whose fp32 accumulators stay in registers for the whole K loop;
//   * K advances in steps of BK through two LDS buffers: the next step's
//     global loads are issued before the current step's MFMAs and written to
//     the other buffer afterwards, so one barrier per step suffices;
//   * each operand is staged in LDS in the orientation it has in HBM, so the
//     global->LDS path is always 16-byte vector loads/stores:
//       K-contiguous operands (A, or B^T)  -> LDS [rows][BK + 4]
//       row-contiguous operands (A^T, B)   -> LDS [BK][rows + 4]
//   * the summation order inside each group of 8 k values is permuted so a
//     lane's 4 consecutive MFMA steps use 4 consecutive k of its half-wave:
//     k = 8*kb + 4*(lane/32) + s. A K-contiguous operand then feeds 4 MFMAs
//     from one 16-byte LDS read;
//   * blockIdx is remapped so consecutive C blocks land on the same XCD
//     (workgroups are dispatched round-robin over the 8 XCDs, each with its
//     own L2), then grouped along M for L2 reuse of the B panel.
// Ragged M, N, K are handled by zero-filling out-of-range loads and
// predicating stores; leading dimensions that are not multiples of 4 (or
// unaligned pointers) select a scalar-load instantiation.
#include "common.hpp"

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

struct GemmArgs {
  int m, n, k;
  float alpha, beta;
  const float* A;
  const float* B;
  float* C;
  int64_t lda, ldb, ldc;
  int epi;
  const float* bias;
  const float* res;
  int64_t ldr;
  float* aux;
  int64_t ldaux;
};

__device__ __forceinline__ float gelu_tanh(float u) {
  const float c = 0.7978845608028654f;  // sqrt(2/pi)
  float a = c * (u + 0.044715f * u * u * u);
  return 0.5f * u * (1.f + tanhf(a));
}

__device__ __forceinline__ float gelu_tanh_grad(float u) {
  const float c = 0.7978845608028654f;
  float a = c * (u + 0.044715f * u * u * u);
  float t = tanhf(a);
  return 0.5f * (1.f + t) + 0.5f * u * (1.f - t * t) * c * (1.f + 3.f * 0.044715f * u * u);
}

// Loads a float4 of an operand at (r, c) of a matrix with `rows` x `cols`
// valid elements (row-major, leading dimension ld), zero-filling outside.
template <bool VEC>
__device__ __forceinline__ f32x4 load4(const float* __restrict__ p, int64_t ld, int r, int c, int rows,
                                       int cols) {
  f32x4 v = {0.f, 0.f, 0.f, 0.f};
  if (r >= rows) return v;
  const float* q = p + (int64_t)r * ld + c;
  if (VEC && c + 3 < cols) return *reinterpret_cast<const f32x4*>(q);
#pragma unroll
  for (int i = 0; i < 4; ++i)
    if (c + i < cols) v[i] = q[i];
  return v;
}

template <int BM, int BN, int BK, bool TA, bool TB, bool VA, bool VB>
__global__ __launch_bounds__(256) void gemm_kernel(GemmArgs g) {
  constexpr int WM = BM / 2, WN = BN / 2;      // wave sub-block
  constexpr int FM = WM / 32, FN = WN / 32;    // 32x32 MFMA tiles per wave
  // LDS geometry per operand: "KC" = [rows][BK+4], "RC" = [BK][rows+4]
  constexpr int A_KC = !TA, B_KC = TB;
  constexpr int A_LD = A_KC ? BK + 4 : BM + 4;
  constexpr int B_LD = B_KC ? BK + 4 : BN + 4;
  constexpr int A_SZ = A_KC ? BM * A_LD : BK * A_LD;
  constexpr int B_SZ = B_KC ? BN * B_LD : BK * B_LD;
  // float4 slots per operand tile and per thread
  constexpr int A_V4 = BM * BK / 4, B_V4 = BN * BK / 4;
  constexpr int A_PT = A_V4 / 256, B_PT = B_V4 / 256;
  static_assert(A_V4 % 256 == 0 && B_V4 % 256 == 0, "tile must split evenly over 256 threads");

  __shared__ __attribute__((aligned(16))) float lds[2 * (A_SZ + B_SZ)];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int half = lane >> 5, l32 = lane & 31;

  // ---- block -> C tile: XCD-contiguous, then grouped along M
  const int grid_m = (g.m + BM - 1) / BM, grid_n = (g.n + BN - 1) / BN;
  const int nb = grid_m * grid_n;
  int b = blockIdx.x;
  {
    const int per = nb / 8, rem = nb % 8, x = b % 8;
    b = x * per + min(x, rem) + b / 8;
  }
  constexpr int GROUP = 8;
  const int in_group = GROUP * grid_n;
  const int first_m = (b / in_group) * GROUP;
  const int gsz = min(grid_m - first_m, GROUP);
  const int tm = first_m + (b % in_group) % gsz;
  const int tn = (b % in_group) / gsz;
  const int m0 = tm * BM, n0 = tn * BN;

  // ---- global -> register staging
  f32x4 ra[A_PT], rb[B_PT];
  auto gload = [&](int k0) {
#pragma unroll
    for (int i = 0; i < A_PT; ++i) {
      int idx = tid + 256 * i;
      if (A_KC) {  // A[m][k]: rows m, 4-wide along k
        int r = idx / (BK / 4), c = (idx % (BK / 4)) * 4;
        ra[i] = load4<VA>(g.A, g.lda, m0 + r, k0 + c, g.m, g.k);
      } else {     // A^T stored [k][m]: rows k, 4-wide along m
        int r = idx / (BM / 4), c = (idx % (BM / 4)) * 4;
        ra[i] = load4<VA>(g.A, g.lda, k0 + r, m0 + c, g.k, g.m);
      }
    }
#pragma unroll
    for (int i = 0; i < B_PT; ++i) {
      int idx = tid + 256 * i;
      if (B_KC) {  // B^T stored [n][k]
        int r = idx / (BK / 4), c = (idx % (BK / 4)) * 4;
        rb[i] = load4<VB>(g.B, g.ldb, n0 + r, k0 + c, g.n, g.k);
      } else {     // B stored [k][n]
        int r = idx / (BN / 4), c = (idx % (BN / 4)) * 4;
        rb[i] = load4<VB>(g.B, g.ldb, k0 + r, n0 + c, g.k, g.n);
      }
    }
  };
  auto sstore = [&](int buf) {
    float* As = lds + buf * (A_SZ + B_SZ);
    float* Bs = As + A_SZ;
#pragma unroll
    for (int i = 0; i < A_PT; ++i) {
      int idx = tid + 256 * i;
      int r = A_KC ? idx / (BK / 4) : idx / (BM / 4);
      int c = A_KC ? (idx % (BK / 4)) * 4 : (idx % (BM / 4)) * 4;
      *reinterpret_cast<f32x4*>(As + r * A_LD + c) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < B_PT; ++i) {
      int idx = tid + 256 * i;
      int r = B_KC ? idx / (BK / 4) : idx / (BN / 4);
      int c = B_KC ? (idx % (BK / 4)) * 4 : (idx % (BN / 4)) * 4;
      *reinterpret_cast<f32x4*>(Bs + r * B_LD + c) = rb[i];
    }
  };

  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int nk = (g.k + BK - 1) / BK;
  gload(0);
  sstore(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) gload((kt + 1) * BK);
    const float* As = lds + cur * (A_SZ + B_SZ);
    const float* Bs = As + A_SZ;
#pragma unroll
    for (int kb = 0; kb < BK / 8; ++kb) {
      const int kk = kb * 8 + half * 4;   // this half-wave's 4 consecutive k
      f32x4 fa[FM], fb[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const int row = wm * WM + i * 32 + l32;
        if (A_KC) {
          fa[i] = *reinterpret_cast<const f32x4*>(As + row * A_LD + kk);
        } else {
#pragma unroll
          for (int s = 0; s < 4; ++s) fa[i][s] = As[(kk + s) * A_LD + row];
        }
      }
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int col = wn * WN + j * 32 + l32;
        if (B_KC) {
          fb[j] = *reinterpret_cast<const f32x4*>(Bs + col * B_LD + kk);
        } else {
#pragma unroll
          for (int s = 0; s < 4; ++s) fb[j][s] = Bs[(kk + s) * B_LD + col];
        }
      }
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(fa[i][s], fb[j][s], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) sstore(cur ^ 1);
    __syncthreads();
  }

  // ---- epilogue: accumulator register r of lane l holds
  //      row 8*(r/4) + 4*(l/32) + (r%4), column l%32 of its 32x32 tile
  const bool gelu = g.epi & TT_EPI_GELU, gelu_bwd = g.epi & TT_EPI_GELU_BWD;
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int col = n0 + wn * WN + j * 32 + l32;
      if (col >= g.n) continue;
      const float bcol = (g.epi & TT_EPI_BIAS) ? g.bias[col] : 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = m0 + wm * WM + i * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
        if (row >= g.m) continue;
        float v = g.alpha * acc[i][j][r];
        if (g.beta != 0.f) {
          const float src = gelu ? g.aux[(int64_t)row * g.ldaux + col] : g.C[(int64_t)row * g.ldc + col];
          v += g.beta * src;
        }
        v += bcol;
        if (g.epi & TT_EPI_RES) v += g.res[(int64_t)row * g.ldr + col];
        if (gelu) {
          g.aux[(int64_t)row * g.ldaux + col] = v;
          v = gelu_tanh(v);
        } else if (gelu_bwd) {
          v *= gelu_tanh_grad(g.aux[(int64_t)row * g.ldaux + col]);
        }
        g.C[(int64_t)row * g.ldc + col] = v;
      }
    }
}

template <int BM, int BN, int BK, bool TA, bool TB>
int launch_v(const GemmArgs& g, bool va, bool vb, hipStream_t s) {
  const int nb = ((g.m + BM - 1) / BM) * ((g.n + BN - 1) / BN);
  dim3 grid(nb), block(256);
  if (va && vb) hipLaunchKernelGGL((gemm_kernel<BM, BN, BK, TA, TB, true, true>), grid, block, 0, s, g);
  else if (va) hipLaunchKernelGGL((gemm_kernel<BM, BN, BK, TA, TB, true, false>), grid, block, 0, s, g);
  else if (vb) hipLaunchKernelGGL((gemm_kernel<BM, BN, BK, TA, TB, false, true>), grid, block, 0, s, g);
  else hipLaunchKernelGGL((gemm_kernel<BM, BN, BK, TA, TB, false, false>), grid, block, 0, s, g);
  return tt::launch_status("tile_gemm");
}

template <bool TA, bool TB>
int launch_t(const GemmArgs& g, bool va, bool vb, hipStream_t s) {
  // 128x128 blocks when they give at least ~2 blocks per CU, else 64x64
  const int64_t big = ((int64_t)(g.m + 127) / 128) * ((g.n + 127) / 128);
  if (big >= 512) return launch_v<128, 128, 16, TA, TB>(g, va, vb, s);
  return launch_v<64, 64, 16, TA, TB>(g, va, vb, s);
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

}  // namespace

extern "C" int tile_gemm(void* stream, int transA, int transB, int64_t m, int64_t n, int64_t k, float alpha,
                         const float* A, int64_t lda, const float* B, int64_t ldb, float beta, float* C,
                         int64_t ldc, int epilogue, const float* bias, const float* res, int64_t ldr,
                         float* aux, int64_t ldaux) {
  using tt::fail;
  if (m < 0 || n < 0 || k < 0) return fail(TT_ERR_ARG, "tile_gemm: negative size");
  if (m == 0 || n == 0) return TT_OK;
  if (m > INT32_MAX || n > INT32_MAX || k > INT32_MAX) return fail(TT_ERR_ARG, "tile_gemm: size exceeds int32");
  if (!C || (k > 0 && (!A || !B))) return fail(TT_ERR_ARG, "tile_gemm: null operand");
  if (ldc < n) return fail(TT_ERR_ARG, "tile_gemm: ldc < n");
  if (k > 0 && lda < (transA ? m : k)) return fail(TT_ERR_ARG, "tile_gemm: lda too small");
  if (k > 0 && ldb < (transB ? k : n)) return fail(TT_ERR_ARG, "tile_gemm: ldb too small");
  if (epilogue & ~(TT_EPI_BIAS | TT_EPI_RES | TT_EPI_GELU | TT_EPI_GELU_BWD))
    return fail(TT_ERR_ARG, "tile_gemm: unknown epilogue bits");
  if ((epilogue & TT_EPI_GELU) && (epilogue & TT_EPI_GELU_BWD))
    return fail(TT_ERR_ARG, "tile_gemm: GELU and GELU_BWD are exclusive");
  if ((epilogue & TT_EPI_BIAS) && !bias) return fail(TT_ERR_ARG, "tile_gemm: BIAS without bias");
  if ((epilogue & TT_EPI_RES) && (!res || ldr < n)) return fail(TT_ERR_ARG, "tile_gemm: bad residual");
  if ((epilogue & (TT_EPI_GELU | TT_EPI_GELU_BWD)) && (!aux || ldaux < n))
    return fail(TT_ERR_ARG, "tile_gemm: GELU epilogue needs aux");
  GemmArgs g{(int)m, (int)n, (int)k, alpha, beta, A, B, C, lda, ldb, ldc, epilogue, bias, res, ldr, aux, ldaux};
  if (k == 0) {  // C = beta*S (+epilogue): run the kernel with an empty K loop
    g.k = 0;
  }
  const bool va = k > 0 && aligned16(A) && lda % 4 == 0;
  const bool vb = k > 0 && aligned16(B) && ldb % 4 == 0;
  hipStream_t s = tt::as_stream(stream);
  if (!transA && !transB) return launch_t<false, false>(g, va, vb, s);
  if (!transA && transB) return launch_t<false, true>(g, va, vb, s);
  if (transA && !transB) return launch_t<true, false>(g, va, vb, s);
  return launch_t<true, true>(g, va, vb, s);
}
