// tile_gemm: fp32 GEMM on the CDNA4 matrix cores (v_mfma_f32_32x32x2_f32).
//
// The linear layers and the tied LM head of the GPT2 step are dense
// contractions, so their tile tasks run on MFMA in true fp32 (no xf32/TF32).
//
// Work decomposition (one launch = one tile task):
//   * a workgroup of 256 threads (4 wave64s, 2x2) computes a BM x BN block of
//     C; each wave owns a (BM/2) x (BN/2) sub-block made of 32x32 MFMA tiles
//     whose fp32 accumulators stay in registers for the whole K loop;
//   * K advances in steps of BK (16 or 32, per plan) through two LDS
//     buffers and two register sets: the global loads of step t+2 are
//     issued before step t's MFMAs, step t+1 (loaded a step earlier) is
//     written to the other LDS buffer after them, and one barrier per step
//     suffices; the global latency is covered by two steps of MFMAs;
//   * inside a step the fragments of k group g+1 are requested from LDS
//     before the MFMAs of group g (a scheduling barrier keeps the compiler
//     from sinking them), so LDS latency is paid once per step, not once
//     per group;
//   * blocks whose every load is in range run a branch-free copy of the
//     loop (uniform base pointer + per-thread offsets); edge blocks run the
//     same loop with guarded, zero-filling loads;
//   * each operand is staged in LDS in the orientation it has in HBM, so the
//     global->LDS path is always 16-byte vector loads/stores:
//       K-contiguous operands (A, or B^T)  -> LDS [rows][BK + 4]
//       row-contiguous operands (A^T, B)   -> LDS [BK][rows + 8]
//     (paddings chosen so 16-byte reads of the first and 4-byte reads of
//     the second are free of bank conflicts);
//   * the summation order inside each group of 8 k values is permuted so a
//     lane's 4 consecutive MFMA steps use 4 consecutive k of its half-wave:
//     k = 8*kb + 4*(lane/32) + s. A K-contiguous operand then feeds 4 MFMAs
//     from one 16-byte LDS read;
//   * blockIdx is remapped so consecutive C blocks land on the same XCD
//     (workgroups are dispatched round-robin over the 8 XCDs, each with its
//     own L2), then grouped along M for L2 reuse of the B panel;
//   * split-K: when C has too few blocks to fill 256 CUs and K is long (the
//     weight-gradient GEMMs, K = tokens), S workgroups share a C block, each
//     reducing a K range into its own slice of a workspace; a second kernel
//     adds the slices in slice order and applies the epilogue (deterministic:
//     no atomics). S is picked so the workgroup count sits just under a
//     multiple of the CU count;
//   * block shape by C's shape: 128x128 (BK 16) for large C (the kernel
//     keeps three workgroups per CU), 64x64 (BK 32) for small C.
// Ragged M, N, K are handled by zero-filling out-of-range loads and
// predicating stores; leading dimensions that are not multiples of 4 (or
// unaligned pointers) select a scalar-load instantiation.
#include <cstdlib>
#include <type_traits>
#include <vector>

#include "common.hpp"

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kSplitAlign = 32;  // split-K chunks are multiples of every BK used
constexpr int64_t kCUs = 256;    // MI355X compute units (8 XCDs x 32)

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
  float* ws;       // split-K partials [splits][m][n], or null
  int splits;      // K ranges (1 = no split)
  int kchunk;      // K per split (multiple of kSplitAlign)
  // TT_EPI_XSTATS (128x128 blocks, no split): per row and 64-column group of
  // C, (max, sum exp(x - max), x at the row's label) -> xparts[(group * m +
  // row) * 3 ..]; the label's column is xlab[row] - xvoff
  const int32_t* xlab;
  float* xparts;
  int64_t xvoff;
  int64_t xstride;  // batched: floats between the partials of consecutive products
  int64_t xvtile;   // batched: vocab offset step between consecutive products
};

// tanh(a) = 1 - 2 / (exp(2a) + 1), on the hardware exp2 and reciprocal
// (each within about an ulp, so the result is within a few 1e-7 of tanh,
// absolutely). exp2 overflows to inf or underflows to 0 for large |a|,
// which gives exactly +1 or -1. Far fewer instructions than tanhf: the
// GELU epilogues of the MLP's 4096 x 3072 GEMMs run in every block at the
// same moment, with the matrix cores idle.
__device__ __forceinline__ float tanh_fast(float a) {
  const float e = __builtin_amdgcn_exp2f(a * 2.8853900817779268f);  // 2 / ln 2
  return 1.f - 2.f * __builtin_amdgcn_rcpf(e + 1.f);
}

__device__ __forceinline__ float gelu_tanh(float u) {
  const float c = 0.7978845608028654f;  // sqrt(2/pi)
  float a = c * (u + 0.044715f * u * u * u);
  return 0.5f * u * (1.f + tanh_fast(a));
}

__device__ __forceinline__ float gelu_tanh_grad(float u) {
  const float c = 0.7978845608028654f;
  float a = c * (u + 0.044715f * u * u * u);
  float t = tanh_fast(a);
  return 0.5f * (1.f + t) + 0.5f * u * (1.f - t * t) * c * (1.f + 3.f * 0.044715f * u * u);
}

// acc (already alpha-scaled) -> C, with beta source, bias, residual, GELU;
// returns the value stored
__device__ __forceinline__ float epilogue_store(const GemmArgs& g, int row, int col, float v) {
  const bool gelu = g.epi & TT_EPI_GELU;
  if (g.beta != 0.f)
    v += g.beta * (gelu ? g.aux[(int64_t)row * g.ldaux + col] : g.C[(int64_t)row * g.ldc + col]);
  if (g.epi & TT_EPI_BIAS) v += g.bias[col];
  if (g.epi & TT_EPI_RES) v += g.res[(int64_t)row * g.ldr + col];
  if (gelu) {
    g.aux[(int64_t)row * g.ldaux + col] = v;
    v = gelu_tanh(v);
  } else if (g.epi & TT_EPI_GELU_BWD) {
    v *= gelu_tanh_grad(g.aux[(int64_t)row * g.ldaux + col]);
  }
  g.C[(int64_t)row * g.ldc + col] = v;
  return v;
}

// float4 of an operand at (r, c) of a `rows` x `cols` row-major matrix with
// leading dimension ld; zero outside.
template <bool VEC>
__device__ __forceinline__ f32x4 load4(const float* __restrict__ p, int64_t ld, int r, int c, int rows, int cols) {
  f32x4 v = {0.f, 0.f, 0.f, 0.f};
  if (r >= rows) return v;
  const float* q = p + (int64_t)r * ld + c;
  if (VEC && c + 3 < cols) return *reinterpret_cast<const f32x4*>(q);
#pragma unroll
  for (int i = 0; i < 4; ++i)
    if (c + i < cols) v[i] = q[i];
  return v;
}

// Thread -> (row, k) of a K-contiguous operand block [rows][BK]: float4
// `idx` covers k = c..c+3 of row r. With BK = 32 eight consecutive threads
// take one row (LDS row stride 36 floats: the 8 float4 of a store cycle hit
// distinct banks). With BK = 16 the row stride is 20 floats, and two rows'
// float4s would share banks within a cycle, so 16 consecutive threads take
// 16 different rows at the same k: rows r and r' then differ by 5(r - r')
// float4 units, distinct modulo 8 for 8 consecutive rows. Either way a wave
// fetches the same bytes per load instruction.
template <int BK>
__device__ __forceinline__ void kc_index(int idx, int* r, int* c) {
  if (BK == 16) {
    *r = (idx >> 6) * 16 + (idx & 15);
    *c = ((idx >> 4) & 3) * 4;
  } else {
    *r = idx / (BK / 4);
    *c = (idx % (BK / 4)) * 4;
  }
}

// LDS floats of one gemm_block configuration (two stages of A and B)
template <int BM, int BN, int BK, bool TA, bool TB>
struct GemmLds {
  static constexpr int A_LD = !TA ? BK + 4 : BM + 8;
  static constexpr int B_LD = TB ? BK + 4 : BN + 8;
  static constexpr int A_SZ = !TA ? BM * A_LD : BK * A_LD;
  static constexpr int B_SZ = TB ? BN * B_LD : BK * B_LD;
  static constexpr int FLOATS = 2 * (A_SZ + B_SZ);
};

// Workgroups are dispatched round-robin over the 8 XCDs: linear index b ->
// a block index such that consecutive blocks run on the same XCD (its L2
// then serves their shared operand panels).
__device__ __forceinline__ int xcd_contiguous(int b, int nb) {
  const int per = nb / 8, rem = nb % 8, x = b % 8;
  return x * per + min(x, rem) + b / 8;
}

// One BM x BN block of C (K range `split` of g.splits): block index b, after
// the XCD remap, over the ntile * splits blocks of this product.
template <int BM, int BN, int BK, bool TA, bool TB, bool VA, bool VB, bool SPLIT>
__device__ __forceinline__ void gemm_block(const GemmArgs& g, int b, float* lds) {
  constexpr int WM = BM / 2, WN = BN / 2;      // wave sub-block
  constexpr int FM = WM / 32, FN = WN / 32;    // 32x32 MFMA tiles per wave
  constexpr int A_KC = !TA, B_KC = TB;
  using LL = GemmLds<BM, BN, BK, TA, TB>;
  constexpr int A_LD = LL::A_LD, B_LD = LL::B_LD, A_SZ = LL::A_SZ, B_SZ = LL::B_SZ;
  constexpr int A_V4 = BM * BK / 4, B_V4 = BN * BK / 4;
  constexpr int A_PT = A_V4 / 256, B_PT = B_V4 / 256;
  static_assert(A_V4 % 256 == 0 && B_V4 % 256 == 0, "tile must split evenly over 256 threads");

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int half = lane >> 5, l32 = lane & 31;

  // ---- block -> (C tile, K range): grouped along M
  const int grid_m = (g.m + BM - 1) / BM, grid_n = (g.n + BN - 1) / BN;
  const int ntile = grid_m * grid_n;
  const int split = b / ntile;
  b -= split * ntile;
  constexpr int GROUP = 8;
  int tm, tn;
  if (TA) {
    // A stored [k][m] (the weight gradients: A = an activation or logits
    // tile read down its columns): grouped along N, so the blocks that share
    // an A panel run side by side and find it in L2 (25 products 2048 x
    // 2048 x 4096: 80.9 -> 81.8 % of the fp32 peak; 16 products 8192 x 2048
    // x 4096: 84.5 -> 85.2 %)
    const int in_group = GROUP * grid_m;
    const int first_n = (b / in_group) * GROUP;
    const int gsz = min(grid_n - first_n, GROUP);
    tn = first_n + (b % in_group) % gsz;
    tm = (b % in_group) / gsz;
  } else {
    const int in_group = GROUP * grid_n;
    const int first_m = (b / in_group) * GROUP;
    const int gsz = min(grid_m - first_m, GROUP);
    tm = first_m + (b % in_group) % gsz;
    tn = (b % in_group) / gsz;
  }
  const int m0 = tm * BM, n0 = tn * BN;
  const int kbeg = split * g.kchunk;
  const int kend = min(g.k, kbeg + g.kchunk);

  const int nk = kend > kbeg ? (kend - kbeg + BK - 1) / BK : 0;
  // Interior blocks (every load of every K step in range and 16-byte
  // loadable) run a branch-free copy of the loop; edge blocks a guarded one.
  const bool fast = VA && VB && m0 + BM <= g.m && n0 + BN <= g.n && (kend - kbeg) % BK == 0 &&
                    (int64_t)BM * g.lda < INT32_MAX && (int64_t)BN * g.ldb < INT32_MAX;

  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  auto run = [&](auto guard_tag) {
    constexpr bool G = decltype(guard_tag)::value;
    // Two register sets of staged operands: the global loads of step t+2
    // are in flight while step t is multiplied and step t+1 is written to LDS.
    f32x4 ra0[A_PT], rb0[B_PT], ra1[A_PT], rb1[B_PT];
    // fast path: per-thread element offsets inside a K step (32-bit; the
    // step's base pointer is uniform)
    int oa[A_PT], ob[B_PT];
#pragma unroll
    for (int i = 0; i < A_PT; ++i) {
      const int idx = tid + 256 * i;
      int r = idx / (BM / 4), c = (idx % (BM / 4)) * 4;
      if (A_KC) kc_index<BK>(idx, &r, &c);
      oa[i] = r * (int)g.lda + c;
    }
#pragma unroll
    for (int i = 0; i < B_PT; ++i) {
      const int idx = tid + 256 * i;
      int r = idx / (BN / 4), c = (idx % (BN / 4)) * 4;
      if (B_KC) kc_index<BK>(idx, &r, &c);
      ob[i] = r * (int)g.ldb + c;
    }
    // K step `st` -> registers. st is clamped to the last step, so every
    // call issues the same loads (the compiler's wait counts stay exact);
    // the repeated loads of the last step are never stored.
    auto gload = [&](int st, f32x4(&ra)[A_PT], f32x4(&rb)[B_PT]) {
      const int k0 = kbeg + min(st, nk - 1) * BK;
      if constexpr (!G) {
        const float* pa = A_KC ? g.A + (int64_t)m0 * g.lda + k0 : g.A + (int64_t)k0 * g.lda + m0;
        const float* pb = B_KC ? g.B + (int64_t)n0 * g.ldb + k0 : g.B + (int64_t)k0 * g.ldb + n0;
#pragma unroll
        for (int i = 0; i < A_PT; ++i) ra[i] = *reinterpret_cast<const f32x4*>(pa + oa[i]);
#pragma unroll
        for (int i = 0; i < B_PT; ++i) rb[i] = *reinterpret_cast<const f32x4*>(pb + ob[i]);
      } else {
#pragma unroll
        for (int i = 0; i < A_PT; ++i) {
          const int idx = tid + 256 * i;
          int r = idx / (BM / 4), c = (idx % (BM / 4)) * 4;
          if (A_KC) {
            kc_index<BK>(idx, &r, &c);
            ra[i] = load4<VA>(g.A, g.lda, m0 + r, k0 + c, g.m, kend);
          } else {
            ra[i] = load4<VA>(g.A, g.lda, k0 + r, m0 + c, kend, g.m);
          }
        }
#pragma unroll
        for (int i = 0; i < B_PT; ++i) {
          const int idx = tid + 256 * i;
          int r = idx / (BN / 4), c = (idx % (BN / 4)) * 4;
          if (B_KC) {
            kc_index<BK>(idx, &r, &c);
            rb[i] = load4<VB>(g.B, g.ldb, n0 + r, k0 + c, g.n, kend);
          } else {
            rb[i] = load4<VB>(g.B, g.ldb, k0 + r, n0 + c, kend, g.n);
          }
        }
      }
    };
    auto sstore = [&](int buf, const f32x4(&ra)[A_PT], const f32x4(&rb)[B_PT]) {
      float* As = lds + buf * (A_SZ + B_SZ);
      float* Bs = As + A_SZ;
#pragma unroll
      for (int i = 0; i < A_PT; ++i) {
        const int idx = tid + 256 * i;
        int r = idx / (BM / 4), c = (idx % (BM / 4)) * 4;
        if (A_KC) kc_index<BK>(idx, &r, &c);
        *reinterpret_cast<f32x4*>(As + r * A_LD + c) = ra[i];
      }
#pragma unroll
      for (int i = 0; i < B_PT; ++i) {
        const int idx = tid + 256 * i;
        int r = idx / (BN / 4), c = (idx % (BN / 4)) * 4;
        if (B_KC) kc_index<BK>(idx, &r, &c);
        *reinterpret_cast<f32x4*>(Bs + r * B_LD + c) = rb[i];
      }
    };
    // fragments of k group kb (8 k values) of LDS buffer `buf`
    auto frag = [&](int buf, int kb, f32x4(&fa)[FM], f32x4(&fb)[FN]) {
      const float* As = lds + buf * (A_SZ + B_SZ);
      const float* Bs = As + A_SZ;
      const int kk = kb * 8 + half * 4;
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
    };
    auto mfmas = [&](const f32x4(&fa)[FM], const f32x4(&fb)[FN]) {
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(fa[i][s], fb[j][s], acc[i][j], 0, 0, 0);
    };
    // One K step from LDS buffer `buf`, software-pipelined by k group: the
    // fragments of group kb+1 are requested before the MFMAs of group kb
    // are issued (the scheduling barrier keeps the compiler from sinking
    // the reads next to their use, which would expose an LDS latency per
    // group).
    auto compute = [&](int buf) {
      f32x4 fa0[FM], fb0[FN], fa1[FM], fb1[FN];
      frag(buf, 0, fa0, fb0);
#pragma unroll
      for (int kb = 0; kb < BK / 8; ++kb) {
        if (kb + 1 < BK / 8) {
          if (kb & 1) frag(buf, kb + 1, fa0, fb0);
          else frag(buf, kb + 1, fa1, fb1);
        }
        __builtin_amdgcn_sched_barrier(0);
        if (kb & 1) mfmas(fa1, fb1);
        else mfmas(fa0, fb0);
      }
    };

    if (nk == 0) return;
    gload(0, ra0, rb0);
    gload(1, ra1, rb1);
    sstore(0, ra0, rb0);
    __syncthreads();
    // steps t (even) use LDS buffer 0 and register set 0, odd ones buffer 1
    // and set 1; a set is reloaded (step t+2) as soon as step t is in LDS.
    // The loop body has no early exit (an odd last step runs after it), so
    // the accumulators keep one register assignment throughout.
    int kt = 0;
    for (; kt + 1 < nk; kt += 2) {
      gload(kt + 2, ra0, rb0);
      compute(0);
      sstore(1, ra1, rb1);
      __syncthreads();
      gload(kt + 3, ra1, rb1);
      compute(1);
      if (kt + 2 < nk) sstore(0, ra0, rb0);
      __syncthreads();
    }
    if (kt < nk) compute(0);
  };
  if (fast) run(std::false_type{});
  else run(std::true_type{});

  // ---- epilogue: accumulator register r of lane l holds
  //      row 8*(r/4) + 4*(l/32) + (r%4), column l%32 of its 32x32 tile
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int col = n0 + wn * WN + j * 32 + l32;
      if (col >= g.n) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = m0 + wm * WM + i * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
        if (row >= g.m) continue;
        if (SPLIT)
          g.ws[((int64_t)split * g.m + row) * g.n + col] = acc[i][j][r];
        else
          acc[i][j][r] = epilogue_store(g, row, col, g.alpha * acc[i][j][r]);
      }
    }
  // ---- cross-entropy statistics of the stored values: each wave's 64
  // columns are one group. The wave's 64 x 64 values go through LDS (the
  // staging buffers, free once every wave is past its last K step) so that
  // lane l owns row l of the tile: it takes (max, sum exp(x - max), x at the
  // row's label) over the group's columns inside C in column order and
  // writes them, 64 lanes to 64 consecutive rows
  // (128x128x32 blocks: the plan tile_gemm_batch_xstats always launches)
  constexpr int XLD = 65;  // row stride: lane l reads row l, consecutive lanes hit consecutive banks
  if constexpr (!SPLIT && WN == 64 && LL::FLOATS >= 4 * 64 * XLD) {
    if (g.epi & TT_EPI_XSTATS) {
      __syncthreads();
      float* xs = lds + wave * 64 * XLD;
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r) xs[(i * 32 + 8 * (r >> 2) + 4 * half + (r & 3)) * XLD + j * 32 + l32] = acc[i][j][r];
      __syncthreads();
      const int c0 = n0 + wn * WN, row = m0 + wm * WM + lane;
      if (c0 < g.n && row < g.m) {
        const float* rp = xs + lane * XLD;
        const int ncol = min(64, g.n - c0);
        const int64_t lab = (int64_t)g.xlab[row] - g.xvoff - c0;
        float mx = -INFINITY;
        for (int c = 0; c < ncol; ++c) mx = fmaxf(mx, rp[c]);
        float se = 0.f;
        for (int c = 0; c < ncol; ++c) se += __builtin_amdgcn_exp2f((rp[c] - mx) * 1.4426950408889634f);
        float* q = g.xparts + ((int64_t)(c0 / 64) * g.m + row) * 3;
        q[0] = mx;
        q[1] = se;
        q[2] = (lab >= 0 && lab < ncol) ? rp[lab] : 0.f;
      }
    }
  }
}

template <int BM, int BN, int BK, bool TA, bool TB, bool VA, bool VB, bool SPLIT>
__global__ __launch_bounds__(256, 2) void gemm_kernel(GemmArgs g) {
  __shared__ __attribute__((aligned(16))) float lds[GemmLds<BM, BN, BK, TA, TB>::FLOATS];
  const int nb = ((g.m + BM - 1) / BM) * ((g.n + BN - 1) / BN) * g.splits;
  gemm_block<BM, BN, BK, TA, TB, VA, VB, SPLIT>(g, xcd_contiguous(blockIdx.x, nb), lds);
}

// ---- batch: C_t = alpha * op(A_t) op(B_t) + beta * C_t for a list of
// independent products that share transposes, K and the scalars, each with
// its own m, n and leading dimensions (the LM head: one product per vocab
// tile, the last one ragged), in one launch. The blocks of all products
// form one grid, remapped XCD-contiguously, so each XCD works through a
// contiguous run of products and keeps their operand panels in its L2;
// each operand of each product loads 16 bytes at a time where its leading
// dimension and alignment allow, else 4 (chosen per product and operand).
constexpr int kBatchMax = 72;  // products per launch (kernel arguments stay under 4 KB)
struct GemmBatch {
  const float* A[kBatchMax];
  const float* B[kBatchMax];
  float* C[kBatchMax];
  int m[kBatchMax], n[kBatchMax];
  int lda[kBatchMax], ldb[kBatchMax], ldc[kBatchMax];
  int first[kBatchMax];                       // first block of each product
  unsigned va[(kBatchMax + 31) / 32];         // bit t: product t loads A 16 bytes at a time
  unsigned vb[(kBatchMax + 31) / 32];         // bit t: product t loads B 16 bytes at a time
  short orig[kBatchMax];                      // position of product t in the caller's list
  int count;
};
static_assert(sizeof(GemmArgs) + sizeof(GemmBatch) <= 4096, "kernel arguments over 4 KB");

// With split-K (g.splits > 1) every product's blocks come in g.splits K
// ranges; the partial sums of product t go to the workspace region that
// starts at its first block times BM * BN floats (a region of (blocks of t)
// x BM x BN floats holds its splits x m x n partials), and
// gemm_batch_finish adds them in slice order.
template <int BM, int BN, int BK, bool TA, bool TB, bool SPLIT>
__global__ __launch_bounds__(256, 2) void gemm_batch_kernel(GemmArgs g, GemmBatch P) {
  __shared__ __attribute__((aligned(16))) float lds[GemmLds<BM, BN, BK, TA, TB>::FLOATS];
  const int b = xcd_contiguous(blockIdx.x, gridDim.x);
  int t = 0;  // the product owning block b (uniform)
  while (t + 1 < P.count && P.first[t + 1] <= b) ++t;
  GemmArgs h = g;
  h.m = P.m[t];
  h.n = P.n[t];
  h.A = P.A[t];
  h.B = P.B[t];
  h.C = P.C[t];
  h.lda = P.lda[t];
  h.ldb = P.ldb[t];
  h.ldc = P.ldc[t];
  if (SPLIT) h.ws = g.ws + (int64_t)P.first[t] * (BM * BN);
  if (g.epi & TT_EPI_XSTATS) {  // product o of the call: its partials region and vocab offset
    const int o = P.orig[t];
    h.xparts = g.xparts + (int64_t)o * g.xstride;
    h.xvoff = g.xvoff + (int64_t)o * g.xvtile;
  }
  const bool va = (P.va[t >> 5] >> (t & 31)) & 1u, vb = (P.vb[t >> 5] >> (t & 31)) & 1u;
  const int lb = b - P.first[t];
  if (va && vb) gemm_block<BM, BN, BK, TA, TB, true, true, SPLIT>(h, lb, lds);
  else if (vb) gemm_block<BM, BN, BK, TA, TB, false, true, SPLIT>(h, lb, lds);
  else if (va) gemm_block<BM, BN, BK, TA, TB, true, false, SPLIT>(h, lb, lds);
  else gemm_block<BM, BN, BK, TA, TB, false, false, SPLIT>(h, lb, lds);
}

// split-K finish of every product of a batch launch (blockIdx.y = product)
template <int BM, int BN, int VEC>
__global__ __launch_bounds__(256) void gemm_batch_finish(GemmArgs g, GemmBatch P) {
  const int t = blockIdx.y;
  GemmArgs h = g;
  h.m = P.m[t];
  h.n = P.n[t];
  h.C = P.C[t];
  h.ldc = P.ldc[t];
  h.ws = g.ws + (int64_t)P.first[t] * (BM * BN);
  split_finish<VEC>(h);
}

// Sum of the split-K slices in slice order, then the epilogue.
// Each thread sums VEC consecutive elements; the loads of up to 8 slices are
// issued together, the additions stay in slice order.
template <int VEC>
__device__ __forceinline__ void split_finish(const GemmArgs& g) {
  using V = typename std::conditional<VEC == 4, f32x4, float>::type;
  const int64_t i = (blockIdx.x * (int64_t)blockDim.x + threadIdx.x) * VEC;
  const int64_t mn = (int64_t)g.m * g.n;
  if (i >= mn) return;
  const V* w = reinterpret_cast<const V*>(g.ws + i);
  const int64_t stride = mn / VEC;
  V s = {};
  int z = 0;
  for (; z + 8 <= g.splits; z += 8) {
    V v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = w[(z + u) * stride];
#pragma unroll
    for (int u = 0; u < 8; ++u) s += v[u];
  }
  for (; z < g.splits; ++z) s += w[z * stride];
  if constexpr (VEC == 4) {
#pragma unroll
    for (int e = 0; e < 4; ++e) epilogue_store(g, (int)((i + e) / g.n), (int)((i + e) % g.n), g.alpha * s[e]);
  } else {
    epilogue_store(g, (int)(i / g.n), (int)(i % g.n), g.alpha * s);
  }
}

template <int VEC>
__global__ __launch_bounds__(256) void gemm_split_finish(GemmArgs g) {
  split_finish<VEC>(g);
}

template <int BM, int BN, int BK, bool TA, bool TB, bool SPLIT>
void launch_v(const GemmArgs& g, bool va, bool vb, hipStream_t s) {
  const int nb = ((g.m + BM - 1) / BM) * ((g.n + BN - 1) / BN) * g.splits;
  dim3 grid(nb), block(256);
  if (va && vb) hipLaunchKernelGGL((gemm_kernel<BM, BN, BK, TA, TB, true, true, SPLIT>), grid, block, 0, s, g);
  else if (va) hipLaunchKernelGGL((gemm_kernel<BM, BN, BK, TA, TB, true, false, SPLIT>), grid, block, 0, s, g);
  else if (vb) hipLaunchKernelGGL((gemm_kernel<BM, BN, BK, TA, TB, false, true, SPLIT>), grid, block, 0, s, g);
  else hipLaunchKernelGGL((gemm_kernel<BM, BN, BK, TA, TB, false, false, SPLIT>), grid, block, 0, s, g);
}

struct Plan {
  int bm, bn, bk, splits, kchunk;
};

// Tuning override "bm,bn,bk,splits" (e.g. "128,128,16,1") read once from
// TT_GEMM_PLAN; only configurations this file instantiates are accepted.
bool plan_override(Plan* p, int64_t k) {
  static int parsed = 0;
  static Plan forced{0, 0, 0, 1, 0};
  if (!parsed) {
    parsed = -1;
    if (const char* e = getenv("TT_GEMM_PLAN")) {
      Plan q{0, 0, 0, 1, 0};
      if (sscanf(e, "%d,%d,%d,%d", &q.bm, &q.bn, &q.bk, &q.splits) == 4 && (q.bk == 16 || q.bk == 32) &&
          q.splits >= 1 && ((q.bm == 128 && (q.bn == 128 || q.bn == 64)) || (q.bm == 64 && q.bn == 64))) {
        forced = q;
        parsed = 1;
      }
    }
  }
  if (parsed != 1) return false;
  *p = forced;
  int64_t chunk = (k + p->splits - 1) / p->splits;
  chunk = (chunk + kSplitAlign - 1) / kSplitAlign * kSplitAlign;
  p->kchunk = (int)std::max<int64_t>(chunk, kSplitAlign);
  p->splits = (int)std::max<int64_t>(1, (k + p->kchunk - 1) / p->kchunk);
  if (p->splits == 1) p->kchunk = (int)k;
  return true;
}

// Whether b128 (>= 512) blocks of 128x128 keep that tile rather than 64x64.
// A launch lasts as long as its busiest CU, and with b128 blocks over kCUs
// CUs the last round is partly idle; 64x64 blocks (four times as many) fill
// their rounds nearly evenly but reuse each loaded element half as often.
// Measured on MI355X (tile_gemm, A [m][k], B [k][n]): at full rounds 64x64
// reaches 0.97-0.99 of 128x128's rate for K = 768 and 0.88 for K = 2048 to
// 8192 (a short K leaves the larger tile's per-block costs less amortised),
// so 128x128 stays while its rounds are at least that full: 4096 x 2304 x 768
// (576 blocks, rounds 75 % full) runs at 99 TFLOP/s on 64x64 against 79,
// 8192 x 2304 x 768 (1152, 90 %) at 113 against 105, 4096 x 2304 x 3072 at
// 112 against 91-97, while 4096 x 2048 x 8192 (512, full) keeps 124-127 on
// 128x128 against 112.
bool rounds_favour_128(int64_t b128, int64_t k) {
  const int64_t rounds = (b128 + kCUs - 1) / kCUs;
  const double fill = (double)b128 / (double)(rounds * kCUs);
  return fill >= (k <= 1024 ? 0.97 : 0.88);
}

// Block shape and split count: fill at least ~2 workgroups per CU.
Plan plan_for(int64_t m, int64_t n, int64_t k, size_t ws_bytes) {
  const int64_t want = 512;
  auto blocks = [&](int bm, int bn) { return ((m + bm - 1) / bm) * ((n + bn - 1) / bn); };
  // Choices measured per tile-op class on MI355X (isolated launches): 128x128
  // with BK 16 when it gives >= 2 blocks per CU and the blocks split evenly
  // over the CUs; split-K only when C is small (<= 144 such blocks) and K
  // long; otherwise 64x64 blocks, whose larger block count beats the bigger
  // tile's reuse at these sizes.
  Plan p{128, 128, 16, 1, (int)k};
  if (plan_override(&p, k)) {
    // an override never splits without the workspace the split needs
    if (p.splits > 1 && (size_t)p.splits * m * n * sizeof(float) > ws_bytes) {
      p.splits = 1;
      p.kchunk = (int)k;
    }
    return p;
  }
  const int64_t b128 = blocks(128, 128);
  if (b128 >= want) {
    if (!rounds_favour_128(b128, k)) return Plan{64, 64, 32, 1, (int)k};
    // BK 16 keeps three workgroups per CU, BK 32 two: a block count that is
    // a multiple of 512 fills whole rounds of two, and there BK 32 wins
    // (the wide model's MLP output chain links, 4096 x 2048 x 8192: 84.0 ->
    // 85.1 % of the fp32 peak in the step, the step 697.0 -> 695.3 ms;
    // 4096 x 2048 x 768: 101 -> 104 TFLOP/s), while 768 blocks fill one
    // round of three (4096 x 3072 x 768: 103 TFLOP/s at BK 16, 87 at BK 32)
    if (b128 % 512 == 0) p.bk = 32;
    return p;
  }
  if (k >= 2048 && b128 <= 144 && ws_bytes > 0) {
    // split count by CU balance: workgroups run in rounds of one per CU, so
    // b128*s just under a multiple of 256 keeps every CU equally loaded
    // (measured: 36 tiles x 7 beats x 8 by 1.3x, 144 tiles x 7 beats x 4)
    int best_s = 1;
    int64_t best_chunk = k;
    double best_bal = 0.0;
    for (int s = 2; s <= 8; ++s) {
      int64_t chunk = (k + s - 1) / s;
      chunk = (chunk + kSplitAlign - 1) / kSplitAlign * kSplitAlign;
      const int64_t sa = (k + chunk - 1) / chunk;
      if (chunk < 256 || (size_t)sa * m * n * sizeof(float) > ws_bytes) continue;
      const int64_t nwg = b128 * sa;
      const double bal = (double)nwg / (double)(((nwg + kCUs - 1) / kCUs) * kCUs);
      if (bal > best_bal + 0.01) {
        best_bal = bal;
        best_s = (int)sa;
        best_chunk = chunk;
      }
    }
    if (best_s > 1) return Plan{128, 128, 32, best_s, (int)best_chunk};
  }
  // small tiles (the small-tile workload's GEMMs, e.g. 512 x 512 x 1024 or
  // 1024 x 512 x 512): fewer 64x64 blocks than CUs and a K of at least 512
  // -> split over 64x64 blocks by the same balance rule
  const int64_t b64 = blocks(64, 64);
  if (k >= 512 && b64 < kCUs && ws_bytes > 0) {
    int best_s = 1;
    int64_t best_chunk = k;
    double best_bal = (double)b64 / (double)kCUs;
    for (int s = 2; s <= 8; ++s) {
      int64_t chunk = (k + s - 1) / s;
      chunk = (chunk + kSplitAlign - 1) / kSplitAlign * kSplitAlign;
      const int64_t sa = (k + chunk - 1) / chunk;
      if (chunk < 128 || (size_t)sa * m * n * sizeof(float) > ws_bytes) continue;
      const int64_t nwg = b64 * sa;
      const double bal = (double)nwg / (double)(((nwg + kCUs - 1) / kCUs) * kCUs);
      if (bal > best_bal + 0.01) {
        best_bal = bal;
        best_s = (int)sa;
        best_chunk = chunk;
      }
    }
    if (best_s > 1) return Plan{64, 64, 32, best_s, (int)best_chunk};
  }
  return Plan{64, 64, 32, 1, (int)k};
}

template <bool TA, bool TB>
int launch_t(GemmArgs g, bool va, bool vb, size_t ws_bytes, hipStream_t s) {
  const Plan p = plan_for(g.m, g.n, g.k, ws_bytes);
  g.splits = p.splits;
  g.kchunk = p.kchunk;
  if (p.splits > 1) {
    if (p.bk == 16) {
      if (p.bm == 128 && p.bn == 128) launch_v<128, 128, 16, TA, TB, true>(g, va, vb, s);
      else if (p.bm == 128) launch_v<128, 64, 16, TA, TB, true>(g, va, vb, s);
      else launch_v<64, 64, 16, TA, TB, true>(g, va, vb, s);
    } else {
      if (p.bm == 128 && p.bn == 128) launch_v<128, 128, 32, TA, TB, true>(g, va, vb, s);
      else if (p.bm == 128) launch_v<128, 64, 32, TA, TB, true>(g, va, vb, s);
      else launch_v<64, 64, 32, TA, TB, true>(g, va, vb, s);
    }
    if (int rc = tt::launch_status("tile_gemm(split)")) return rc;
    const int64_t mn = (int64_t)g.m * g.n;
    // the workspace comes from hipMalloc (256-byte aligned) and each slice
    // plane starts at a multiple of mn floats
    if (mn % 4 == 0 && (reinterpret_cast<uintptr_t>(g.ws) & 15) == 0)
      hipLaunchKernelGGL(gemm_split_finish<4>, dim3((unsigned)((mn / 4 + 255) / 256)), dim3(256), 0, s, g);
    else
      hipLaunchKernelGGL(gemm_split_finish<1>, dim3((unsigned)((mn + 255) / 256)), dim3(256), 0, s, g);
    return tt::launch_status("tile_gemm(split finish)");
  }
  if (p.bk == 16) {
    if (p.bm == 128 && p.bn == 128) launch_v<128, 128, 16, TA, TB, false>(g, va, vb, s);
    else if (p.bm == 128) launch_v<128, 64, 16, TA, TB, false>(g, va, vb, s);
    else launch_v<64, 64, 16, TA, TB, false>(g, va, vb, s);
  } else {
    if (p.bm == 128 && p.bn == 128) launch_v<128, 128, 32, TA, TB, false>(g, va, vb, s);
    else if (p.bm == 128) launch_v<128, 64, 32, TA, TB, false>(g, va, vb, s);
    else launch_v<64, 64, 32, TA, TB, false>(g, va, vb, s);
  }
  return tt::launch_status("tile_gemm");
}


// ---- K-sum: C = alpha * sum_t A_t B_t + beta * C (both operands in HBM
// orientation: A_t [m][k_t], B_t [k_t][n]) in one launch over a list of
// tile pairs that share m, n and the leading dimensions, every k_t a
// multiple of BK and every load 16-byte aligned and in range. The LM head's
// input gradient is such a sum, one product per vocab tile; one launch
// replaces a chain of accumulating GEMMs (each of which reads and writes C)
// by one long K loop. Same main loop as gemm_kernel's fast path; the sum
// runs over the pairs in list order.
constexpr int kKsumMax = 96;  // pairs per launch (kernel arguments stay under 4 KB)
struct KsumPair {
  const float* A;
  const float* B;
  int64_t steps;  // k_t / BK
};
struct KsumArgs {
  int m, n, nk;  // nk = total K steps over the pairs
  float alpha, beta;
  float* C;
  int64_t lda, ldb, ldc;
  int epi;             // epilogue of tile_gemm applied to the whole sum
  const float* bias;
  const float* res;
  int64_t ldr;
  float* aux;
  int64_t ldaux;
  float* ws;   // split-K partial sums (SPLIT): splits x m x n, slice-major
  int chunk;   // K steps per slice (SPLIT)
  KsumPair t[kKsumMax];
};
static_assert(sizeof(KsumArgs) <= 4096, "kernel arguments over 4 KB");

// TB: B_t is stored [n][k_t] (B_t^T in HBM, K-contiguous, the linear
// layers' input gradients dX = sum_t dY_t W_t^T) instead of [k_t][n].
// SPLIT: the grid holds nb x splits blocks; slice z sums the K steps
// [z * chunk, (z + 1) * chunk) of the concatenated pair list into its own
// m x n region of P.ws (no epilogue); gemm_split_finish adds the slices in
// slice order and applies alpha, beta and the epilogue.
// 256 x 256 blocks (each wave 128 x 128, 256 accumulators per lane) run one
// workgroup per CU and may use every register of a SIMD
template <int BM, int BN, int BK, bool TB, bool SPLIT>
__global__ __launch_bounds__(256, (BM * BN >= 256 * 256) ? 1 : 2) void gemm_ksum_kernel(KsumArgs P) {
  constexpr int WM = BM / 2, WN = BN / 2;
  constexpr int FM = WM / 32, FN = WN / 32;
  constexpr int A_LD = BK + 4, B_LD = TB ? BK + 4 : BN + 8;  // A K-contiguous; B either way
  constexpr int A_SZ = BM * A_LD, B_SZ = TB ? BN * B_LD : BK * B_LD;
  constexpr int A_PT = BM * BK / 4 / 256, B_PT = BN * BK / 4 / 256;
  static_assert(A_PT * 256 * 4 == BM * BK && B_PT * 256 * 4 == BN * BK, "tile must split evenly over 256 threads");
  __shared__ __attribute__((aligned(16))) float lds[2 * (A_SZ + B_SZ)];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int half = lane >> 5, l32 = lane & 31;

  // block -> C tile: XCD-contiguous, then grouped along M (as gemm_kernel)
  const int grid_m = P.m / BM, grid_n = P.n / BN;
  const int nb = grid_m * grid_n;
  int b = blockIdx.x;
  {
    const int tot = (int)gridDim.x;  // nb, or nb x splits
    const int per = tot / 8, rem = tot % 8, x = b % 8;
    b = x * per + min(x, rem) + b / 8;
  }
  int split = 0;
  if (SPLIT) {  // consecutive blocks on an XCD: one slice, neighbouring C tiles
    split = b / nb;
    b -= split * nb;
  }
  constexpr int GROUP = 8;
  const int in_group = GROUP * grid_n;
  const int first_m = (b / in_group) * GROUP;
  const int gsz = min(grid_m - first_m, GROUP);
  const int tm = first_m + (b % in_group) % gsz;
  const int tn = (b % in_group) / gsz;
  const int m0 = tm * BM, n0 = tn * BN;
  const int kbeg = SPLIT ? split * P.chunk : 0;
  const int nk = SPLIT ? min(P.nk - kbeg, P.chunk) : P.nk;  // steps of this block

  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  int oa[A_PT], ob[B_PT];
#pragma unroll
  for (int i = 0; i < A_PT; ++i) {
    int r, c;
    kc_index<BK>(tid + 256 * i, &r, &c);
    oa[i] = r * (int)P.lda + c;
  }
#pragma unroll
  for (int i = 0; i < B_PT; ++i) {
    const int idx = tid + 256 * i;
    if (TB) {
      int r, c;
      kc_index<BK>(idx, &r, &c);
      ob[i] = r * (int)P.ldb + c;
    } else {
      ob[i] = (idx / (BN / 4)) * (int)P.ldb + (idx % (BN / 4)) * 4;
    }
  }
  // step -> pair: the steps are requested in non-decreasing order, so a
  // cursor walks the list (uniform, scalar)
  int cur = 0;
  int64_t before = 0;
  f32x4 ra0[A_PT], rb0[B_PT], ra1[A_PT], rb1[B_PT];
  auto gload = [&](int st, f32x4(&ra)[A_PT], f32x4(&rb)[B_PT]) {
    st = kbeg + min(st, nk - 1);
    while (st >= before + P.t[cur].steps) before += P.t[cur++].steps;
    const int k0 = (int)(st - before) * BK;
    const float* pa = P.t[cur].A + (int64_t)m0 * P.lda + k0;
    const float* pb = TB ? P.t[cur].B + (int64_t)n0 * P.ldb + k0 : P.t[cur].B + (int64_t)k0 * P.ldb + n0;
#pragma unroll
    for (int i = 0; i < A_PT; ++i) ra[i] = *reinterpret_cast<const f32x4*>(pa + oa[i]);
#pragma unroll
    for (int i = 0; i < B_PT; ++i) rb[i] = *reinterpret_cast<const f32x4*>(pb + ob[i]);
  };
  auto sstore = [&](int buf, const f32x4(&ra)[A_PT], const f32x4(&rb)[B_PT]) {
    float* As = lds + buf * (A_SZ + B_SZ);
    float* Bs = As + A_SZ;
#pragma unroll
    for (int i = 0; i < A_PT; ++i) {
      int r, c;
      kc_index<BK>(tid + 256 * i, &r, &c);
      *reinterpret_cast<f32x4*>(As + r * A_LD + c) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < B_PT; ++i) {
      const int idx = tid + 256 * i;
      if (TB) {
        int r, c;
        kc_index<BK>(idx, &r, &c);
        *reinterpret_cast<f32x4*>(Bs + r * B_LD + c) = rb[i];
      } else {
        *reinterpret_cast<f32x4*>(Bs + (idx / (BN / 4)) * B_LD + (idx % (BN / 4)) * 4) = rb[i];
      }
    }
  };
  auto frag = [&](int buf, int kb, f32x4(&fa)[FM], f32x4(&fb)[FN]) {
    const float* As = lds + buf * (A_SZ + B_SZ);
    const float* Bs = As + A_SZ;
    const int kk = kb * 8 + half * 4;
#pragma unroll
    for (int i = 0; i < FM; ++i) fa[i] = *reinterpret_cast<const f32x4*>(As + (wm * WM + i * 32 + l32) * A_LD + kk);
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int col = wn * WN + j * 32 + l32;
      if (TB) {
        fb[j] = *reinterpret_cast<const f32x4*>(Bs + col * B_LD + kk);
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) fb[j][q] = Bs[(kk + q) * B_LD + col];
      }
    }
  };
  auto mfmas = [&](const f32x4(&fa)[FM], const f32x4(&fb)[FN]) {
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(fa[i][q], fb[j][q], acc[i][j], 0, 0, 0);
  };
  auto compute = [&](int buf) {
    f32x4 fa0[FM], fb0[FN], fa1[FM], fb1[FN];
    frag(buf, 0, fa0, fb0);
    // 128 x 128 blocks with B stored [k][n] (ten LDS reads per fragment
    // set, four of them per B fragment): the next fragments' reads are
    // spread between this group's MFMAs, two MFMAs per read (4096 x 2048
    // sums over K 4 x 2048: 83.0 -> 84.9 %, over 24 x 2048: 84.8 -> 86.9 %;
    // B stored [n][k] unchanged, the 256 x 128 blocks 0.9 points slower)
    constexpr bool SPREAD = !TB && BM == 128 && BN == 128;
#pragma unroll
    for (int kb = 0; kb < BK / 8; ++kb) {
      if constexpr (SPREAD) {
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_setprio(1);
        if (kb + 1 < BK / 8) {
          if (kb & 1) frag(buf, kb + 1, fa0, fb0);
          else frag(buf, kb + 1, fa1, fb1);
        }
        if (kb & 1) mfmas(fa1, fb1);
        else mfmas(fa0, fb0);
        if (kb + 1 < BK / 8) {
          constexpr int NR = FM + 4 * FN;  // 10 reads among 16 MFMAs
#pragma unroll
          for (int r = 0; r < NR; ++r) {
            __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);  // MFMA
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
          }
        }
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_setprio(0);
        continue;
      }
      if (kb + 1 < BK / 8) {
        if (kb & 1) frag(buf, kb + 1, fa0, fb0);
        else frag(buf, kb + 1, fa1, fb1);
      }
      __builtin_amdgcn_sched_barrier(0);
      // the wave issuing MFMAs takes priority over the workgroup's other
      // waves while it does (their loads and LDS stores fill the gaps):
      // measured 77.8 -> 84.4 % of the fp32 peak on a 4096 x 8192 sum of
      // four K = 2048 pairs with B stored [n][k]; the same in gemm_block
      // measured slower (4096 x 2048 x 8192: 86 -> 82 %)
      __builtin_amdgcn_s_setprio(1);
      if (kb & 1) mfmas(fa1, fb1);
      else mfmas(fa0, fb0);
      __builtin_amdgcn_s_setprio(0);
    }
  };

  if (nk > 0) {
    gload(0, ra0, rb0);
    gload(1, ra1, rb1);
    sstore(0, ra0, rb0);
    __syncthreads();
    int kt = 0;
    for (; kt + 1 < nk; kt += 2) {
      gload(kt + 2, ra0, rb0);
      compute(0);
      sstore(1, ra1, rb1);
      __syncthreads();
      gload(kt + 3, ra1, rb1);
      compute(1);
      if (kt + 2 < nk) sstore(0, ra0, rb0);
      __syncthreads();
    }
    if (kt < nk) compute(0);
  }

  if (SPLIT) {
    float* w = P.ws + (int64_t)split * P.m * P.n;
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int col = n0 + wn * WN + j * 32 + l32;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = m0 + wm * WM + i * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
          w[(int64_t)row * P.n + col] = acc[i][j][r];
        }
      }
    return;
  }
  GemmArgs g{};
  g.beta = P.beta;
  g.C = P.C;
  g.ldc = P.ldc;
  g.epi = P.epi;
  g.bias = P.bias;
  g.res = P.res;
  g.ldr = P.ldr;
  g.aux = P.aux;
  g.ldaux = P.ldaux;
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int col = n0 + wn * WN + j * 32 + l32;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = m0 + wm * WM + i * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
        epilogue_store(g, row, col, P.alpha * acc[i][j][r]);
      }
    }
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

// plans of a batch launch: 128x128x32 / 64x64x32 blocks, or 128x128x32 with
// split-K. The big plan's BK 32 (two workgroups per CU) against BK 16
// (three): 85.3 against 82.6 % of the fp32 peak for 16 products 8192 x 2048
// x 4096 with A stored [k][m], 85.1 against 81.2 % for 25 products 4096 x
// 2048 x 2048 with B stored [n][k]
// (256 x 128 x 16 blocks, which speed up the long-K sums, do not fit the
// batch kernel's loop in 256 VGPRs and spill inside it; with one workgroup
// per CU they measured 77 against 85 % on the wide model's weight gradients)
enum BatchPlan { kBatchBig, kBatchSmall, kBatchSplit };

template <bool TA, bool TB>
int launch_batch(const GemmArgs& g, const GemmBatch& P, int blocks, BatchPlan plan, int64_t max_mn, bool vec_mn,
                 hipStream_t s) {
  const dim3 grid((unsigned)blocks), block(256);
  if (plan == kBatchBig) hipLaunchKernelGGL((gemm_batch_kernel<128, 128, 32, TA, TB, false>), grid, block, 0, s, g, P);
  else if (plan == kBatchSmall) hipLaunchKernelGGL((gemm_batch_kernel<64, 64, 32, TA, TB, false>), grid, block, 0, s, g, P);
  else hipLaunchKernelGGL((gemm_batch_kernel<128, 128, 32, TA, TB, true>), grid, block, 0, s, g, P);
  if (int rc = tt::launch_status("tile_gemm_batch")) return rc;
  if (plan != kBatchSplit) return TT_OK;
  // the workspace is 256-byte aligned and every product's region starts at
  // a multiple of 128 x 128 floats
  if (vec_mn)
    hipLaunchKernelGGL((gemm_batch_finish<128, 128, 4>), dim3((unsigned)((max_mn / 4 + 255) / 256), (unsigned)P.count),
                       block, 0, s, g, P);
  else
    hipLaunchKernelGGL((gemm_batch_finish<128, 128, 1>), dim3((unsigned)((max_mn + 255) / 256), (unsigned)P.count),
                       block, 0, s, g, P);
  return tt::launch_status("tile_gemm_batch(split finish)");
}

// split count for a batch whose products have b128 128x128 blocks in all
// and share k: as plan_for (long K, few blocks; workgroup count just under
// a multiple of the CU count); 1 = no split
int batch_splits(int64_t b128, int64_t k, size_t ws_bytes, int64_t* chunk_out) {
  if (k < 2048 || b128 > 144 || ws_bytes == 0) return 1;
  int best_s = 1;
  double best_bal = 0.0;
  for (int s = 2; s <= 8; ++s) {
    int64_t chunk = (k + s - 1) / s;
    chunk = (chunk + kSplitAlign - 1) / kSplitAlign * kSplitAlign;
    const int64_t sa = (k + chunk - 1) / chunk;
    if (chunk < 256 || (size_t)(b128 * sa) * 128 * 128 * sizeof(float) > ws_bytes) continue;
    const int64_t nwg = b128 * sa;
    const double bal = (double)nwg / (double)(((nwg + kCUs - 1) / kCUs) * kCUs);
    if (bal > best_bal + 0.01) {
      best_bal = bal;
      best_s = (int)sa;
      *chunk_out = chunk;
    }
  }
  return best_s;
}

}  // namespace

extern "C" size_t tile_gemm_workspace(int64_t m, int64_t n, int64_t k) {
  if (m <= 0 || n <= 0 || k <= 0) return 0;
  const Plan p = plan_for(m, n, k, (size_t)-1);
  return p.splits > 1 ? (size_t)p.splits * m * n * sizeof(float) : 0;
}

extern "C" int tile_gemm_ws(void* stream, int transA, int transB, int64_t m, int64_t n, int64_t k, float alpha,
                            const float* A, int64_t lda, const float* B, int64_t ldb, float beta, float* C,
                            int64_t ldc, int epilogue, const float* bias, const float* res, int64_t ldr, float* aux,
                            int64_t ldaux, void* workspace, size_t workspace_bytes) {
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
  if (workspace_bytes > 0 && !workspace) return fail(TT_ERR_ARG, "tile_gemm: null workspace");
  GemmArgs g{(int)m, (int)n, (int)k, alpha, beta, A, B, C, lda, ldb, ldc, epilogue, bias, res, ldr, aux, ldaux,
             (float*)workspace, 1, (int)k};
  const bool va = k > 0 && aligned16(A) && lda % 4 == 0;
  const bool vb = k > 0 && aligned16(B) && ldb % 4 == 0;
  const size_t wsb = workspace ? workspace_bytes : 0;
  hipStream_t s = tt::as_stream(stream);
  if (!transA && !transB) return launch_t<false, false>(g, va, vb, wsb, s);
  if (!transA && transB) return launch_t<false, true>(g, va, vb, wsb, s);
  if (transA && !transB) return launch_t<true, false>(g, va, vb, wsb, s);
  return launch_t<true, true>(g, va, vb, wsb, s);
}

extern "C" int tile_gemm(void* stream, int transA, int transB, int64_t m, int64_t n, int64_t k, float alpha,
                         const float* A, int64_t lda, const float* B, int64_t ldb, float beta, float* C, int64_t ldc,
                         int epilogue, const float* bias, const float* res, int64_t ldr, float* aux, int64_t ldaux) {
  return tile_gemm_ws(stream, transA, transB, m, n, k, alpha, A, lda, B, ldb, beta, C, ldc, epilogue, bias, res, ldr,
                      aux, ldaux, nullptr, 0);
}

namespace {

// K-sum block plan: 128x128 blocks when there are >= 512 of them, BK 32
// (two workgroups per CU; measured against BK 16 on 4096 x 2048 outputs:
// 83.5 against 82.5 % for four K = 2048 pairs, 87.5 against 86.1 % for four
// K = 8192 pairs with B stored [n][k]), else 64x64x32. TT_KSUM_BK=16|32
// overrides the big blocks' BK (tuning).
// 256 x 128 x 16 blocks (each wave 128 x 64: 8 MFMA tiles against 4, so
// a quarter fewer LDS reads and global loads per flop; 250-256 VGPRs, two
// workgroups per CU) for long-K sums of >= 1024 blocks of 128 x 128, i.e.
// >= 512 of the larger ones: the wide model's MLP input layer (4096 x 8192,
// K 4 x 2048) 82.8 -> 86.3 % of the fp32 peak, its output layer's input
// gradient 83.5 -> 84.5 %. Measured alternatives on the same sums: 128 x 256
// x 16 85.1 / 84.6 %; BK 32 (332-368 VGPRs, one workgroup per CU) 78 / 76 %;
// 256 x 256 (256 accumulators per lane) spills them to scratch: 32 %.
// TT_KSUM_HUGE = "BMxBNxBK" (256x128, 128x256 or 256x256 with BK 16 or 32)
// or "off" overrides (tuning).
struct HugePlan {
  int bm = 0, bn = 0, bk = 0;
};
HugePlan ksum_huge() {
  static HugePlan p{256, 128, 16};
  static bool read = false;
  if (!read) {
    read = true;
    if (const char* e = getenv("TT_KSUM_HUGE")) {
      int a = 0, b = 0, c = 0;
      if (sscanf(e, "%dx%dx%d", &a, &b, &c) == 3 && (c == 16 || c == 32) &&
          ((a == 256 && (b == 128 || b == 256)) || (a == 128 && b == 256)))
        p = HugePlan{a, b, c};
      else
        p = HugePlan{};
    }
  }
  return p;
}

int ksum_big_bk(int64_t) {
  static int forced = -1;
  if (forced < 0) {
    forced = 0;
    if (const char* e = getenv("TT_KSUM_BK")) forced = atoi(e) == 32 ? 32 : (atoi(e) == 16 ? 16 : 0);
  }
  return forced ? forced : 32;
}

}  // namespace

namespace {

// Split-K K-sums: outputs of at most 128 blocks of 128 x 128 (m and n
// multiples of 128) with a workspace split the concatenated K steps (BK 32)
// into slices so that blocks x slices comes to 512 (two workgroups per CU),
// at most 16 slices of at least 16 steps each. Between 129 and 511 blocks
// the 64x64 plan already has 516 to 2044 workgroups (measured: a 4096 x 768
// sum over 66 pairs of K 768 at 2.66 ms per GPT2-small step unsplit, 3.16 ms
// as 192 blocks x 2 slices).
constexpr int kKsumSplitMax = 16, kKsumSplitMinSteps = 16;
bool ksum_split_shape(int64_t m, int64_t n) {
  return m % 128 == 0 && n % 128 == 0 && (m / 128) * (n / 128) <= 128;
}
int ksum_splits(int64_t m, int64_t n, int64_t steps, size_t ws_bytes) {
  const int64_t b128 = (m / 128) * (n / 128);
  int64_t sp = std::min<int64_t>(kKsumSplitMax, std::max<int64_t>(1, 512 / b128));
  sp = std::min<int64_t>(sp, steps / kKsumSplitMinSteps);
  sp = std::min<int64_t>(sp, (int64_t)(ws_bytes / ((size_t)m * n * sizeof(float))));
  return (int)std::max<int64_t>(1, sp);
}

}  // namespace

extern "C" size_t tile_gemm_ksum_workspace(int64_t m, int64_t n) {
  if (m <= 0 || n <= 0 || !ksum_split_shape(m, n)) return 0;
  const int64_t b128 = (m / 128) * (n / 128);
  return (size_t)std::min<int64_t>(kKsumSplitMax, std::max<int64_t>(1, 512 / b128)) * m * n * sizeof(float);
}

extern "C" int tile_gemm_ksum_ex(void* stream, int count, int transB, int64_t m, int64_t n, const int64_t* k,
                                 float alpha, const float* const* A, const int64_t* lda, const float* const* B,
                                 const int64_t* ldb, float beta, float* C, int64_t ldc, int epilogue,
                                 const float* bias, const float* res, int64_t ldr, float* aux, int64_t ldaux) {
  return tile_gemm_ksum_ws(stream, count, transB, m, n, k, alpha, A, lda, B, ldb, beta, C, ldc, epilogue, bias, res,
                           ldr, aux, ldaux, nullptr, 0);
}

extern "C" int tile_gemm_ksum_ws(void* stream, int count, int transB, int64_t m, int64_t n, const int64_t* k,
                                 float alpha, const float* const* A, const int64_t* lda, const float* const* B,
                                 const int64_t* ldb, float beta, float* C, int64_t ldc, int epilogue,
                                 const float* bias, const float* res, int64_t ldr, float* aux, int64_t ldaux,
                                 void* workspace, size_t workspace_bytes) {
  using tt::fail;
  if (count < 0 || m < 0 || n < 0) return fail(TT_ERR_ARG, "tile_gemm_ksum: negative count or size");
  if (m == 0 || n == 0) return TT_OK;
  if (m > INT32_MAX || n > INT32_MAX) return fail(TT_ERR_ARG, "tile_gemm_ksum: size exceeds int32");
  if (!C || ldc < n) return fail(TT_ERR_ARG, "tile_gemm_ksum: bad C");
  if (count > 0 && (!k || !A || !lda || !B || !ldb)) return fail(TT_ERR_ARG, "tile_gemm_ksum: null array");
  if (epilogue & ~(TT_EPI_BIAS | TT_EPI_RES | TT_EPI_GELU | TT_EPI_GELU_BWD))
    return fail(TT_ERR_ARG, "tile_gemm_ksum: unknown epilogue bits");
  if ((epilogue & TT_EPI_GELU) && (epilogue & TT_EPI_GELU_BWD))
    return fail(TT_ERR_ARG, "tile_gemm_ksum: GELU and GELU_BWD are exclusive");
  if ((epilogue & TT_EPI_BIAS) && !bias) return fail(TT_ERR_ARG, "tile_gemm_ksum: BIAS without bias");
  if ((epilogue & TT_EPI_RES) && (!res || ldr < n)) return fail(TT_ERR_ARG, "tile_gemm_ksum: bad residual");
  if ((epilogue & (TT_EPI_GELU | TT_EPI_GELU_BWD)) && (!aux || ldaux < n))
    return fail(TT_ERR_ARG, "tile_gemm_ksum: GELU epilogue needs aux");
  for (int t = 0; t < count; ++t) {
    if (k[t] < 0 || k[t] > INT32_MAX) return fail(TT_ERR_ARG, "tile_gemm_ksum: bad k of pair %d", t);
    if (k[t] > 0 && (!A[t] || !B[t] || lda[t] < k[t] || ldb[t] < (transB ? k[t] : n)))
      return fail(TT_ERR_ARG, "tile_gemm_ksum: bad operand of pair %d", t);
  }
  if (workspace_bytes > 0 && (!workspace || !aligned16(workspace)))
    return fail(TT_ERR_ARG, "tile_gemm_ksum: null or misaligned workspace");
  hipStream_t s = tt::as_stream(stream);
  // block plan: 128x128 blocks when there are >= 512 of them; split-K over
  // 128x128x32 blocks for fewer than 256 with a workspace; else 64x64x32
  const int64_t b128 = (m / 128) * (n / 128);
  const bool big = b128 >= 512;
  const HugePlan hp = ksum_huge();
  // both plans run two workgroups per CU (512 slots): the larger blocks
  // only where their last round is as full as the smaller ones' (a 4096 x
  // 5632 output -- the LLaMA-style wide model's ragged SwiGLU tile -- is
  // 1408 blocks of 128 x 128, 92 % of 3 rounds, but 704 of 256 x 128, 69 %
  // of 2: 85 -> 79 % of the fp32 peak), allowing their ~4 % per block
  auto round_fill = [](int64_t blocks) { return (double)blocks / (double)(((blocks + 511) / 512) * 512); };
  const bool huge = b128 >= 1024 && hp.bm > 0 && m % hp.bm == 0 && n % hp.bn == 0 &&
                    1.04 * round_fill((m / hp.bm) * (n / hp.bn)) >= round_fill(b128);
  int64_t total_steps = 0;
  for (int t = 0; t < count; ++t) total_steps += k[t] / 32;
  const bool try_split = !big && workspace && ksum_split_shape(m, n) &&
                         ksum_splits(m, n, total_steps, workspace_bytes) > 1;
  const int bm = huge ? hp.bm : (big || try_split ? 128 : 64), bn = huge ? hp.bn : bm;
  const int bk = huge ? hp.bk : (big ? ksum_big_bk(b128) : 32);
  auto fits = [&](int t) {  // a pair the branch-free long-K launch can take
    return k[t] % bk == 0 && m % bm == 0 && n % bn == 0 && aligned16(A[t]) && aligned16(B[t]) && lda[t] % 4 == 0 &&
           ldb[t] % 4 == 0 && (int64_t)bm * lda[t] < INT32_MAX && (int64_t)(transB ? bn : bk) * ldb[t] < INT32_MAX;
  };
  if (epilogue != TT_EPI_NONE) {  // the epilogue needs the whole sum in one launch
    int live = 0;
    for (int t = 0; t < count; ++t)
      if (k[t] > 0) {
        if (!fits(t) || lda[t] != lda[0] || ldb[t] != ldb[0])
          return fail(TT_ERR_UNSUPPORTED, "tile_gemm_ksum: with an epilogue every pair must fit one launch");
        ++live;
      }
    if (live == 0 || live > kKsumMax)
      return fail(TT_ERR_UNSUPPORTED, "tile_gemm_ksum: with an epilogue 1..%d pairs are needed", kKsumMax);
  }
  float b = beta;  // C's own weight: beta in the first contribution, 1 afterwards
  bool wrote = false;
  int t = 0;
  while (t < count) {
    if (k[t] == 0) {
      ++t;
      continue;
    }
    if (!fits(t)) {  // on its own, through the general kernel
      if (int rc = tile_gemm(stream, 0, transB ? 1 : 0, m, n, k[t], alpha, A[t], lda[t], B[t], ldb[t], b, C, ldc,
                             TT_EPI_NONE, nullptr, nullptr, 0, nullptr, 0))
        return rc;
      b = 1.f;
      wrote = true;
      ++t;
      continue;
    }
    KsumArgs P{};
    P.m = (int)m;
    P.n = (int)n;
    P.alpha = alpha;
    P.beta = b;
    P.C = C;
    P.lda = lda[t];
    P.ldb = ldb[t];
    P.ldc = ldc;
    P.epi = epilogue;
    P.bias = bias;
    P.res = res;
    P.ldr = ldr;
    P.aux = aux;
    P.ldaux = ldaux;
    int c = 0;
    int64_t steps = 0;
    while (t < count && c < kKsumMax && (k[t] == 0 || (fits(t) && lda[t] == P.lda && ldb[t] == P.ldb))) {
      if (k[t] > 0) {
        P.t[c++] = {A[t], B[t], k[t] / bk};
        steps += k[t] / bk;
      }
      ++t;
    }
    if (steps > INT32_MAX) return fail(TT_ERR_ARG, "tile_gemm_ksum: K too long");
    P.nk = (int)steps;
    const int splits = try_split ? ksum_splits(m, n, steps, workspace_bytes) : 1;
    if (splits > 1) {
      P.ws = (float*)workspace;
      P.chunk = (int)((steps + splits - 1) / splits);
      const int used = (int)((steps + P.chunk - 1) / P.chunk);  // every slice non-empty
      const dim3 grid((unsigned)(b128 * used));
      if (transB) hipLaunchKernelGGL((gemm_ksum_kernel<128, 128, 32, true, true>), grid, dim3(256), 0, s, P);
      else hipLaunchKernelGGL((gemm_ksum_kernel<128, 128, 32, false, true>), grid, dim3(256), 0, s, P);
      if (int rc = tt::launch_status("tile_gemm_ksum(split)")) return rc;
      GemmArgs g{(int)m, (int)n, 0, alpha, b, nullptr, nullptr, C, 0, 0, ldc, epilogue, bias, res, ldr, aux, ldaux,
                 (float*)workspace, used, 0};
      const int64_t mn = m * n;  // a multiple of 128 x 128
      hipLaunchKernelGGL(gemm_split_finish<4>, dim3((unsigned)((mn / 4 + 255) / 256)), dim3(256), 0, s, g);
      if (int rc = tt::launch_status("tile_gemm_ksum(split finish)")) return rc;
    } else {
      const dim3 grid((unsigned)((m / bm) * (n / bn)));
      if (huge) {
#define TT_KH(BM_, BN_, BK_)                                                                              \
  if (bm == BM_ && bn == BN_ && bk == BK_) {                                                              \
    if (transB) hipLaunchKernelGGL((gemm_ksum_kernel<BM_, BN_, BK_, true, false>), grid, dim3(256), 0, s, P); \
    else hipLaunchKernelGGL((gemm_ksum_kernel<BM_, BN_, BK_, false, false>), grid, dim3(256), 0, s, P);       \
  }
        TT_KH(256, 128, 16)
        TT_KH(256, 128, 32)
        TT_KH(128, 256, 16)
        TT_KH(128, 256, 32)
        TT_KH(256, 256, 16)
        TT_KH(256, 256, 32)
#undef TT_KH
      } else if (transB) {
        if (big && bk == 32) hipLaunchKernelGGL((gemm_ksum_kernel<128, 128, 32, true, false>), grid, dim3(256), 0, s, P);
        else if (big) hipLaunchKernelGGL((gemm_ksum_kernel<128, 128, 16, true, false>), grid, dim3(256), 0, s, P);
        else if (bm == 128) hipLaunchKernelGGL((gemm_ksum_kernel<128, 128, 32, true, false>), grid, dim3(256), 0, s, P);
        else hipLaunchKernelGGL((gemm_ksum_kernel<64, 64, 32, true, false>), grid, dim3(256), 0, s, P);
      } else {
        if (big && bk == 32) hipLaunchKernelGGL((gemm_ksum_kernel<128, 128, 32, false, false>), grid, dim3(256), 0, s, P);
        else if (big) hipLaunchKernelGGL((gemm_ksum_kernel<128, 128, 16, false, false>), grid, dim3(256), 0, s, P);
        else if (bm == 128) hipLaunchKernelGGL((gemm_ksum_kernel<128, 128, 32, false, false>), grid, dim3(256), 0, s, P);
        else hipLaunchKernelGGL((gemm_ksum_kernel<64, 64, 32, false, false>), grid, dim3(256), 0, s, P);
      }
      if (int rc = tt::launch_status("tile_gemm_ksum")) return rc;
    }
    b = 1.f;
    wrote = true;
  }
  if (!wrote)  // no product at all: C = beta * C
    return tile_gemm(stream, 0, 0, m, n, 0, alpha, nullptr, 1, nullptr, n, beta, C, ldc, TT_EPI_NONE, nullptr, nullptr,
                     0, nullptr, 0);
  return TT_OK;
}

extern "C" int tile_gemm_ksum(void* stream, int count, int transB, int64_t m, int64_t n, const int64_t* k,
                              float alpha, const float* const* A, const int64_t* lda, const float* const* B,
                              const int64_t* ldb, float beta, float* C, int64_t ldc) {
  return tile_gemm_ksum_ex(stream, count, transB, m, n, k, alpha, A, lda, B, ldb, beta, C, ldc, TT_EPI_NONE, nullptr,
                           nullptr, 0, nullptr, 0);
}

extern "C" size_t tile_gemm_batch_workspace(int count, const int64_t* m, const int64_t* n, int64_t k) {
  if (count <= 0 || !m || !n || k <= 0) return 0;
  int64_t b128 = 0;
  for (int t = 0; t < count; ++t)
    if (m[t] > 0 && n[t] > 0) b128 += ((m[t] + 127) / 128) * ((n[t] + 127) / 128);
  int64_t chunk = k;
  const int sp = batch_splits(b128, k, (size_t)-1, &chunk);
  return sp > 1 ? (size_t)(b128 * sp) * 128 * 128 * sizeof(float) : 0;
}

namespace {

// cross-entropy statistics epilogue of a batched launch (tile_gemm_batch_xstats)
struct XStats {
  const int32_t* labels;
  float* parts;
  int64_t part_stride, v_off0, v_tile;
};

int batch_run(void* stream, int count, int transA, int transB, const int64_t* m, const int64_t* n, int64_t k,
              float alpha, const float* const* A, const int64_t* lda, const float* const* B, const int64_t* ldb,
              float beta, float* const* C, const int64_t* ldc, void* workspace, size_t workspace_bytes,
              const XStats* xs) {
  using tt::fail;
  if (count < 0 || k < 0) return fail(TT_ERR_ARG, "tile_gemm_batch: negative count or k");
  if (count == 0) return TT_OK;
  if (k > INT32_MAX) return fail(TT_ERR_ARG, "tile_gemm_batch: k exceeds int32");
  if (!m || !n || !A || !lda || !B || !ldb || !C || !ldc) return fail(TT_ERR_ARG, "tile_gemm_batch: null array");
  if (workspace_bytes > 0 && !workspace) return fail(TT_ERR_ARG, "tile_gemm_batch: null workspace");
  for (int t = 0; t < count; ++t) {
    if (m[t] < 0 || n[t] < 0 || m[t] > INT32_MAX || n[t] > INT32_MAX)
      return fail(TT_ERR_ARG, "tile_gemm_batch: bad size of product %d", t);
    if (m[t] == 0 || n[t] == 0) continue;
    if (!C[t] || ldc[t] < n[t] || ldc[t] > INT32_MAX) return fail(TT_ERR_ARG, "tile_gemm_batch: bad C of product %d", t);
    if (k > 0 && (!A[t] || !B[t] || lda[t] < (transA ? m[t] : k) || ldb[t] < (transB ? k : n[t]) ||
                  lda[t] > INT32_MAX || ldb[t] > INT32_MAX))
      return fail(TT_ERR_ARG, "tile_gemm_batch: bad operand of product %d", t);
  }
  hipStream_t s = tt::as_stream(stream);
  // the plan tile_gemm would pick if the products were one C: split-K over
  // 128x128x32 blocks for few blocks and a long K (with a workspace),
  // 128x128x32 blocks when there are >= 512 of them, else 64x64x32. Unlike
  // tile_gemm's single products, a batch keeps 128x128 whatever the fill of
  // its last round: the small-tile wide model's LM head (99 products of
  // 1024 x 512 x 512, rounds 95 % full) ran at 45 % of the fp32 peak on
  // 64x64 blocks against 56 % on 128x128
  int64_t b128 = 0;
  for (int t = 0; t < count; ++t)
    if (m[t] > 0 && n[t] > 0) b128 += ((m[t] + 127) / 128) * ((n[t] + 127) / 128);
  int64_t chunk = k;
  // the statistics epilogue needs whole 128x128 blocks in one pass
  const int splits = xs ? 1 : batch_splits(b128, k, workspace ? workspace_bytes : 0, &chunk);
  const BatchPlan plan = splits > 1 ? kBatchSplit : (b128 >= 512 || xs) ? kBatchBig : kBatchSmall;
  const int bm = plan == kBatchSmall ? 64 : 128, bn = bm;
  GemmArgs g{0, 0, (int)k, alpha, beta, nullptr, nullptr, nullptr, 0, 0, 0, TT_EPI_NONE, nullptr,
             nullptr, 0, nullptr, 0, (float*)workspace, splits, (int)chunk};
  if (xs) {
    g.epi = TT_EPI_XSTATS;
    g.xlab = xs->labels;
    g.xparts = xs->parts;
    g.xvoff = xs->v_off0;
    g.xstride = xs->part_stride;
    g.xvtile = xs->v_tile;
  }
  // products whose loads are scalar (a ragged tile's odd leading dimension)
  // run slower blocks: they go first in the grid, so the hardware starts
  // them first and the rest fill in around them (longest first)
  auto vec_a = [&](int t) { return k > 0 && lda[t] % 4 == 0 && aligned16(A[t]); };
  auto vec_b = [&](int t) { return k > 0 && ldb[t] % 4 == 0 && aligned16(B[t]); };
  auto vec_ok = [&](int t) { return vec_a(t) && vec_b(t); };
  std::vector<int> order;
  for (int t = 0; t < count; ++t)
    if (!vec_ok(t)) order.push_back(t);
  for (int t = 0; t < count; ++t)
    if (vec_ok(t)) order.push_back(t);
  // grid.x * 256 work-items must stay below 2^32
  const int64_t max_blocks = (int64_t)(UINT32_MAX / 256);
  int o = 0;
  while (o < count) {
    GemmBatch P{};
    int64_t blocks = 0, max_mn = 0;
    bool vec_mn = true;
    while (o < count && P.count < kBatchMax) {
      const int t = order[o];
      const int64_t nb =
          m[t] == 0 || n[t] == 0 ? 0 : ((m[t] + bm - 1) / bm) * ((n[t] + bn - 1) / bn) * (int64_t)splits;
      if (nb > max_blocks) return fail(TT_ERR_SHAPE, "tile_gemm_batch: product %d too large for one launch", t);
      if (blocks + nb > max_blocks) break;
      if (nb > 0) {
        const int c = P.count++;
        P.A[c] = A[t];
        P.B[c] = B[t];
        P.C[c] = C[t];
        P.m[c] = (int)m[t];
        P.n[c] = (int)n[t];
        P.lda[c] = (int)lda[t];
        P.ldb[c] = (int)ldb[t];
        P.ldc[c] = (int)ldc[t];
        P.first[c] = (int)blocks;
        P.orig[c] = (short)t;
        if (vec_a(t)) P.va[c >> 5] |= 1u << (c & 31);
        if (vec_b(t)) P.vb[c >> 5] |= 1u << (c & 31);
        blocks += nb;
        max_mn = std::max<int64_t>(max_mn, m[t] * n[t]);
        vec_mn = vec_mn && (m[t] * n[t]) % 4 == 0;
      }
      ++o;
    }
    if (P.count == 0) continue;
    int rc;
    if (!transA && !transB) rc = launch_batch<false, false>(g, P, (int)blocks, plan, max_mn, vec_mn, s);
    else if (!transA && transB) rc = launch_batch<false, true>(g, P, (int)blocks, plan, max_mn, vec_mn, s);
    else if (transA && !transB) rc = launch_batch<true, false>(g, P, (int)blocks, plan, max_mn, vec_mn, s);
    else rc = launch_batch<true, true>(g, P, (int)blocks, plan, max_mn, vec_mn, s);
    if (rc) return rc;
  }
  return TT_OK;
}

}  // namespace

extern "C" int tile_gemm_batch_ws(void* stream, int count, int transA, int transB, const int64_t* m,
                                  const int64_t* n, int64_t k, float alpha, const float* const* A, const int64_t* lda,
                                  const float* const* B, const int64_t* ldb, float beta, float* const* C,
                                  const int64_t* ldc, void* workspace, size_t workspace_bytes) {
  return batch_run(stream, count, transA, transB, m, n, k, alpha, A, lda, B, ldb, beta, C, ldc, workspace,
                   workspace_bytes, nullptr);
}

extern "C" int tile_gemm_batch_xstats(void* stream, int count, int transB, int64_t m, const int64_t* n, int64_t k,
                                      float alpha, const float* const* A, const int64_t* lda, const float* const* B,
                                      const int64_t* ldb, float beta, float* const* C, const int64_t* ldc,
                                      const int32_t* labels, int64_t v_off0, int64_t v_tile, float* parts,
                                      int64_t part_stride) {
  using tt::fail;
  if (count < 0 || m < 0 || k < 0) return fail(TT_ERR_ARG, "tile_gemm_batch_xstats: negative count or size");
  if (count == 0 || m == 0) return TT_OK;
  if (count > INT16_MAX) return fail(TT_ERR_ARG, "tile_gemm_batch_xstats: more than %d products", INT16_MAX);
  if (!n || !labels || !parts || v_tile < 1 || v_off0 < 0)
    return fail(TT_ERR_ARG, "tile_gemm_batch_xstats: null array, labels or partials, or bad vocab offsets");
  int64_t groups = 0;
  for (int t = 0; t < count; ++t) {
    if (n[t] < 1 || n[t] > v_tile) return fail(TT_ERR_ARG, "tile_gemm_batch_xstats: n of product %d not in 1..v_tile", t);
    groups = std::max<int64_t>(groups, (n[t] + 63) / 64);
  }
  if (part_stride < groups * m * 3)
    return fail(TT_ERR_ARG, "tile_gemm_batch_xstats: part_stride below %lld floats", (long long)(groups * m * 3));
  std::vector<int64_t> ms(count, m);
  const XStats xs{labels, parts, part_stride, v_off0, v_tile};
  return batch_run(stream, count, 0, transB, ms.data(), n, k, alpha, A, lda, B, ldb, beta, C, ldc, nullptr, 0, &xs);
}

extern "C" int tile_gemm_batch(void* stream, int count, int transA, int transB, const int64_t* m, const int64_t* n,
                               int64_t k, float alpha, const float* const* A, const int64_t* lda,
                               const float* const* B, const int64_t* ldb, float beta, float* const* C,
                               const int64_t* ldc) {
  return tile_gemm_batch_ws(stream, count, transA, transB, m, n, k, alpha, A, lda, B, ldb, beta, C, ldc, nullptr, 0);
}
