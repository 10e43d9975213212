// LayerNorm tile tasks (forward, backward) and the deterministic column sums
// they and the linear-layer bias gradient use.
//
// LayerNorm is HBM-bound: each row (token) is read once, reduced with one
// wave64 butterfly and written once. One wave owns one row at a time; a row
// tile of up to 2048 features stays in registers (NV float4 per lane), so
// the two-pass mean / squared-deviation statistics cost no second read.
// When the embedding axis is split into several feature tiles, each tile
// contributes (count, mean, M2) and the partials are merged in tile order
// with the parallel-variance update of Chan, Golub and LeVeque.
#include "rowops.hpp"

#include <mutex>

using tt::f32x4;

namespace {

constexpr int kWaves = 4;  // waves per workgroup

// ------------------------------------------------------------- forward

// phase FUSED: stats + y; phase PARTIAL: (count, mean, M2) only
template <int NV, bool VEC>
__global__ __launch_bounds__(256) void ln_fwd_rows(int phase, int rows, int cols, const float* __restrict__ x,
                                                   int64_t ldx, const float* __restrict__ gamma,
                                                   const float* __restrict__ beta, float* __restrict__ parts,
                                                   float* __restrict__ stats, float* __restrict__ y, int64_t ldy,
                                                   float eps) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * kWaves + (threadIdx.x >> 6);
  if (row >= rows) return;
  f32x4 v[NV];
  float sum = 0.f;
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const int c = (j * 64 + lane) * 4;
    v[j] = c < cols ? tt::ld4<VEC>(x, ldx, row, c, cols) : f32x4{0.f, 0.f, 0.f, 0.f};
    sum += (v[j][0] + v[j][1]) + (v[j][2] + v[j][3]);
  }
  const float mean = tt::wave_sum(sum) / (float)cols;
  float m2 = 0.f;
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const int c = (j * 64 + lane) * 4;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (c + i < cols) {
        const float d = v[j][i] - mean;
        m2 += d * d;
      }
  }
  m2 = tt::wave_sum(m2);
  if (phase == TT_LN_PARTIAL) {
    if (lane == 0) {
      parts[(int64_t)row * 3 + 0] = (float)cols;
      parts[(int64_t)row * 3 + 1] = mean;
      parts[(int64_t)row * 3 + 2] = m2;
    }
    return;
  }
  const float rstd = 1.f / sqrtf(m2 / (float)cols + eps);
  if (lane == 0) {
    stats[(int64_t)row * 2 + 0] = mean;
    stats[(int64_t)row * 2 + 1] = rstd;
  }
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const int c = (j * 64 + lane) * 4;
    if (c >= cols) continue;
    const f32x4 g = tt::ldv4<VEC>(gamma, c, cols), b = tt::ldv4<VEC>(beta, c, cols);
    f32x4 o;
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = (v[j][i] - mean) * rstd * g[i] + b[i];
    tt::st4<VEC>(y, ldy, row, c, cols, o);
  }
}

__global__ void ln_fwd_merge(int rows, int n_parts, const float* __restrict__ parts, int64_t stride,
                             float* __restrict__ stats, float eps) {
  const int row = blockIdx.x * blockDim.x + threadIdx.x;
  if (row >= rows) return;
  float n = parts[(int64_t)row * 3], mean = parts[(int64_t)row * 3 + 1], m2 = parts[(int64_t)row * 3 + 2];
  for (int p = 1; p < n_parts; ++p) {
    const float* q = parts + p * stride + (int64_t)row * 3;
    const float nb = q[0], mb = q[1], m2b = q[2];
    const float nn = n + nb, delta = mb - mean;
    mean += delta * (nb / nn);
    m2 += m2b + delta * delta * (n * nb / nn);
    n = nn;
  }
  stats[(int64_t)row * 2] = mean;
  stats[(int64_t)row * 2 + 1] = 1.f / sqrtf(m2 / n + eps);
}

template <bool VEC>
__global__ void ln_fwd_apply(int rows, int cols, const float* __restrict__ x, int64_t ldx,
                             const float* __restrict__ gamma, const float* __restrict__ beta,
                             const float* __restrict__ stats, float* __restrict__ y, int64_t ldy) {
  const int c4 = (blockIdx.x * blockDim.x + threadIdx.x) * 4;
  const int row = blockIdx.y;
  if (c4 >= cols) return;
  const float mean = stats[(int64_t)row * 2], rstd = stats[(int64_t)row * 2 + 1];
  const f32x4 v = tt::ld4<VEC>(x, ldx, row, c4, cols);
  const f32x4 g = tt::ldv4<VEC>(gamma, c4, cols), b = tt::ldv4<VEC>(beta, c4, cols);
  f32x4 o;
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = (v[i] - mean) * rstd * g[i] + b[i];
  tt::st4<VEC>(y, ldy, row, c4, cols, o);
}

// ------------------------------------------------------------- backward

// Each wave takes kRowsPerWave consecutive rows; a workgroup has bwd_waves(NV)
// waves (as many as the row's registers allow), so one block covers
// kRowsPerWave * waves rows and few per-block column partials remain.
constexpr int kRowsPerWave = 2;
__host__ __device__ constexpr int bwd_waves(int nv) { return nv <= 2 ? 16 : (nv <= 4 ? 8 : 4); }

// phase PARTIAL: parts = (sum dxhat, sum dxhat*xhat); FUSED / APPLY: dx and
// per-block column partials of dy*xhat and dy into ws[block][2][cols].
template <int NV, bool VEC>
__global__ __launch_bounds__(64 * bwd_waves(NV)) void ln_bwd_rows(
    int phase, int rows, int cols, float n_total, const float* __restrict__ dy, int64_t lddy,
    const float* __restrict__ x, int64_t ldx, const float* __restrict__ gamma, const float* __restrict__ stats,
    float* __restrict__ parts, int n_parts, int64_t part_stride, float* __restrict__ dx, int64_t lddx, int dx_acc,
    float* __restrict__ ws) {
  constexpr int kWaves = bwd_waves(NV);
  constexpr int kRowsPerBlock = kWaves * kRowsPerWave;
  __shared__ f32x4 red[kWaves][2][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  f32x4 g[NV], dg[NV], db[NV];
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const int c = (j * 64 + lane) * 4;
    g[j] = c < cols ? tt::ldv4<VEC>(gamma, c, cols) : f32x4{0.f, 0.f, 0.f, 0.f};
    dg[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    db[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const float inv_n = 1.f / n_total;
  for (int rr = 0; rr < kRowsPerWave; ++rr) {
    const int row = blockIdx.x * kRowsPerBlock + wave * kRowsPerWave + rr;
    if (row >= rows) break;
    const float mean = stats[(int64_t)row * 2], rstd = stats[(int64_t)row * 2 + 1];
    f32x4 xh[NV], dxh[NV];
    float s1 = 0.f, s2 = 0.f;
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const int c = (j * 64 + lane) * 4;
      f32x4 xv = f32x4{0.f, 0.f, 0.f, 0.f}, dv = xv;
      if (c < cols) {
        xv = tt::ld4<VEC>(x, ldx, row, c, cols);
        dv = tt::ld4<VEC>(dy, lddy, row, c, cols);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool ok = c + i < cols;
        xh[j][i] = ok ? (xv[i] - mean) * rstd : 0.f;
        dxh[j][i] = dv[i] * g[j][i];
        s1 += dxh[j][i];
        s2 += dxh[j][i] * xh[j][i];
        dg[j][i] += dv[i] * xh[j][i];
        db[j][i] += dv[i];
      }
    }
    if (phase == TT_LN_PARTIAL) {
      s1 = tt::wave_sum(s1);
      s2 = tt::wave_sum(s2);
      if (lane == 0) {
        parts[(int64_t)row * 2] = s1;
        parts[(int64_t)row * 2 + 1] = s2;
      }
      continue;
    }
    if (phase == TT_LN_FUSED) {
      s1 = tt::wave_sum(s1);
      s2 = tt::wave_sum(s2);
    } else {  // APPLY: merge the per-tile partial sums in tile order
      s1 = 0.f;
      s2 = 0.f;
      for (int p = 0; p < n_parts; ++p) {
        s1 += parts[p * part_stride + (int64_t)row * 2];
        s2 += parts[p * part_stride + (int64_t)row * 2 + 1];
      }
    }
    const float a1 = s1 * inv_n, a2 = s2 * inv_n;
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const int c = (j * 64 + lane) * 4;
      if (c >= cols) continue;
      f32x4 o;
#pragma unroll
      for (int i = 0; i < 4; ++i) o[i] = rstd * (dxh[j][i] - a1 - xh[j][i] * a2);
      if (dx_acc) {
        const f32x4 old = tt::ld4<VEC>(dx, lddx, row, c, cols);
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] += old[i];
      }
      tt::st4<VEC>(dx, lddx, row, c, cols, o);
    }
  }
  if (phase == TT_LN_PARTIAL) return;
  // combine the 4 waves' column partials in wave order, one 256-column chunk at a time
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    red[wave][0][lane] = dg[j];
    red[wave][1][lane] = db[j];
    __syncthreads();
    if (wave == 0) {
      const int c = (j * 64 + lane) * 4;
      f32x4 a = red[0][0][lane], b = red[0][1][lane];
#pragma unroll
      for (int w = 1; w < kWaves; ++w) {
        a += red[w][0][lane];
        b += red[w][1][lane];
      }
      float* out = ws + (int64_t)blockIdx.x * 2 * cols;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (c + i < cols) {
          out[c + i] = a[i];
          out[cols + c + i] = b[i];
        }
    }
    __syncthreads();
  }
}

}  // namespace

// Column sums of nblk partial rows -> out[c] (+)= sum_b ws[b*ws_ld + ws_off + c],
// in a fixed order. One workgroup: kSumCols (16) columns x 64 row groups;
// group g sums rows g, g+64, ... (loads issued 4 at a time), then the 64
// group sums are added in group order. Narrow workgroups give a 768-column
// sum 48 workgroups instead of the 12 of 64-column ones (the RMSNorm gain
// gradient over 1024 partial rows: 8.1 -> 5.2 us). blockIdx.y = 1 does the
// same for (ws_off2, out2): LayerNorm's dgamma and dbeta in one launch.
constexpr int kSumCols = 16;
__device__ __forceinline__ void colsum_finish_block(int nblk, int cols, const float* __restrict__ ws, int64_t ws_ld,
                                                    int64_t ws_off, float* __restrict__ out, int accumulate) {
  constexpr int G = 1024 / kSumCols;
  __shared__ float red[G][kSumCols];
  const int cl = threadIdx.x % kSumCols, grp = threadIdx.x / kSumCols;
  const int c = blockIdx.x * kSumCols + cl;
  float s = 0.f;
  if (c < cols) {
    const float* src = ws + ws_off + c;
    int b = grp;
    for (; b + 3 * G < nblk; b += 4 * G) {
      const float v0 = src[(int64_t)b * ws_ld], v1 = src[(int64_t)(b + G) * ws_ld];
      const float v2 = src[(int64_t)(b + 2 * G) * ws_ld], v3 = src[(int64_t)(b + 3 * G) * ws_ld];
      s += v0;
      s += v1;
      s += v2;
      s += v3;
    }
    for (; b < nblk; b += G) s += src[(int64_t)b * ws_ld];
  }
  red[grp][cl] = s;
  __syncthreads();
  if (grp == 0 && c < cols) {
    float t = 0.f;
    for (int i = 0; i < G; ++i) t += red[i][cl];
    out[c] = accumulate ? out[c] + t : t;
  }
}

__global__ __launch_bounds__(1024) void colsum_finish(int nblk, int cols, const float* __restrict__ ws,
                                                      int64_t ws_ld, int64_t ws_off, float* __restrict__ out,
                                                      int accumulate, int64_t ws_off2, float* __restrict__ out2) {
  if (blockIdx.y == 1) colsum_finish_block(nblk, cols, ws, ws_ld, ws_off2, out2, accumulate);
  else colsum_finish_block(nblk, cols, ws, ws_ld, ws_off, out, accumulate);
}

namespace {

template <int NV>
int launch_ln_fwd_rows(bool vec, int phase, int rows, int cols, const float* x, int64_t ldx, const float* gamma,
                       const float* beta, float* parts, float* stats, float* y, int64_t ldy, float eps,
                       hipStream_t s) {
  dim3 grid((rows + kWaves - 1) / kWaves), block(256);
  if (vec)
    hipLaunchKernelGGL((ln_fwd_rows<NV, true>), grid, block, 0, s, phase, rows, cols, x, ldx, gamma, beta, parts,
                       stats, y, ldy, eps);
  else
    hipLaunchKernelGGL((ln_fwd_rows<NV, false>), grid, block, 0, s, phase, rows, cols, x, ldx, gamma, beta, parts,
                       stats, y, ldy, eps);
  return tt::launch_status("tile_layernorm_fwd");
}

template <int NV>
int launch_ln_bwd_rows(bool vec, int phase, int rows, int cols, float n_total, const float* dy, int64_t lddy,
                       const float* x, int64_t ldx, const float* gamma, const float* stats, float* parts,
                       int n_parts, int64_t part_stride, float* dx, int64_t lddx, int dx_acc, float* ws,
                       hipStream_t s) {
  constexpr int rpb = bwd_waves(NV) * kRowsPerWave;
  dim3 grid((rows + rpb - 1) / rpb), block(64 * bwd_waves(NV));
  if (vec)
    hipLaunchKernelGGL((ln_bwd_rows<NV, true>), grid, block, 0, s, phase, rows, cols, n_total, dy, lddy, x, ldx,
                       gamma, stats, parts, n_parts, part_stride, dx, lddx, dx_acc, ws);
  else
    hipLaunchKernelGGL((ln_bwd_rows<NV, false>), grid, block, 0, s, phase, rows, cols, n_total, dy, lddy, x, ldx,
                       gamma, stats, parts, n_parts, part_stride, dx, lddx, dx_acc, ws);
  return tt::launch_status("tile_layernorm_bwd");
}

constexpr int kMaxCols = 2048;  // 8 float4 per lane

// instantiated float4-per-lane counts and the rows one backward block covers
int nv_for(int64_t cols) {
  const int nv = (int)((cols + 255) / 256);
  return nv <= 4 ? nv : (nv <= 6 ? 6 : 8);
}
int64_t bwd_rows_per_block(int64_t cols) { return (int64_t)bwd_waves(nv_for(cols)) * kRowsPerWave; }

}  // namespace

extern "C" int tile_layernorm_fwd(void* stream, int phase, int64_t rows, int64_t cols, const float* x, int64_t ldx,
                                  const float* gamma, const float* beta, float* parts, int64_t n_parts,
                                  int64_t part_stride, float* stats, float* y, int64_t ldy, float eps) {
  using tt::fail;
  hipStream_t s = tt::as_stream(stream);
  if (rows < 0 || cols < 0) return fail(TT_ERR_ARG, "tile_layernorm_fwd: negative size");
  if (rows == 0) return TT_OK;
  if (rows > INT32_MAX) return fail(TT_ERR_ARG, "tile_layernorm_fwd: too many rows");
  if (phase == TT_LN_MERGE) {
    if (!parts || !stats || n_parts < 1) return fail(TT_ERR_ARG, "tile_layernorm_fwd(MERGE): bad argument");
    hipLaunchKernelGGL(ln_fwd_merge, dim3((rows + 255) / 256), dim3(256), 0, s, (int)rows, (int)n_parts, parts,
                       part_stride, stats, eps);
    return tt::launch_status("tile_layernorm_fwd(MERGE)");
  }
  if (cols < 1 || cols > kMaxCols) return fail(TT_ERR_SHAPE, "tile_layernorm_fwd: cols %lld not in [1, %d]",
                                               (long long)cols, kMaxCols);
  if (!x || ldx < cols) return fail(TT_ERR_ARG, "tile_layernorm_fwd: bad x");
  const bool vec = ldx % 4 == 0 && tt::aligned16(x);
  if (phase == TT_LN_APPLY) {
    if (!stats || !y || !gamma || !beta || ldy < cols) return fail(TT_ERR_ARG, "tile_layernorm_fwd(APPLY): bad argument");
    const bool v2 = vec && ldy % 4 == 0 && tt::aligned16(y) && tt::aligned16(gamma) && tt::aligned16(beta);
    dim3 grid((unsigned)((cols / 4 + 1 + 63) / 64), (unsigned)rows), block(64);
    if (v2) hipLaunchKernelGGL(ln_fwd_apply<true>, grid, block, 0, s, (int)rows, (int)cols, x, ldx, gamma, beta, stats, y, ldy);
    else hipLaunchKernelGGL(ln_fwd_apply<false>, grid, block, 0, s, (int)rows, (int)cols, x, ldx, gamma, beta, stats, y, ldy);
    return tt::launch_status("tile_layernorm_fwd(APPLY)");
  }
  if (phase == TT_LN_PARTIAL) {
    if (!parts) return fail(TT_ERR_ARG, "tile_layernorm_fwd(PARTIAL): null parts");
  } else if (phase == TT_LN_FUSED) {
    if (!stats || !y || !gamma || !beta || ldy < cols) return fail(TT_ERR_ARG, "tile_layernorm_fwd(FUSED): bad argument");
  } else {
    return fail(TT_ERR_ARG, "tile_layernorm_fwd: bad phase %d", phase);
  }
  const bool v2 = vec && (phase == TT_LN_PARTIAL ||
                          (ldy % 4 == 0 && tt::aligned16(y) && tt::aligned16(gamma) && tt::aligned16(beta)));
  const int nv = (int)((cols + 255) / 256);
  const int r = (int)rows, c = (int)cols;
  switch (nv) {
    case 1: return launch_ln_fwd_rows<1>(v2, phase, r, c, x, ldx, gamma, beta, parts, stats, y, ldy, eps, s);
    case 2: return launch_ln_fwd_rows<2>(v2, phase, r, c, x, ldx, gamma, beta, parts, stats, y, ldy, eps, s);
    case 3: return launch_ln_fwd_rows<3>(v2, phase, r, c, x, ldx, gamma, beta, parts, stats, y, ldy, eps, s);
    case 4: return launch_ln_fwd_rows<4>(v2, phase, r, c, x, ldx, gamma, beta, parts, stats, y, ldy, eps, s);
    case 5: case 6: return launch_ln_fwd_rows<6>(v2, phase, r, c, x, ldx, gamma, beta, parts, stats, y, ldy, eps, s);
    default: return launch_ln_fwd_rows<8>(v2, phase, r, c, x, ldx, gamma, beta, parts, stats, y, ldy, eps, s);
  }
}

extern "C" size_t tile_layernorm_bwd_workspace(int64_t rows, int64_t cols) {
  const int64_t rpb = bwd_rows_per_block(cols);
  const int64_t nblk = (rows + rpb - 1) / rpb;
  return (size_t)(nblk * 2 * cols * sizeof(float));
}

extern "C" int tile_layernorm_bwd(void* stream, int phase, int64_t rows, int64_t cols, int64_t n_total,
                                  const float* dy, int64_t lddy, const float* x, int64_t ldx, const float* gamma,
                                  const float* stats, float* parts, int64_t n_parts, int64_t part_stride, float* dx,
                                  int64_t lddx, int dx_acc, float* dgamma, float* dbeta, void* workspace) {
  using tt::fail;
  hipStream_t s = tt::as_stream(stream);
  if (rows < 0 || cols < 0) return fail(TT_ERR_ARG, "tile_layernorm_bwd: negative size");
  if (rows == 0) return TT_OK;
  if (rows > INT32_MAX) return fail(TT_ERR_ARG, "tile_layernorm_bwd: too many rows");
  if (cols < 1 || cols > kMaxCols) return fail(TT_ERR_SHAPE, "tile_layernorm_bwd: cols %lld not in [1, %d]",
                                               (long long)cols, kMaxCols);
  if (phase != TT_LN_PARTIAL && phase != TT_LN_APPLY && phase != TT_LN_FUSED)
    return fail(TT_ERR_ARG, "tile_layernorm_bwd: bad phase %d", phase);
  if (!dy || !x || !gamma || !stats || lddy < cols || ldx < cols) return fail(TT_ERR_ARG, "tile_layernorm_bwd: bad input");
  if (phase == TT_LN_FUSED && n_total != cols) return fail(TT_ERR_SHAPE, "tile_layernorm_bwd(FUSED): n_total != cols");
  if (n_total < cols) return fail(TT_ERR_SHAPE, "tile_layernorm_bwd: n_total < cols");
  if (phase != TT_LN_FUSED && !parts) return fail(TT_ERR_ARG, "tile_layernorm_bwd: null parts");
  if (phase == TT_LN_APPLY && n_parts < 1) return fail(TT_ERR_ARG, "tile_layernorm_bwd(APPLY): n_parts < 1");
  if (phase != TT_LN_PARTIAL && (!dx || lddx < cols || !dgamma || !dbeta || !workspace))
    return fail(TT_ERR_ARG, "tile_layernorm_bwd: bad output");
  const bool vec = lddy % 4 == 0 && ldx % 4 == 0 && tt::aligned16(dy) && tt::aligned16(x) && tt::aligned16(gamma) &&
                   (phase == TT_LN_PARTIAL || (lddx % 4 == 0 && tt::aligned16(dx)));
  const int nv = (int)((cols + 255) / 256);
  const int r = (int)rows, c = (int)cols;
  float* ws = (float*)workspace;
  int rc;
#define TT_LNB(NV)                                                                                              \
  launch_ln_bwd_rows<NV>(vec, phase, r, c, (float)n_total, dy, lddy, x, ldx, gamma, stats, parts, (int)n_parts, \
                         part_stride, dx, lddx, dx_acc, ws, s)
  switch (nv) {
    case 1: rc = TT_LNB(1); break;
    case 2: rc = TT_LNB(2); break;
    case 3: rc = TT_LNB(3); break;
    case 4: rc = TT_LNB(4); break;
    case 5: case 6: rc = TT_LNB(6); break;
    default: rc = TT_LNB(8); break;
  }
#undef TT_LNB
  if (rc || phase == TT_LN_PARTIAL) return rc;
  const int nblk = (int)((r + bwd_rows_per_block(c) - 1) / bwd_rows_per_block(c));
  dim3 grid((c + kSumCols - 1) / kSumCols, 2), block(1024);
  hipLaunchKernelGGL(colsum_finish, grid, block, 0, s, nblk, c, ws, (int64_t)2 * c, (int64_t)0, dgamma, 1, (int64_t)c,
                     dbeta);
  return tt::launch_status("tile_layernorm_bwd(colsum)");
}

// ------------------------------------------- LayerNorm over several tiles
//
// A row block whose features are split over n tiles (n >= 2, all tiles as
// wide as the first but the last, widths multiples of 4) in one pass: every
// row is read once and written once, so the forward moves 8 bytes per
// element and the backward 12 (16 when dx accumulates) -- against 12 and
// 20 for the per-tile partial / merge / apply phases, which read every tile
// twice. A workgroup of BT threads holds a whole row in registers (VPT
// float4 per thread) and takes several consecutive rows, keeping gamma and
// beta in registers across them. Sums over a row combine the lanes of each
// wave by a fixed butterfly and the waves in wave order (deterministic).

namespace {

constexpr int kLnTilesMax = 16;
struct LnRowTiles {
  const float* x[kLnTilesMax];
  const float* dy[kLnTilesMax];
  const float* g[kLnTilesMax];
  const float* b[kLnTilesMax];
  float* y[kLnTilesMax];   // forward: y; backward: dx
  float* dg[kLnTilesMax];
  float* db[kLnTilesMax];
  int n, c0, total;
};

// tile of row element `col` (a multiple of 4), its column in that tile and the tile's width
__device__ __forceinline__ int ln_tile(const LnRowTiles& P, int col, int* within, int* width) {
  int t = col / P.c0;
  if (t > P.n - 1) t = P.n - 1;
  *within = col - t * P.c0;
  *width = t < P.n - 1 ? P.c0 : P.total - (P.n - 1) * P.c0;
  return t;
}

// sum over the workgroup: waves by butterfly, then the wave sums in wave
// order by every thread (the same order everywhere)
template <int BT>
__device__ __forceinline__ void block_sum2(float& a, float& b, float (*red)[BT / 64]) {
  a = tt::wave_sum(a);
  b = tt::wave_sum(b);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    red[0][w] = a;
    red[1][w] = b;
  }
  __syncthreads();
  a = 0.f;
  b = 0.f;
#pragma unroll
  for (int i = 0; i < BT / 64; ++i) {
    a += red[0][i];
    b += red[1][i];
  }
  __syncthreads();
}

template <int BT, int VPT>
__global__ __launch_bounds__(BT) void ln_fwd_multi(int rows, int rows_per_block, LnRowTiles P,
                                                   float* __restrict__ stats, float eps) {
  __shared__ float red[2][BT / 64];
  const float* xp[VPT];
  float* yp[VPT];
  int ld[VPT];
  bool ok[VPT];
  f32x4 g[VPT], b[VPT];
#pragma unroll
  for (int k = 0; k < VPT; ++k) {
    const int col = 4 * ((int)threadIdx.x + k * BT);
    ok[k] = col < P.total;
    int w = 0, width = 4, t = 0;
    if (ok[k]) t = ln_tile(P, col, &w, &width);
    xp[k] = P.x[t] + w;
    yp[k] = P.y[t] + w;
    ld[k] = width;
    g[k] = ok[k] ? *reinterpret_cast<const f32x4*>(P.g[t] + w) : f32x4{0.f, 0.f, 0.f, 0.f};
    b[k] = ok[k] ? *reinterpret_cast<const f32x4*>(P.b[t] + w) : f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const float inv_n = 1.f / (float)P.total;
  const int r0 = blockIdx.x * rows_per_block, r1 = min(rows, r0 + rows_per_block);
  // the next row's loads are issued before this row's reductions (the
  // barriers wait for LDS only), so they overlap the compute and stores
  // x is read once: non-temporal loads (y stays a plain store: the next
  // GEMM reads it)
  f32x4 v[VPT];
#pragma unroll
  for (int k = 0; k < VPT; ++k)
    v[k] = ok[k] && r0 < r1 ? __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(xp[k] + (int64_t)r0 * ld[k]))
                            : f32x4{0.f, 0.f, 0.f, 0.f};
  for (int r = r0; r < r1; ++r) {
    f32x4 nx[VPT];
    const bool more = r + 1 < r1;
#pragma unroll
    for (int k = 0; k < VPT; ++k)
      nx[k] = ok[k] && more
                  ? __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(xp[k] + (int64_t)(r + 1) * ld[k]))
                  : f32x4{0.f, 0.f, 0.f, 0.f};
    float s = 0.f, unused = 0.f;
#pragma unroll
    for (int k = 0; k < VPT; ++k) s += (v[k][0] + v[k][1]) + (v[k][2] + v[k][3]);
    block_sum2<BT>(s, unused, red);
    const float mean = s * inv_n;
    float m2 = 0.f;
#pragma unroll
    for (int k = 0; k < VPT; ++k)
      if (ok[k]) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float d = v[k][i] - mean;
          m2 += d * d;
        }
      }
    unused = 0.f;
    block_sum2<BT>(m2, unused, red);
    const float rstd = 1.f / sqrtf(m2 * inv_n + eps);
    if (threadIdx.x == 0) {
      stats[(int64_t)r * 2] = mean;
      stats[(int64_t)r * 2 + 1] = rstd;
    }
#pragma unroll
    for (int k = 0; k < VPT; ++k)
      if (ok[k]) {
        f32x4 o;
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] = (v[k][i] - mean) * rstd * g[k][i] + b[k][i];
        *reinterpret_cast<f32x4*>(yp[k] + (int64_t)r * ld[k]) = o;
      }
#pragma unroll
    for (int k = 0; k < VPT; ++k) v[k] = nx[k];
  }
}

// dx (+)= rstd * (dxhat - mean(dxhat) - xhat * mean(dxhat * xhat)) for the
// block's rows; the block's column partials of dy*xhat and dy go to
// ws[block][2][total]
template <int BT, int VPT>
__global__ __launch_bounds__(BT) void ln_bwd_multi(int rows, int rows_per_block, LnRowTiles P,
                                                   const float* __restrict__ stats, int dx_acc, float* __restrict__ ws) {
  __shared__ float red[2][BT / 64];
  const float *xp[VPT], *dyp[VPT];
  float* dxp[VPT];
  int ld[VPT];
  bool ok[VPT];
  f32x4 g[VPT], dg[VPT], db[VPT];
#pragma unroll
  for (int k = 0; k < VPT; ++k) {
    const int col = 4 * ((int)threadIdx.x + k * BT);
    ok[k] = col < P.total;
    int w = 0, width = 4, t = 0;
    if (ok[k]) t = ln_tile(P, col, &w, &width);
    xp[k] = P.x[t] + w;
    dyp[k] = P.dy[t] + w;
    dxp[k] = P.y[t] + w;
    ld[k] = width;
    g[k] = ok[k] ? *reinterpret_cast<const f32x4*>(P.g[t] + w) : f32x4{0.f, 0.f, 0.f, 0.f};
    dg[k] = f32x4{0.f, 0.f, 0.f, 0.f};
    db[k] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const float inv_n = 1.f / (float)P.total;
  const int r0 = blockIdx.x * rows_per_block, r1 = min(rows, r0 + rows_per_block);
  for (int r = r0; r < r1; ++r) {
    const float mean = stats[(int64_t)r * 2], rstd = stats[(int64_t)r * 2 + 1];
    f32x4 xh[VPT], dxh[VPT];
    float s1 = 0.f, s2 = 0.f;
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
      f32x4 xv = f32x4{0.f, 0.f, 0.f, 0.f}, dv = xv;
      if (ok[k]) {  // x, dy and dx are each read or written once: non-temporal accesses
        xv = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(xp[k] + (int64_t)r * ld[k]));
        dv = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(dyp[k] + (int64_t)r * ld[k]));
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        xh[k][i] = ok[k] ? (xv[i] - mean) * rstd : 0.f;
        dxh[k][i] = dv[i] * g[k][i];
        s1 += dxh[k][i];
        s2 += dxh[k][i] * xh[k][i];
        dg[k][i] += dv[i] * xh[k][i];
        db[k][i] += dv[i];
      }
    }
    block_sum2<BT>(s1, s2, red);
    const float a1 = s1 * inv_n, a2 = s2 * inv_n;
#pragma unroll
    for (int k = 0; k < VPT; ++k)
      if (ok[k]) {
        float* q = dxp[k] + (int64_t)r * ld[k];
        f32x4 o;
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] = rstd * (dxh[k][i] - a1 - xh[k][i] * a2);
        if (dx_acc) o += __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(q));
        __builtin_nontemporal_store(o, reinterpret_cast<f32x4*>(q));
      }
  }
  float* out = ws + (int64_t)blockIdx.x * 2 * P.total;
#pragma unroll
  for (int k = 0; k < VPT; ++k)
    if (ok[k]) {
      const int col = 4 * ((int)threadIdx.x + k * BT);
      *reinterpret_cast<f32x4*>(out + col) = dg[k];
      *reinterpret_cast<f32x4*>(out + P.total + col) = db[k];
    }
}

// dgamma / dbeta of every tile += the column sums of the block partials,
// blockIdx.y = 2 * tile + (0: dgamma, 1: dbeta)
__global__ __launch_bounds__(1024) void ln_colsum_finish_multi(int nblk, LnRowTiles P, const float* __restrict__ ws) {
  const int t = blockIdx.y >> 1, which = blockIdx.y & 1;
  const int width = t < P.n - 1 ? P.c0 : P.total - (P.n - 1) * P.c0;
  if ((int)blockIdx.x * kSumCols >= width) return;
  colsum_finish_block(nblk, width, ws, (int64_t)2 * P.total, (int64_t)which * P.total + (int64_t)t * P.c0,
                      which ? P.db[t] : P.dg[t], 1);
}

constexpr int kLnFwdRowsPerBlock = 4;
constexpr int kLnBwdRowsPerBlock = 16;

// workgroup size and float4 per thread for a row of `total` features
void ln_multi_geometry(int64_t total, int* bt, int* vpt) {
  const int64_t f4 = total / 4;
  *bt = f4 <= 256 ? 256 : (f4 <= 512 ? 512 : 1024);
  const int v = (int)((f4 + *bt - 1) / *bt);
  *vpt = v <= 1 ? 1 : (v <= 2 ? 2 : 4);
}

// checks shared by both directions; fills the tile table's geometry
int ln_multi_check(const char* nm, int count, int64_t rows, const int64_t* cols, LnRowTiles* P) {
  using tt::fail;
  if (count < 2 || count > kLnTilesMax) return fail(TT_ERR_ARG, "%s: count must be 2..%d", nm, kLnTilesMax);
  if (rows < 0 || rows > INT32_MAX) return fail(TT_ERR_ARG, "%s: bad row count", nm);
  if (!cols) return fail(TT_ERR_ARG, "%s: null cols", nm);
  int64_t total = 0;
  for (int t = 0; t < count; ++t) {
    if (cols[t] < 4 || cols[t] % 4 || (t < count - 1 && cols[t] != cols[0]) || cols[t] > cols[0])
      return fail(TT_ERR_SHAPE, "%s: tile widths must be multiples of 4, equal but for a narrower last tile", nm);
    total += cols[t];
  }
  if (total > 16384) return fail(TT_ERR_SHAPE, "%s: %lld features exceed 16384", nm, (long long)total);
  P->n = count;
  P->c0 = (int)cols[0];
  P->total = (int)total;
  return TT_OK;
}

}  // namespace

extern "C" int tile_layernorm_fwd_multi(void* stream, int count, int64_t rows, const int64_t* cols,
                                        const float* const* x, const float* const* gamma, const float* const* beta,
                                        float* stats, float* const* y, float eps) {
  using tt::fail;
  LnRowTiles P{};
  if (int rc = ln_multi_check("tile_layernorm_fwd_multi", count, rows, cols, &P)) return rc;
  if (rows == 0) return TT_OK;
  if (!x || !gamma || !beta || !y || !stats) return fail(TT_ERR_ARG, "tile_layernorm_fwd_multi: null array");
  for (int t = 0; t < count; ++t) {
    if (!tt::aligned16(x[t]) || !tt::aligned16(y[t]) || !tt::aligned16(gamma[t]) || !tt::aligned16(beta[t]))
      return fail(TT_ERR_ARG, "tile_layernorm_fwd_multi: tile %d is null or not 16-byte aligned", t);
    P.x[t] = x[t];
    P.y[t] = y[t];
    P.g[t] = gamma[t];
    P.b[t] = beta[t];
  }
  int bt, vpt;
  ln_multi_geometry(P.total, &bt, &vpt);
  const int r = (int)rows;
  dim3 grid((unsigned)((r + kLnFwdRowsPerBlock - 1) / kLnFwdRowsPerBlock));
  hipStream_t s = tt::as_stream(stream);
#define TT_LNF(BT, VPT) hipLaunchKernelGGL((ln_fwd_multi<BT, VPT>), grid, dim3(BT), 0, s, r, kLnFwdRowsPerBlock, P, stats, eps)
  if (bt == 256) TT_LNF(256, 1);
  else if (bt == 512) TT_LNF(512, 1);
  else if (vpt == 1) TT_LNF(1024, 1);
  else if (vpt == 2) TT_LNF(1024, 2);
  else TT_LNF(1024, 4);
#undef TT_LNF
  return tt::launch_status("tile_layernorm_fwd_multi");
}

extern "C" size_t tile_layernorm_bwd_multi_workspace(int64_t rows, int64_t total) {
  const int64_t nblk = (rows + kLnBwdRowsPerBlock - 1) / kLnBwdRowsPerBlock;
  return (size_t)(nblk * 2 * total * sizeof(float));
}

extern "C" int tile_layernorm_bwd_multi(void* stream, int count, int64_t rows, const int64_t* cols,
                                        const float* const* dy, const float* const* x, const float* const* gamma,
                                        const float* stats, float* const* dx, int dx_acc, float* const* dgamma,
                                        float* const* dbeta, void* workspace, size_t workspace_bytes) {
  using tt::fail;
  LnRowTiles P{};
  if (int rc = ln_multi_check("tile_layernorm_bwd_multi", count, rows, cols, &P)) return rc;
  if (rows == 0) return TT_OK;
  if (!dy || !x || !gamma || !dx || !dgamma || !dbeta || !stats || !workspace)
    return fail(TT_ERR_ARG, "tile_layernorm_bwd_multi: null array or workspace");
  if (workspace_bytes < tile_layernorm_bwd_multi_workspace(rows, P.total) || !tt::aligned16(workspace))
    return fail(TT_ERR_ARG, "tile_layernorm_bwd_multi: workspace too small or misaligned");
  for (int t = 0; t < count; ++t) {
    if (!tt::aligned16(x[t]) || !tt::aligned16(dy[t]) || !tt::aligned16(dx[t]) || !tt::aligned16(gamma[t]) ||
        !dgamma[t] || !dbeta[t])
      return fail(TT_ERR_ARG, "tile_layernorm_bwd_multi: tile %d is null or not 16-byte aligned", t);
    P.x[t] = x[t];
    P.dy[t] = dy[t];
    P.y[t] = dx[t];
    P.g[t] = gamma[t];
    P.dg[t] = dgamma[t];
    P.db[t] = dbeta[t];
  }
  int bt, vpt;
  ln_multi_geometry(P.total, &bt, &vpt);
  const int r = (int)rows;
  const int nblk = (r + kLnBwdRowsPerBlock - 1) / kLnBwdRowsPerBlock;
  float* ws = (float*)workspace;
  hipStream_t s = tt::as_stream(stream);
#define TT_LNB(BT, VPT) \
  hipLaunchKernelGGL((ln_bwd_multi<BT, VPT>), dim3(nblk), dim3(BT), 0, s, r, kLnBwdRowsPerBlock, P, stats, dx_acc, ws)
  if (bt == 256) TT_LNB(256, 1);
  else if (bt == 512) TT_LNB(512, 1);
  else if (vpt == 1) TT_LNB(1024, 1);
  else if (vpt == 2) TT_LNB(1024, 2);
  else TT_LNB(1024, 4);
#undef TT_LNB
  if (int rc = tt::launch_status("tile_layernorm_bwd_multi")) return rc;
  hipLaunchKernelGGL(ln_colsum_finish_multi, dim3((unsigned)((P.c0 + kSumCols - 1) / kSumCols), (unsigned)(2 * count)), dim3(1024), 0,
                     s, nblk, P, ws);
  return tt::launch_status("tile_layernorm_bwd_multi(colsum)");
}

// ------------------------------------------------------------------ RMSNorm
//
// tile_rmsnorm_fwd / tile_rmsnorm_bwd: the LLaMA block's normalisation,
// y = x * rstd * g with rstd = 1 / sqrt(mean(x^2) + eps) over a row whose
// features lie in 1..16 tiles, no shift and no mean. Same geometry as the
// multi-tile LayerNorm above: a workgroup holds whole rows in registers,
// row sums combine lanes by a fixed butterfly and waves in wave order
// (deterministic); the backward writes per-block column partials of dy*n
// that a second launch sums in block order into dgamma.

namespace {

template <int BT, int VPT>
__global__ __launch_bounds__(BT) void rms_fwd_multi(int rows, int rows_per_block, LnRowTiles P,
                                                    float* __restrict__ rstd_out, float eps) {
  __shared__ float red[2][BT / 64];
  const float* xp[VPT];
  float* yp[VPT];
  int ld[VPT];
  bool ok[VPT];
  f32x4 g[VPT];
#pragma unroll
  for (int k = 0; k < VPT; ++k) {
    const int col = 4 * ((int)threadIdx.x + k * BT);
    ok[k] = col < P.total;
    int w = 0, width = 4, t = 0;
    if (ok[k]) t = ln_tile(P, col, &w, &width);
    xp[k] = P.x[t] + w;
    yp[k] = P.y[t] + w;
    ld[k] = width;
    g[k] = ok[k] ? *reinterpret_cast<const f32x4*>(P.g[t] + w) : f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const float inv_n = 1.f / (float)P.total;
  const int r0 = blockIdx.x * rows_per_block, r1 = min(rows, r0 + rows_per_block);
  f32x4 v[VPT];
#pragma unroll
  for (int k = 0; k < VPT; ++k)
    v[k] = ok[k] && r0 < r1 ? __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(xp[k] + (int64_t)r0 * ld[k]))
                            : f32x4{0.f, 0.f, 0.f, 0.f};
  for (int r = r0; r < r1; ++r) {
    f32x4 nx[VPT];
    const bool more = r + 1 < r1;
#pragma unroll
    for (int k = 0; k < VPT; ++k)
      nx[k] = ok[k] && more
                  ? __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(xp[k] + (int64_t)(r + 1) * ld[k]))
                  : f32x4{0.f, 0.f, 0.f, 0.f};
    float s = 0.f, unused = 0.f;
#pragma unroll
    for (int k = 0; k < VPT; ++k) s += (v[k][0] * v[k][0] + v[k][1] * v[k][1]) + (v[k][2] * v[k][2] + v[k][3] * v[k][3]);
    block_sum2<BT>(s, unused, red);
    const float rstd = 1.f / sqrtf(s * inv_n + eps);
    if (threadIdx.x == 0) rstd_out[r] = rstd;
#pragma unroll
    for (int k = 0; k < VPT; ++k)
      if (ok[k]) {
        f32x4 o;
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] = v[k][i] * rstd * g[k][i];
        *reinterpret_cast<f32x4*>(yp[k] + (int64_t)r * ld[k]) = o;
      }
#pragma unroll
    for (int k = 0; k < VPT; ++k) v[k] = nx[k];
  }
}

// dx (+)= rstd * (dn - n * mean(dn * n)) with n = x * rstd, dn = dy * g; the
// block's column partials of dy * n go to ws[block][total]
template <int BT, int VPT>
__global__ __launch_bounds__(BT) void rms_bwd_multi(int rows, int rows_per_block, LnRowTiles P,
                                                    const float* __restrict__ rstd_in, int dx_acc,
                                                    float* __restrict__ ws) {
  __shared__ float red[2][BT / 64];
  const float *xp[VPT], *dyp[VPT];
  float* dxp[VPT];
  int ld[VPT];
  bool ok[VPT];
  f32x4 g[VPT], dg[VPT];
#pragma unroll
  for (int k = 0; k < VPT; ++k) {
    const int col = 4 * ((int)threadIdx.x + k * BT);
    ok[k] = col < P.total;
    int w = 0, width = 4, t = 0;
    if (ok[k]) t = ln_tile(P, col, &w, &width);
    xp[k] = P.x[t] + w;
    dyp[k] = P.dy[t] + w;
    dxp[k] = P.y[t] + w;
    ld[k] = width;
    g[k] = ok[k] ? *reinterpret_cast<const f32x4*>(P.g[t] + w) : f32x4{0.f, 0.f, 0.f, 0.f};
    dg[k] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const float inv_n = 1.f / (float)P.total;
  const int r0 = blockIdx.x * rows_per_block, r1 = min(rows, r0 + rows_per_block);
  for (int r = r0; r < r1; ++r) {
    const float rstd = rstd_in[r];
    f32x4 n[VPT], dn[VPT];
    float s = 0.f, unused = 0.f;
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
      f32x4 xv = f32x4{0.f, 0.f, 0.f, 0.f}, dv = xv;
      if (ok[k]) {
        xv = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(xp[k] + (int64_t)r * ld[k]));
        dv = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(dyp[k] + (int64_t)r * ld[k]));
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        n[k][i] = xv[i] * rstd;
        dn[k][i] = dv[i] * g[k][i];
        s += dn[k][i] * n[k][i];
        dg[k][i] += dv[i] * n[k][i];
      }
    }
    block_sum2<BT>(s, unused, red);
    const float a = s * inv_n;
#pragma unroll
    for (int k = 0; k < VPT; ++k)
      if (ok[k]) {
        float* q = dxp[k] + (int64_t)r * ld[k];
        f32x4 o;
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] = rstd * (dn[k][i] - n[k][i] * a);
        if (dx_acc) o += __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(q));
        __builtin_nontemporal_store(o, reinterpret_cast<f32x4*>(q));
      }
  }
  float* out = ws + (int64_t)blockIdx.x * P.total;
#pragma unroll
  for (int k = 0; k < VPT; ++k)
    if (ok[k]) *reinterpret_cast<f32x4*>(out + 4 * ((int)threadIdx.x + k * BT)) = dg[k];
}

// dgamma of every tile += the column sums of the block partials (blockIdx.y = tile)
__global__ __launch_bounds__(1024) void rms_colsum_finish_multi(int nblk, LnRowTiles P, const float* __restrict__ ws) {
  const int t = blockIdx.y;
  const int width = t < P.n - 1 ? P.c0 : P.total - (P.n - 1) * P.c0;
  if ((int)blockIdx.x * kSumCols >= width) return;
  colsum_finish_block(nblk, width, ws, (int64_t)P.total, (int64_t)t * P.c0, P.dg[t], 1);
}

// rows per backward workgroup: up to 16 (fewer column partials to sum), but
// at least ~1024 workgroups when the rows allow (a 4096-row block of 768
// features on 16 rows per workgroup makes 256 workgroups, one per CU:
// 20 % of HBM)
constexpr int kRmsBwdRowsPerBlock = 16;
int rms_bwd_rows_per_block(int64_t rows) {
  return (int)std::max<int64_t>(1, std::min<int64_t>(kRmsBwdRowsPerBlock, rows / 1024));
}

// like ln_multi_check, one tile allowed
int rms_check(const char* nm, int count, int64_t rows, const int64_t* cols, LnRowTiles* P) {
  using tt::fail;
  if (count < 1 || count > kLnTilesMax) return fail(TT_ERR_ARG, "%s: count must be 1..%d", nm, kLnTilesMax);
  if (rows < 0 || rows > INT32_MAX) return fail(TT_ERR_ARG, "%s: bad row count", nm);
  if (!cols) return fail(TT_ERR_ARG, "%s: null cols", nm);
  int64_t total = 0;
  for (int t = 0; t < count; ++t) {
    if (cols[t] < 4 || cols[t] % 4 || (t < count - 1 && cols[t] != cols[0]) || cols[t] > cols[0])
      return fail(TT_ERR_SHAPE, "%s: tile widths must be multiples of 4, equal but for a narrower last tile", nm);
    total += cols[t];
  }
  if (total > 16384) return fail(TT_ERR_SHAPE, "%s: %lld features exceed 16384", nm, (long long)total);
  P->n = count;
  P->c0 = (int)cols[0];
  P->total = (int)total;
  return TT_OK;
}

}  // namespace

extern "C" int tile_rmsnorm_fwd(void* stream, int count, int64_t rows, const int64_t* cols, const float* const* x,
                                const float* const* gamma, float* rstd, float* const* y, float eps) {
  using tt::fail;
  LnRowTiles P{};
  if (int rc = rms_check("tile_rmsnorm_fwd", count, rows, cols, &P)) return rc;
  if (rows == 0) return TT_OK;
  if (!x || !gamma || !y || !rstd) return fail(TT_ERR_ARG, "tile_rmsnorm_fwd: null array");
  for (int t = 0; t < count; ++t) {
    if (!tt::aligned16(x[t]) || !tt::aligned16(y[t]) || !tt::aligned16(gamma[t]) || !x[t] || !y[t] || !gamma[t])
      return fail(TT_ERR_ARG, "tile_rmsnorm_fwd: tile %d is null or not 16-byte aligned", t);
    P.x[t] = x[t];
    P.y[t] = y[t];
    P.g[t] = gamma[t];
  }
  int bt, vpt;
  ln_multi_geometry(P.total, &bt, &vpt);
  const int r = (int)rows;
  dim3 grid((unsigned)((r + kLnFwdRowsPerBlock - 1) / kLnFwdRowsPerBlock));
  hipStream_t s = tt::as_stream(stream);
#define TT_RMSF(BT, VPT) \
  hipLaunchKernelGGL((rms_fwd_multi<BT, VPT>), grid, dim3(BT), 0, s, r, kLnFwdRowsPerBlock, P, rstd, eps)
  if (bt == 256) TT_RMSF(256, 1);
  else if (bt == 512) TT_RMSF(512, 1);
  else if (vpt == 1) TT_RMSF(1024, 1);
  else if (vpt == 2) TT_RMSF(1024, 2);
  else TT_RMSF(1024, 4);
#undef TT_RMSF
  return tt::launch_status("tile_rmsnorm_fwd");
}

extern "C" size_t tile_rmsnorm_bwd_workspace(int64_t rows, int64_t total) {
  if (rows < 0 || total < 0) return 0;
  const int rpb = rms_bwd_rows_per_block(rows);
  const int64_t nblk = (rows + rpb - 1) / rpb;
  return (size_t)(nblk * total * sizeof(float));
}

extern "C" int tile_rmsnorm_bwd(void* stream, int count, int64_t rows, const int64_t* cols, const float* const* dy,
                                const float* const* x, const float* const* gamma, const float* rstd,
                                float* const* dx, int dx_acc, float* const* dgamma, void* workspace,
                                size_t workspace_bytes) {
  using tt::fail;
  LnRowTiles P{};
  if (int rc = rms_check("tile_rmsnorm_bwd", count, rows, cols, &P)) return rc;
  if (rows == 0) return TT_OK;
  if (!dy || !x || !gamma || !dx || !dgamma || !rstd || !workspace)
    return fail(TT_ERR_ARG, "tile_rmsnorm_bwd: null array or workspace");
  if (workspace_bytes < tile_rmsnorm_bwd_workspace(rows, P.total) || !tt::aligned16(workspace))
    return fail(TT_ERR_ARG, "tile_rmsnorm_bwd: workspace too small or misaligned");
  for (int t = 0; t < count; ++t) {
    if (!x[t] || !dy[t] || !dx[t] || !gamma[t] || !dgamma[t] || !tt::aligned16(x[t]) || !tt::aligned16(dy[t]) ||
        !tt::aligned16(dx[t]) || !tt::aligned16(gamma[t]))
      return fail(TT_ERR_ARG, "tile_rmsnorm_bwd: tile %d is null or not 16-byte aligned", t);
    P.x[t] = x[t];
    P.dy[t] = dy[t];
    P.y[t] = dx[t];
    P.g[t] = gamma[t];
    P.dg[t] = dgamma[t];
  }
  int bt, vpt;
  ln_multi_geometry(P.total, &bt, &vpt);
  const int r = (int)rows;
  const int rpb = rms_bwd_rows_per_block(rows);
  const int nblk = (r + rpb - 1) / rpb;
  float* ws = (float*)workspace;
  hipStream_t s = tt::as_stream(stream);
#define TT_RMSB(BT, VPT) \
  hipLaunchKernelGGL((rms_bwd_multi<BT, VPT>), dim3(nblk), dim3(BT), 0, s, r, rpb, P, rstd, dx_acc, ws)
  if (bt == 256) TT_RMSB(256, 1);
  else if (bt == 512) TT_RMSB(512, 1);
  else if (vpt == 1) TT_RMSB(1024, 1);
  else if (vpt == 2) TT_RMSB(1024, 2);
  else TT_RMSB(1024, 4);
#undef TT_RMSB
  if (int rc = tt::launch_status("tile_rmsnorm_bwd")) return rc;
  hipLaunchKernelGGL(rms_colsum_finish_multi, dim3((unsigned)((P.c0 + kSumCols - 1) / kSumCols), (unsigned)count),
                     dim3(1024), 0, s, nblk, P, ws);
  return tt::launch_status("tile_rmsnorm_bwd(colsum)");
}

// ------------------------------------ LayerNorm backward without allocation
//
// tile_layernorm_bwd_noalloc: tile_layernorm_bwd with its column-sum
// partials in a file-scope device array instead of a caller workspace, for
// callers that may not allocate (graph capture, serving loops). Each device
// holds its own copy of the array; its address is looked up once per
// device with hipGetSymbolAddress and kept -- the array's name in host code
// is not a device address. Every call on one device shares the array, so
// calls that overlap on a device (two streams at once) race; the partials
// are written in full by each call before they are read, so nothing needs
// clearing between calls.

namespace {

constexpr size_t kLnScratchBytes = size_t(16) << 20;  // 16 MiB per device
__device__ __align__(256) unsigned char scratch[kLnScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

int scratch_for_current_device(void** out) {
  int dev = 0;
  TT_HIP_TRY(hipGetDevice(&dev));
  if (dev < 0 || dev >= kMaxDevices) return tt::fail(TT_ERR_ARG, "layernorm scratch: device %d out of range", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      return tt::fail(TT_ERR_HIP, "layernorm scratch: hipGetSymbolAddress failed: %s", hipGetErrorString(e));
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return TT_OK;
}

}  // namespace

extern "C" size_t tile_layernorm_bwd_noalloc_max_bytes(void) { return kLnScratchBytes; }

extern "C" int tile_layernorm_bwd_noalloc(void* stream, int phase, int64_t rows, int64_t cols, int64_t n_total,
                                          const float* dy, int64_t lddy, const float* x, int64_t ldx,
                                          const float* gamma, const float* stats, float* parts, int64_t n_parts,
                                          int64_t part_stride, float* dx, int64_t lddx, int dx_acc, float* dgamma,
                                          float* dbeta) {
  if (rows < 0 || cols < 0) return tt::fail(TT_ERR_ARG, "tile_layernorm_bwd_noalloc: negative size");
  if (phase != TT_LN_PARTIAL && rows > 0 && cols > 0 &&
      tile_layernorm_bwd_workspace(rows, cols) > kLnScratchBytes)
    return tt::fail(TT_ERR_ARG,
                    "tile_layernorm_bwd_noalloc: %lld rows x %lld columns need %zu bytes of column partials, above "
                    "the %zu-byte scratch array",
                    (long long)rows, (long long)cols, tile_layernorm_bwd_workspace(rows, cols), kLnScratchBytes);
  void* ws = nullptr;
  if (int rc = scratch_for_current_device(&ws)) return rc;
  return tile_layernorm_bwd(stream, phase, rows, cols, n_total, dy, lddy, x, ldx, gamma, stats, parts, n_parts,
                            part_stride, dx, lddx, dx_acc, dgamma, dbeta, ws);
}

// ------------------------------------------------------------ reduce_rows

namespace {
constexpr int kReduceRows = 64;  // rows per stage-1 block

template <bool VEC>
__device__ __forceinline__ void reduce_rows_block(int rows, int cols, const float* __restrict__ X, int64_t ldx,
                                                  float* __restrict__ ws) {
  __shared__ f32x4 red[4][64];
  const int cl = threadIdx.x & 63, grp = threadIdx.x >> 6;
  const int c = (blockIdx.y * 64 + cl) * 4;
  const int r0 = blockIdx.x * kReduceRows + grp * (kReduceRows / 4);
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  if (c < cols) {
    // all loads of the thread's rows in flight before the (ordered) sum
    constexpr int R = kReduceRows / 4;
    f32x4 v[R];
#pragma unroll
    for (int q = 0; q < R; ++q)
      v[q] = r0 + q < rows ? tt::ld4_nt<VEC>(X, ldx, r0 + q, c, cols) : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int q = 0; q < R; ++q) acc += v[q];
  }
  red[grp][cl] = acc;
  __syncthreads();
  if (grp == 0 && c < cols) {
    f32x4 t = red[0][cl];
#pragma unroll
    for (int g = 1; g < 4; ++g) t += red[g][cl];
    float* out = ws + (int64_t)blockIdx.x * cols;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (c + i < cols) out[c + i] = t[i];
  }
}

template <bool VEC>
__global__ __launch_bounds__(256) void reduce_rows_stage1(int rows, int cols, const float* __restrict__ X,
                                                          int64_t ldx, float* __restrict__ ws) {
  reduce_rows_block<VEC>(rows, cols, X, ldx, ws);
}

// several tiles of one row count per launch (the attention block's q, k
// and v bias gradients): tile t in blockIdx.z (stage 1) / blockIdx.y
// (finish), its partial rows in its own workspace region
constexpr int kRowsMax = 16;
struct RowsTiles {
  const float* X[kRowsMax];
  float* out[kRowsMax];
  int64_t ldx[kRowsMax];
  int64_t ws_off[kRowsMax];
  int cols[kRowsMax];
};

template <bool VEC>
__global__ __launch_bounds__(256) void reduce_rows_stage1_multi(int rows, RowsTiles P, float* __restrict__ ws) {
  const int t = blockIdx.z;
  if ((int)blockIdx.y * 256 >= P.cols[t]) return;  // whole workgroup past this tile's columns
  reduce_rows_block<VEC>(rows, P.cols[t], P.X[t], P.ldx[t], ws + P.ws_off[t]);
}

__global__ __launch_bounds__(1024) void colsum_finish_multi(int nblk, RowsTiles P, const float* __restrict__ ws,
                                                            int accumulate) {
  const int t = blockIdx.y;
  if ((int)blockIdx.x * kSumCols >= P.cols[t]) return;
  colsum_finish_block(nblk, P.cols[t], ws, P.cols[t], P.ws_off[t], P.out[t], accumulate);
}
}  // namespace

extern "C" size_t tile_reduce_rows_workspace(int64_t rows, int64_t cols) {
  return (size_t)(((rows + kReduceRows - 1) / kReduceRows) * cols * sizeof(float));
}

extern "C" int tile_reduce_rows(void* stream, int64_t rows, int64_t cols, const float* X, int64_t ldx, float* out,
                                int beta, void* workspace) {
  using tt::fail;
  hipStream_t s = tt::as_stream(stream);
  if (rows < 0 || cols < 0) return fail(TT_ERR_ARG, "tile_reduce_rows: negative size");
  if (cols == 0) return TT_OK;
  if (!out || !workspace) return fail(TT_ERR_ARG, "tile_reduce_rows: null output/workspace");
  if (rows > INT32_MAX || cols > INT32_MAX) return fail(TT_ERR_ARG, "tile_reduce_rows: size exceeds int32");
  const int r = (int)rows, c = (int)cols;
  const int nblk = (r + kReduceRows - 1) / kReduceRows;
  float* ws = (float*)workspace;
  if (rows > 0) {
    if (!X || ldx < cols) return fail(TT_ERR_ARG, "tile_reduce_rows: bad X");
    dim3 grid(nblk, (c + 255) / 256), block(256);
    if (ldx % 4 == 0 && tt::aligned16(X)) hipLaunchKernelGGL(reduce_rows_stage1<true>, grid, block, 0, s, r, c, X, ldx, ws);
    else hipLaunchKernelGGL(reduce_rows_stage1<false>, grid, block, 0, s, r, c, X, ldx, ws);
    if (int rc = tt::launch_status("tile_reduce_rows")) return rc;
  }
  hipLaunchKernelGGL(colsum_finish, dim3((c + kSumCols - 1) / kSumCols), dim3(1024), 0, s, nblk, c, ws, (int64_t)c, (int64_t)0, out,
                     beta, (int64_t)0, out);
  return tt::launch_status("tile_reduce_rows(finish)");
}

extern "C" int tile_reduce_rows_multi(void* stream, int count, int64_t rows, const int64_t* cols, const float* const* X,
                                      const int64_t* ldx, float* const* out, int beta, void* workspace,
                                      size_t workspace_bytes) {
  using tt::fail;
  hipStream_t s = tt::as_stream(stream);
  if (count < 0 || rows < 0) return fail(TT_ERR_ARG, "tile_reduce_rows_multi: negative count or size");
  if (count == 0) return TT_OK;
  if (count > kRowsMax) return fail(TT_ERR_ARG, "tile_reduce_rows_multi: more than %d tiles", kRowsMax);
  if (!cols || !out || (rows > 0 && (!X || !ldx)) || !workspace)
    return fail(TT_ERR_ARG, "tile_reduce_rows_multi: null array or workspace");
  if (rows > INT32_MAX) return fail(TT_ERR_ARG, "tile_reduce_rows_multi: size exceeds int32");
  const int r = (int)rows;
  const int nblk = (r + kReduceRows - 1) / kReduceRows;
  RowsTiles P{};
  int64_t off = 0, maxc = 0;
  bool vec = true;
  for (int t = 0; t < count; ++t) {
    if (cols[t] < 1 || cols[t] > INT32_MAX || !out[t]) return fail(TT_ERR_ARG, "tile_reduce_rows_multi: bad tile %d", t);
    if (rows > 0 && (!X[t] || ldx[t] < cols[t])) return fail(TT_ERR_ARG, "tile_reduce_rows_multi: bad X of tile %d", t);
    P.X[t] = rows > 0 ? X[t] : nullptr;
    P.ldx[t] = rows > 0 ? ldx[t] : 0;
    P.out[t] = out[t];
    P.cols[t] = (int)cols[t];
    P.ws_off[t] = off;
    off += (int64_t)std::max(nblk, 1) * cols[t];
    maxc = std::max(maxc, cols[t]);
    if (rows > 0) vec = vec && ldx[t] % 4 == 0 && tt::aligned16(X[t]);
  }
  if ((size_t)off * sizeof(float) > workspace_bytes) return fail(TT_ERR_ARG, "tile_reduce_rows_multi: workspace too small");
  float* ws = (float*)workspace;
  if (rows > 0) {
    dim3 grid(nblk, (unsigned)((maxc + 255) / 256), count), block(256);
    if (vec) hipLaunchKernelGGL(reduce_rows_stage1_multi<true>, grid, block, 0, s, r, P, ws);
    else hipLaunchKernelGGL(reduce_rows_stage1_multi<false>, grid, block, 0, s, r, P, ws);
    if (int rc = tt::launch_status("tile_reduce_rows_multi")) return rc;
  }
  hipLaunchKernelGGL(colsum_finish_multi, dim3((unsigned)((maxc + kSumCols - 1) / kSumCols), count), dim3(1024), 0, s, nblk, P, ws,
                     beta);
  return tt::launch_status("tile_reduce_rows_multi(finish)");
}
