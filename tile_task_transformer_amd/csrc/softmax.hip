// Row softmax and cross-entropy tile tasks.
//
// The tied LM head's logits are split into vocab tiles, so the softmax over
// a row is assembled from per-tile partials (row max, sum of exp(x - max))
// merged by rescaling to the larger max. The same per-tile pass picks the
// target logit when a row's label falls in the tile, so the loss needs no
// extra read of the logits. All kernels are HBM-bound row sweeps: one wave
// per row, the row held in registers between its max and sum passes.
#include "rowops.hpp"

using tt::f32x4;

namespace {

constexpr int kWaves = 4;

// exp(d) as the hardware 2^x of d * log2(e): two instructions per element
// instead of the library expf's range reduction (the sweeps over the
// logits were limited by that arithmetic, not by HBM); the product's
// rounding adds |d| * 2^-24 relative error, 2e-6 for a logit 30 below the
// row maximum, far inside the loss and gradient tolerances
__device__ __forceinline__ float exp_hw(float d) { return __builtin_amdgcn_exp2f(d * 1.4426950408889634f); }

// (max, sum exp(x - max), picked target) of one row of one tile, by one wave
template <int NV, bool VEC>
__device__ __forceinline__ void stats_row(int row, int cols, int64_t row_off, int64_t col_off, float scale,
                                          int causal, const float* __restrict__ X, int64_t ldx,
                                          const int32_t* __restrict__ labels, float* __restrict__ parts) {
  const int lane = threadIdx.x & 63;
  // valid columns of this row: c < lim
  int lim = cols;
  if (causal) {
    const int64_t l = row_off + row - col_off + 1;
    lim = (int)max((int64_t)0, min((int64_t)cols, l));
  }
  f32x4 v[NV];
  float mx = -INFINITY;
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const int c = (j * 64 + lane) * 4;
    v[j] = c < cols ? tt::ld4<VEC>(X, ldx, row, c, cols) : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[j][i] = c + i < lim ? v[j][i] * scale : -INFINITY;
      mx = fmaxf(mx, v[j][i]);
    }
  }
  mx = tt::wave_max(mx);
  float se = 0.f;
  if (mx > -INFINITY) {
#pragma unroll
    for (int j = 0; j < NV; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) se += exp_hw(v[j][i] - mx);
  }
  se = tt::wave_sum(se);
  if (lane == 0) {
    float picked = 0.f;
    if (labels) {
      const int64_t lab = labels[row] - col_off;
      if (lab >= 0 && lab < lim) picked = X[(int64_t)row * ldx + lab] * scale;
    }
    parts[(int64_t)row * 3 + 0] = mx;
    parts[(int64_t)row * 3 + 1] = se;
    parts[(int64_t)row * 3 + 2] = picked;
  }
}

template <int NV, bool VEC>
__global__ __launch_bounds__(256) void sm_stats(int rows, int cols, int64_t row_off, int64_t col_off, float scale,
                                                int causal, const float* __restrict__ X, int64_t ldx,
                                                const int32_t* __restrict__ labels, float* __restrict__ parts) {
  const int row = blockIdx.x * kWaves + (threadIdx.x >> 6);
  if (row >= rows) return;
  stats_row<NV, VEC>(row, cols, row_off, col_off, scale, causal, X, ldx, labels, parts);
}

// several vocab tiles of one token tile per launch (blockIdx.y = tile)
constexpr int kXeMax = 64;
struct XeTiles {
  float* z[kXeMax];
  int64_t ld[kXeMax];
  int64_t off[kXeMax];
  int cols[kXeMax];
  int part[kXeMax];  // index of the tile's partials (position in the caller's list)
};

template <int NV, bool VEC>
__global__ __launch_bounds__(256) void xe_stats_multi(int rows, XeTiles P, const int32_t* __restrict__ labels,
                                                      float* __restrict__ parts, int64_t part_stride) {
  const int row = blockIdx.x * kWaves + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int t = blockIdx.y;
  stats_row<NV, VEC>(row, P.cols[t], 0, P.off[t], 1.f, 0, P.z[t], P.ld[t], labels, parts + P.part[t] * part_stride);
}

// lse from many (max, sum exp, picked) partials: the 64-column groups of
// the LM head's statistics epilogue. One wave per row; lane l merges the
// partials l, l + 64, ... of the (tile, group) list in order, then the lanes
// combine along a fixed xor tree (each step is commutative, so every lane
// holds the same result and the order is the same on every run).
constexpr int kMergeMaxTiles = 256;
struct GroupList {
  int first[kMergeMaxTiles + 1];  // first[t] = partials before tile t
};

__device__ __forceinline__ void merge3(float& m, float& s, float& p, float mb, float sb, float pb) {
  const float mn = fmaxf(m, mb);
  if (mn > -INFINITY) s = (m > -INFINITY ? s * expf(m - mn) : 0.f) + (mb > -INFINITY ? sb * expf(mb - mn) : 0.f);
  m = mn;
  p += pb;
}

__global__ __launch_bounds__(256) void xe_merge_groups(int rows, int count, GroupList G,
                                                       const float* __restrict__ parts, int64_t stride,
                                                       float* __restrict__ lse, float* __restrict__ row_loss) {
  const int row = blockIdx.x * kWaves + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (row >= rows) return;
  const int total = G.first[count];
  float m = -INFINITY, sm = 0.f, pk = 0.f;
  int t = 0;
  for (int p = lane; p < total; p += 64) {
    while (G.first[t + 1] <= p) ++t;
    const float* q = parts + t * stride + ((int64_t)(p - G.first[t]) * rows + row) * 3;
    merge3(m, sm, pk, q[0], q[1], q[2]);
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const float mb = __shfl_xor(m, o, 64), sb = __shfl_xor(sm, o, 64), pb = __shfl_xor(pk, o, 64);
    merge3(m, sm, pk, mb, sb, pb);
  }
  if (lane == 0) {
    const float l = m + logf(sm);
    lse[row] = l;
    if (row_loss) row_loss[row] = l - pk;
  }
}

__global__ void sm_merge(int rows, int n_parts, const float* __restrict__ parts, int64_t stride,
                         float* __restrict__ lse, float* __restrict__ row_loss) {
  const int row = blockIdx.x * blockDim.x + threadIdx.x;
  if (row >= rows) return;
  float m = -INFINITY, s = 0.f, picked = 0.f;
  for (int p = 0; p < n_parts; ++p) {
    const float* q = parts + p * stride + (int64_t)row * 3;
    const float mb = q[0], sb = q[1];
    picked += q[2];
    const float mn = fmaxf(m, mb);
    if (mn > -INFINITY) s = (m > -INFINITY ? s * expf(m - mn) : 0.f) + (mb > -INFINITY ? sb * expf(mb - mn) : 0.f);
    m = mn;
  }
  const float l = m + logf(s);
  lse[row] = l;
  if (row_loss) row_loss[row] = l - picked;
}

// 4 columns c..c+3 of one row: (exp(x * scale - lse) - onehot) * grad_scale
template <bool VEC>
__device__ __forceinline__ void apply4(int row, int c, int cols, int64_t row_off, int64_t col_off, float scale,
                                       int causal, const float* X, int64_t ldx, const int32_t* __restrict__ labels,
                                       const float* __restrict__ lse, float* Y, int64_t ldy, float grad_scale) {
  const float l = lse[row];
  const int64_t lab = labels ? labels[row] - col_off : -1;
  const int64_t lim = causal ? row_off + row - col_off + 1 : (int64_t)cols;
  const f32x4 x = tt::ld4<VEC>(X, ldx, row, c, cols);
  f32x4 y;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float p = (c + i < lim) ? exp_hw(x[i] * scale - l) : 0.f;
    if (c + i == lab) p -= 1.f;
    y[i] = p * grad_scale;
  }
  tt::st4<VEC>(Y, ldy, row, c, cols, y);
}

template <bool VEC>
__global__ void sm_apply(int rows, int cols, int64_t row_off, int64_t col_off, float scale, int causal,
                         const float* X, int64_t ldx, const int32_t* __restrict__ labels,
                         const float* __restrict__ lse, float* Y, int64_t ldy, float grad_scale) {
  const int c = (blockIdx.x * blockDim.x + threadIdx.x) * 4;
  const int row = blockIdx.y;
  if (c >= cols) return;
  apply4<VEC>(row, c, cols, row_off, col_off, scale, causal, X, ldx, labels, lse, Y, ldy, grad_scale);
}

// The gradient sweep over a vocab tile (rows x cols, row-major, ld == cols:
// one contiguous array) as a flat float4 stream, grid-stride, with
// non-temporal loads and stores (each element is read and written once);
// blockIdx.y = tile. Same per-element arithmetic as apply4.
__global__ __launch_bounds__(256) void xe_grad_multi(int rows, XeTiles P, const int32_t* __restrict__ labels,
                                                     const float* __restrict__ lse, float inv_n) {
  const int t = blockIdx.y, cols = P.cols[t];
  f32x4* z = reinterpret_cast<f32x4*>(P.z[t]);
  const int64_t n4 = (int64_t)rows * cols / 4;
  for (int64_t e = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; e < n4; e += (int64_t)gridDim.x * blockDim.x) {
    const f32x4 x = __builtin_nontemporal_load(z + e);
    const int idx = (int)(e * 4);  // rows * cols < 2^31 (rows <= 65535, cols <= 2048)
    const int row = idx / cols, c = idx - row * cols;
    const float l = lse[row];
    const int64_t lab = labels[row] - P.off[t];
    f32x4 y;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float p = exp_hw(x[i] - l);
      if (c + i == lab) p -= 1.f;
      y[i] = p * inv_n;
    }
    __builtin_nontemporal_store(y, z + e);
  }
}

__global__ __launch_bounds__(256) void xe_loss(int rows, const float* __restrict__ row_loss, float* loss,
                                               int accumulate, float inv_n) {
  __shared__ float red[256];
  float s = 0.f;
  for (int r = threadIdx.x; r < rows; r += 256) s += row_loss[r];
  red[threadIdx.x] = s;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if ((int)threadIdx.x < o) red[threadIdx.x] += red[threadIdx.x + o];
    __syncthreads();
  }
  if (threadIdx.x == 0) loss[0] = (accumulate ? loss[0] : 0.f) + inv_n * red[0];
}

template <int NV>
int launch_stats(bool vec, int rows, int cols, int64_t row_off, int64_t col_off, float scale, int causal,
                 const float* X, int64_t ldx, const int32_t* labels, float* parts, hipStream_t s) {
  dim3 grid((rows + kWaves - 1) / kWaves), block(256);
  if (vec)
    hipLaunchKernelGGL((sm_stats<NV, true>), grid, block, 0, s, rows, cols, row_off, col_off, scale, causal, X, ldx,
                       labels, parts);
  else
    hipLaunchKernelGGL((sm_stats<NV, false>), grid, block, 0, s, rows, cols, row_off, col_off, scale, causal, X, ldx,
                       labels, parts);
  return tt::launch_status("tile_softmax(STATS)");
}

int launch_apply(int rows, int cols, int64_t row_off, int64_t col_off, float scale, int causal, const float* X,
                 int64_t ldx, const int32_t* labels, const float* lse, float* Y, int64_t ldy, float grad_scale,
                 hipStream_t s) {
  const bool vec = ldx % 4 == 0 && ldy % 4 == 0 && tt::aligned16(X) && tt::aligned16(Y);
  dim3 grid((unsigned)(((cols + 3) / 4 + 255) / 256), (unsigned)rows), block(256);
  if (vec)
    hipLaunchKernelGGL(sm_apply<true>, grid, block, 0, s, rows, cols, row_off, col_off, scale, causal, X, ldx, labels,
                       lse, Y, ldy, grad_scale);
  else
    hipLaunchKernelGGL(sm_apply<false>, grid, block, 0, s, rows, cols, row_off, col_off, scale, causal, X, ldx, labels,
                       lse, Y, ldy, grad_scale);
  return tt::launch_status("tile_softmax(APPLY)");
}

constexpr int kMaxCols = 2048;
constexpr int64_t kMaxRows = 65535;

template <int NV>
void launch_stats_multi(bool vec, int rows, int count, const XeTiles& P, const int32_t* labels, float* parts,
                        int64_t part_stride, hipStream_t s) {
  dim3 grid((unsigned)((rows + kWaves - 1) / kWaves), (unsigned)count), block(256);
  if (vec) hipLaunchKernelGGL((xe_stats_multi<NV, true>), grid, block, 0, s, rows, P, labels, parts, part_stride);
  else hipLaunchKernelGGL((xe_stats_multi<NV, false>), grid, block, 0, s, rows, P, labels, parts, part_stride);
}

}  // namespace

extern "C" int tile_softmax(void* stream, int phase, int64_t rows, int64_t cols, int64_t row_offset,
                            int64_t col_offset, float scale, int causal, const float* X, int64_t ldx,
                            const int32_t* labels, float* parts, int64_t n_parts, int64_t part_stride, float* lse,
                            float* row_loss, float* Y, int64_t ldy, float grad_scale) {
  using tt::fail;
  hipStream_t s = tt::as_stream(stream);
  if (rows < 0 || cols < 0) return fail(TT_ERR_ARG, "tile_softmax: negative size");
  if (rows == 0) return TT_OK;
  if (phase == TT_SM_MERGE) {
    if (!parts || !lse || n_parts < 1 || rows > INT32_MAX) return fail(TT_ERR_ARG, "tile_softmax(MERGE): bad argument");
    hipLaunchKernelGGL(sm_merge, dim3((unsigned)((rows + 255) / 256)), dim3(256), 0, s, (int)rows, (int)n_parts, parts,
                       part_stride, lse, row_loss);
    return tt::launch_status("tile_softmax(MERGE)");
  }
  if (cols < 1 || cols > kMaxCols) return fail(TT_ERR_SHAPE, "tile_softmax: cols %lld not in [1, %d]", (long long)cols, kMaxCols);
  if (rows > kMaxRows) return fail(TT_ERR_SHAPE, "tile_softmax: rows %lld > %lld", (long long)rows, (long long)kMaxRows);
  if (!X || ldx < cols) return fail(TT_ERR_ARG, "tile_softmax: bad X");
  if (phase == TT_SM_STATS) {
    if (!parts) return fail(TT_ERR_ARG, "tile_softmax(STATS): null parts");
    const bool vec = ldx % 4 == 0 && tt::aligned16(X);
    const int nv = (int)((cols + 255) / 256);
    const int r = (int)rows, c = (int)cols;
    switch (nv) {
      case 1: return launch_stats<1>(vec, r, c, row_offset, col_offset, scale, causal, X, ldx, labels, parts, s);
      case 2: return launch_stats<2>(vec, r, c, row_offset, col_offset, scale, causal, X, ldx, labels, parts, s);
      case 3: return launch_stats<3>(vec, r, c, row_offset, col_offset, scale, causal, X, ldx, labels, parts, s);
      case 4: return launch_stats<4>(vec, r, c, row_offset, col_offset, scale, causal, X, ldx, labels, parts, s);
      case 5: case 6: return launch_stats<6>(vec, r, c, row_offset, col_offset, scale, causal, X, ldx, labels, parts, s);
      default: return launch_stats<8>(vec, r, c, row_offset, col_offset, scale, causal, X, ldx, labels, parts, s);
    }
  }
  if (phase == TT_SM_APPLY) {
    if (!lse || !Y || ldy < cols) return fail(TT_ERR_ARG, "tile_softmax(APPLY): bad argument");
    return launch_apply((int)rows, (int)cols, row_offset, col_offset, scale, causal, X, ldx, labels, lse, Y, ldy,
                        grad_scale, s);
  }
  return fail(TT_ERR_ARG, "tile_softmax: bad phase %d", phase);
}

extern "C" int tile_xentropy(void* stream, int phase, int64_t rows, int64_t v_len, int64_t v_off,
                             const int32_t* labels, float* logits, int64_t ldz, const float* lse,
                             const float* row_loss, float* loss, int accumulate, float inv_n) {
  using tt::fail;
  hipStream_t s = tt::as_stream(stream);
  if (rows < 0 || v_len < 0) return fail(TT_ERR_ARG, "tile_xentropy: negative size");
  if (phase == TT_XE_LOSS) {
    if (!loss || (rows > 0 && !row_loss) || rows > INT32_MAX) return fail(TT_ERR_ARG, "tile_xentropy(LOSS): bad argument");
    hipLaunchKernelGGL(xe_loss, dim3(1), dim3(256), 0, s, (int)rows, row_loss, loss, accumulate, inv_n);
    return tt::launch_status("tile_xentropy(LOSS)");
  }
  if (phase == TT_XE_GRAD) {
    if (rows == 0 || v_len == 0) return TT_OK;
    if (!labels || !logits || !lse || ldz < v_len) return fail(TT_ERR_ARG, "tile_xentropy(GRAD): bad argument");
    if (v_len > kMaxCols) return fail(TT_ERR_SHAPE, "tile_xentropy: v_len > %d", kMaxCols);
    if (rows > kMaxRows) return fail(TT_ERR_SHAPE, "tile_xentropy: rows > %lld", (long long)kMaxRows);
    return launch_apply((int)rows, (int)v_len, 0, v_off, 1.f, 0, logits, ldz, labels, lse, logits, ldz, inv_n, s);
  }
  return fail(TT_ERR_ARG, "tile_xentropy: bad phase %d", phase);
}

extern "C" int tile_xentropy_multi(void* stream, int phase, int count, int64_t rows, const int64_t* v_len,
                                   const int64_t* v_off, const int32_t* labels, float* const* logits,
                                   const int64_t* ldz, float* parts, int64_t part_stride, const float* lse,
                                   float inv_n) {
  using tt::fail;
  hipStream_t s = tt::as_stream(stream);
  if (count < 0 || rows < 0) return fail(TT_ERR_ARG, "tile_xentropy_multi: negative count or size");
  if (count == 0 || rows == 0) return TT_OK;
  if (phase != TT_XE_STATS && phase != TT_XE_GRAD) return fail(TT_ERR_ARG, "tile_xentropy_multi: bad phase %d", phase);
  if (rows > kMaxRows) return fail(TT_ERR_SHAPE, "tile_xentropy_multi: rows > %lld", (long long)kMaxRows);
  if (!v_len || !v_off || !logits || !ldz || !labels) return fail(TT_ERR_ARG, "tile_xentropy_multi: null array");
  if (phase == TT_XE_STATS && (!parts || part_stride < rows * 3))
    return fail(TT_ERR_ARG, "tile_xentropy_multi(STATS): bad parts");
  if (phase == TT_XE_GRAD && !lse) return fail(TT_ERR_ARG, "tile_xentropy_multi(GRAD): null lse");
  for (int t = 0; t < count; ++t) {
    if (v_len[t] < 1 || v_len[t] > kMaxCols)
      return fail(TT_ERR_SHAPE, "tile_xentropy_multi: v_len of tile %d not in [1, %d]", t, kMaxCols);
    if (!logits[t] || ldz[t] < v_len[t]) return fail(TT_ERR_ARG, "tile_xentropy_multi: bad tile %d", t);
  }
  // tiles in two groups, each launched as one multi-tile kernel per up to
  // kXeMax tiles: those the 16-byte paths take (statistics: ld a multiple
  // of 4 and aligned; gradient: contiguous, ld == cols a multiple of 4, as
  // one flat stream) and the rest (a ragged last vocab tile), so that one
  // odd tile does not send every tile down the scalar path
  const bool grad = phase != TT_XE_STATS;
  auto fast = [&](int t) {
    return grad ? (ldz[t] == v_len[t] && v_len[t] % 4 == 0 && tt::aligned16(logits[t]))
                : (ldz[t] % 4 == 0 && tt::aligned16(logits[t]));
  };
  for (int group = 0; group < 2; ++group) {
    std::vector<int> ids;
    for (int t = 0; t < count; ++t)
      if (fast(t) == (group == 0)) ids.push_back(t);
    for (size_t t0 = 0; t0 < ids.size(); t0 += kXeMax) {
      const int c = (int)std::min<size_t>(kXeMax, ids.size() - t0);
      XeTiles P{};
      int maxc = 1;
      for (int u = 0; u < c; ++u) {
        const int t = ids[t0 + u];
        P.z[u] = logits[t];
        P.ld[u] = ldz[t];
        P.off[u] = v_off[t];
        P.cols[u] = (int)v_len[t];
        P.part[u] = t;
        maxc = std::max(maxc, P.cols[u]);
      }
      const bool vec = group == 0;
      if (!grad) {
        const int r = (int)rows;
        switch ((maxc + 255) / 256) {
          case 1: launch_stats_multi<1>(vec, r, c, P, labels, parts, part_stride, s); break;
          case 2: launch_stats_multi<2>(vec, r, c, P, labels, parts, part_stride, s); break;
          case 3: launch_stats_multi<3>(vec, r, c, P, labels, parts, part_stride, s); break;
          case 4: launch_stats_multi<4>(vec, r, c, P, labels, parts, part_stride, s); break;
          case 5: case 6: launch_stats_multi<6>(vec, r, c, P, labels, parts, part_stride, s); break;
          default: launch_stats_multi<8>(vec, r, c, P, labels, parts, part_stride, s); break;
        }
        if (int rc = tt::launch_status("tile_xentropy_multi(STATS)")) return rc;
      } else if (vec) {
        const int64_t most = rows * (int64_t)maxc / 4;
        const unsigned gx = (unsigned)std::min<int64_t>((most + 255) / 256, std::max<int64_t>(1, 2048 / c));
        hipLaunchKernelGGL(xe_grad_multi, dim3(gx, (unsigned)c), dim3(256), 0, s, (int)rows, P, labels, lse, inv_n);
        if (int rc = tt::launch_status("tile_xentropy_multi(GRAD)")) return rc;
      } else {
        for (int u = 0; u < c; ++u)
          if (int rc = launch_apply((int)rows, P.cols[u], 0, P.off[u], 1.f, 0, P.z[u], P.ld[u], labels, lse, P.z[u],
                                    P.ld[u], inv_n, s))
            return rc;
      }
    }
  }
  return TT_OK;
}

extern "C" int tile_xentropy_merge_groups(void* stream, int64_t rows, int count, const int64_t* v_len, int group,
                                          const float* parts, int64_t part_stride, float* lse, float* row_loss) {
  using tt::fail;
  if (rows < 0 || count < 0) return fail(TT_ERR_ARG, "tile_xentropy_merge_groups: negative size");
  if (rows == 0) return TT_OK;
  if (rows > kMaxRows) return fail(TT_ERR_ARG, "tile_xentropy_merge_groups: rows > %lld", (long long)kMaxRows);
  if (count < 1 || count > kMergeMaxTiles || group < 1 || !v_len || !parts || !lse)
    return fail(TT_ERR_ARG, "tile_xentropy_merge_groups: need 1..%d tiles, group >= 1, parts and lse",
                kMergeMaxTiles);
  GroupList G{};
  int64_t most = 0;
  for (int t = 0; t < count; ++t) {
    if (v_len[t] < 1) return fail(TT_ERR_ARG, "tile_xentropy_merge_groups: v_len of tile %d < 1", t);
    const int64_t gt = (v_len[t] + group - 1) / group;
    most = std::max(most, gt);
    G.first[t + 1] = G.first[t] + (int)gt;
  }
  if (part_stride < most * rows * 3) return fail(TT_ERR_ARG, "tile_xentropy_merge_groups: part_stride too small");
  hipLaunchKernelGGL(xe_merge_groups, dim3((unsigned)((rows + kWaves - 1) / kWaves)), dim3(256), 0,
                     tt::as_stream(stream), (int)rows, count, G, parts, part_stride, lse, row_loss);
  return tt::launch_status("tile_xentropy_merge_groups");
}
