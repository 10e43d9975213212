// Element-wise tile ops of the LLaMA block: the rotary position embedding of
// q and k, and the SwiGLU gate of the MLP.
//
// Rotary embedding (the published LLaMA architecture, which the NNTile
// README's notebook list names as its second model): for i < hd/2 the pair
// (x_i, x_{i + hd/2}) of every head is rotated by t * base^(-2i/hd), t the
// token's position in its sequence. The angles' cosines and sines come from
// a [seq, hd] table (cosines in the first hd/2 columns, sines in the rest)
// that tile_rope_table fills in double precision once. The backward applies
// the transposed rotation (the opposite angle). Both are in place: each
// thread reads its two float4 of a pair before writing them.
//
// SwiGLU: h = silu(a) * b with silu(a) = a / (1 + exp(-a)); its backward
// da = dh * b * s * (1 + a * (1 - s)), db = dh * silu(a) with s the logistic
// function of a. Memory-bound sweeps: float4 accesses, 8 (rope), 12 (swiglu
// forward) and 20 (backward) bytes per element.
#include <algorithm>
#include <cmath>

#include "common.hpp"
#include "rowops.hpp"

using tt::f32x4;

namespace {

__global__ void rope_table_k(int64_t seq, int half, double base, float* __restrict__ table) {
  const int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (i >= seq * half) return;
  const int64_t t = i / half;
  const int j = (int)(i % half);
  const double ang = (double)t * pow(base, -2.0 * (double)j / (double)(2 * half));
  table[t * 2 * half + j] = (float)cos(ang);
  table[t * 2 * half + half + j] = (float)sin(ang);
}

// one thread per (row, head, 4 consecutive pair indices); INV: the
// transposed rotation
struct RopeTiles {
  float* x[4];
};

template <bool INV>
__global__ __launch_bounds__(256) void rope_k(RopeTiles X, int64_t rows, int heads, int hd, int64_t seq_len,
                                              int64_t pos_off, const float* __restrict__ table) {
  const int half = hd >> 1, q4 = half >> 2;
  const int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (i >= rows * heads * q4) return;
  float* __restrict__ x = X.x[blockIdx.y];
  const int j = 4 * (int)(i % q4);
  const int64_t rh = i / q4;
  const int64_t r = rh / heads;
  const int64_t pos = pos_off + r % seq_len;
  float* p = x + rh * hd + j;
  const f32x4 c = *reinterpret_cast<const f32x4*>(table + pos * hd + j);
  const f32x4 s = *reinterpret_cast<const f32x4*>(table + pos * hd + half + j);
  const f32x4 x1 = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
  const f32x4 x2 = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p + half));
  f32x4 y1, y2;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    if (INV) {
      y1[k] = x1[k] * c[k] + x2[k] * s[k];
      y2[k] = x2[k] * c[k] - x1[k] * s[k];
    } else {
      y1[k] = x1[k] * c[k] - x2[k] * s[k];
      y2[k] = x2[k] * c[k] + x1[k] * s[k];
    }
  }
  *reinterpret_cast<f32x4*>(p) = y1;
  *reinterpret_cast<f32x4*>(p + half) = y2;
}

__device__ __forceinline__ float logistic(float a) { return 1.f / (1.f + expf(-a)); }

// VEC: n % 4 == 0 and every pointer 16-byte aligned
template <bool VEC>
__global__ __launch_bounds__(256) void swiglu_fwd_k(int64_t n, const float* __restrict__ a,
                                                    const float* __restrict__ b, float* __restrict__ h) {
  const int64_t i = 4 * (blockIdx.x * (int64_t)blockDim.x + threadIdx.x);
  if (i >= n) return;
  if (VEC) {
    const f32x4 av = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(a + i));
    const f32x4 bv = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(b + i));
    f32x4 o;
#pragma unroll
    for (int k = 0; k < 4; ++k) o[k] = av[k] * logistic(av[k]) * bv[k];
    *reinterpret_cast<f32x4*>(h + i) = o;
  } else {
    for (int64_t e = i; e < n && e < i + 4; ++e) h[e] = a[e] * logistic(a[e]) * b[e];
  }
}

// da, db may alias a, b (each element is read before it is written, by the
// same thread)
template <bool VEC>
__global__ __launch_bounds__(256) void swiglu_bwd_k(int64_t n, const float* dh, const float* a, const float* b,
                                                    float* da, float* db) {
  const int64_t i = 4 * (blockIdx.x * (int64_t)blockDim.x + threadIdx.x);
  if (i >= n) return;
  auto one = [](float d, float av, float bv, float* ga, float* gb) {
    const float s = logistic(av);
    *ga = d * bv * s * (1.f + av * (1.f - s));
    *gb = d * av * s;
  };
  if (VEC) {
    const f32x4 dv = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(dh + i));
    const f32x4 av = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(a + i));
    const f32x4 bv = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(b + i));
    f32x4 oa, ob;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      float ga, gb;
      one(dv[k], av[k], bv[k], &ga, &gb);
      oa[k] = ga;
      ob[k] = gb;
    }
    *reinterpret_cast<f32x4*>(da + i) = oa;
    *reinterpret_cast<f32x4*>(db + i) = ob;
  } else {
    for (int64_t e = i; e < n && e < i + 4; ++e) {
      float ga, gb;
      one(dh[e], a[e], b[e], &ga, &gb);
      da[e] = ga;
      db[e] = gb;
    }
  }
}

bool hd_ok(int64_t hd) { return hd == 16 || hd == 32 || hd == 64 || hd == 128; }

}  // namespace

extern "C" int tile_rope_table(void* stream, int64_t seq, int64_t hd, double base, float* table) {
  using tt::fail;
  if (seq < 0 || !hd_ok(hd) || !(base > 1.0)) return fail(TT_ERR_ARG, "tile_rope_table: bad seq, hd or base");
  if (seq == 0) return TT_OK;
  if (!table) return fail(TT_ERR_ARG, "tile_rope_table: null table");
  const int64_t work = seq * (hd / 2);
  if ((work + 255) / 256 > INT32_MAX) return fail(TT_ERR_ARG, "tile_rope_table: %lld positions exceed one launch", (long long)seq);
  hipLaunchKernelGGL(rope_table_k, dim3((unsigned)((work + 255) / 256)), dim3(256), 0, tt::as_stream(stream), seq,
                     (int)(hd / 2), base, table);
  return tt::launch_status("tile_rope_table");
}

namespace {

int rope_launch(void* stream, int count, float* const* x, int64_t rows, int64_t heads, int64_t hd, int64_t seq_len,
                int64_t pos_off, const float* table, int64_t table_rows, int inverse) {
  using tt::fail;
  if (count < 1 || count > 4 || !x) return fail(TT_ERR_ARG, "tile_rope: 1..4 tiles");
  if (rows < 0 || heads < 1 || !hd_ok(hd) || seq_len < 1 || pos_off < 0)
    return fail(TT_ERR_ARG, "tile_rope: bad size (rows %lld, heads %lld, hd %lld, seq_len %lld, pos_off %lld)",
                (long long)rows, (long long)heads, (long long)hd, (long long)seq_len, (long long)pos_off);
  if (rows == 0) return TT_OK;
  RopeTiles X{};
  for (int t = 0; t < count; ++t) {
    if (!x[t] || !tt::aligned16(x[t])) return fail(TT_ERR_ARG, "tile_rope: x must be non-null and 16-byte aligned");
    X.x[t] = x[t];
  }
  if (!table || !tt::aligned16(table)) return fail(TT_ERR_ARG, "tile_rope: table must be non-null and 16-byte aligned");
  if (pos_off + std::min(rows, seq_len) > table_rows)
    return fail(TT_ERR_SHAPE, "tile_rope: positions up to %lld exceed the table's %lld rows",
                (long long)(pos_off + std::min(rows, seq_len)), (long long)table_rows);
  if (rows * heads > INT64_MAX / hd) return fail(TT_ERR_ARG, "tile_rope: size overflows");
  const int64_t work = rows * heads * (hd / 8);
  if ((work + 255) / 256 > INT32_MAX) return fail(TT_ERR_ARG, "tile_rope: %lld pairs exceed one launch", (long long)work);
  dim3 grid((unsigned)((work + 255) / 256), (unsigned)count), block(256);
  hipStream_t s = tt::as_stream(stream);
  if (inverse)
    hipLaunchKernelGGL(rope_k<true>, grid, block, 0, s, X, rows, (int)heads, (int)hd, seq_len, pos_off, table);
  else
    hipLaunchKernelGGL(rope_k<false>, grid, block, 0, s, X, rows, (int)heads, (int)hd, seq_len, pos_off, table);
  return tt::launch_status("tile_rope");
}

}  // namespace

extern "C" int tile_rope(void* stream, float* x, int64_t rows, int64_t heads, int64_t hd, int64_t seq_len,
                         int64_t pos_off, const float* table, int64_t table_rows, int inverse) {
  if (!x) return tt::fail(TT_ERR_ARG, "tile_rope: null x");
  return rope_launch(stream, 1, &x, rows, heads, hd, seq_len, pos_off, table, table_rows, inverse);
}

extern "C" int tile_rope_multi(void* stream, int count, float* const* x, int64_t rows, int64_t heads, int64_t hd,
                               int64_t seq_len, int64_t pos_off, const float* table, int64_t table_rows,
                               int inverse) {
  return rope_launch(stream, count, x, rows, heads, hd, seq_len, pos_off, table, table_rows, inverse);
}

extern "C" int tile_swiglu_fwd(void* stream, int64_t n, const float* a, const float* b, float* h) {
  using tt::fail;
  if (n < 0) return fail(TT_ERR_ARG, "tile_swiglu_fwd: negative size");
  if (n == 0) return TT_OK;
  if (!a || !b || !h) return fail(TT_ERR_ARG, "tile_swiglu_fwd: null pointer");
  const bool vec = n % 4 == 0 && tt::aligned16(a) && tt::aligned16(b) && tt::aligned16(h);
  const int64_t work = (n + 3) / 4;
  if ((work + 255) / 256 > INT32_MAX) return fail(TT_ERR_ARG, "tile_swiglu_fwd: %lld elements exceed one launch", (long long)n);
  dim3 grid((unsigned)((work + 255) / 256)), block(256);
  hipStream_t s = tt::as_stream(stream);
  if (vec) hipLaunchKernelGGL(swiglu_fwd_k<true>, grid, block, 0, s, n, a, b, h);
  else hipLaunchKernelGGL(swiglu_fwd_k<false>, grid, block, 0, s, n, a, b, h);
  return tt::launch_status("tile_swiglu_fwd");
}

extern "C" int tile_swiglu_bwd(void* stream, int64_t n, const float* dh, const float* a, const float* b, float* da,
                               float* db) {
  using tt::fail;
  if (n < 0) return fail(TT_ERR_ARG, "tile_swiglu_bwd: negative size");
  if (n == 0) return TT_OK;
  if (!dh || !a || !b || !da || !db) return fail(TT_ERR_ARG, "tile_swiglu_bwd: null pointer");
  const bool vec = n % 4 == 0 && tt::aligned16(dh) && tt::aligned16(a) && tt::aligned16(b) && tt::aligned16(da) &&
                   tt::aligned16(db);
  const int64_t work = (n + 3) / 4;
  if ((work + 255) / 256 > INT32_MAX) return fail(TT_ERR_ARG, "tile_swiglu_bwd: %lld elements exceed one launch", (long long)n);
  dim3 grid((unsigned)((work + 255) / 256)), block(256);
  hipStream_t s = tt::as_stream(stream);
  if (vec) hipLaunchKernelGGL(swiglu_bwd_k<true>, grid, block, 0, s, n, dh, a, b, da, db);
  else hipLaunchKernelGGL(swiglu_bwd_k<false>, grid, block, 0, s, n, dh, a, b, da, db);
  return tt::launch_status("tile_swiglu_bwd");
}
