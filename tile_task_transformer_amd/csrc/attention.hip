// Causal multi-head attention tile tasks on the fp32 matrix cores.
//
// One task covers a (query tile, key tile) pair of one (batch tile, head
// tile); the softmax over the key axis is carried across the key tiles of a
// query tile as a running (max, sum, unnormalised output) -- the online
// softmax that makes attention memory-lean (the NNTile README's
// flash-attention flag has the same purpose).
//
// Register layout trick. v_mfma_f32_32x32x2_f32 leaves lane l holding column
// l%32 of its 32x32 result, rows 8*(r/4) + 4*(l/32) + r%4 in register r.
// The forward computes S^T = K Q^T, so each lane owns one QUERY column and
// 16 of the 32 keys; P^T then feeds O^T += V^T P^T directly as the B
// operand (the key supplied by half-wave h at MFMA step s is exactly the key
// that register s of that lane holds), so P never goes through LDS, and the
// per-query softmax statistics need only one cross-half exchange.
// The backward uses the same trick twice: one kernel owns queries (dQ), the
// other owns keys (dK, dV); neither needs atomics, so results are bitwise
// reproducible.
#include "common.hpp"

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kBQ = 128;   // queries per workgroup (4 waves x 32)
constexpr int kBK = 64;    // keys per LDS stage

__device__ __forceinline__ f32x16 mfma(float a, float b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// key (or query) index held by register r of a lane in half-wave h
__device__ __forceinline__ int kidx(int r, int h) { return 8 * (r >> 2) + 4 * h + (r & 3); }

struct AttnGeom {
  int batch, heads, q_len, k_len;
  int64_t q_off, k_off;
  float scale;
};

// token-major tile row of (b, t, h): element (b, t, h, e) at ((b*len + t)*heads + h)*hd + e
__device__ __forceinline__ int64_t row_off(int b, int t, int h, int len, int heads, int hd) {
  return (((int64_t)b * len + t) * heads + h) * hd;
}

// Stage `n` rows (of `len` valid) x HD floats of one (b, h) into LDS [kBK][ld],
// zero-filling rows >= len and columns HD..ld-4.
template <int HD, int LD>
__device__ __forceinline__ void stage_rows(float* __restrict__ dst, const float* __restrict__ src, int b, int h,
                                           int r0, int len, int heads) {
  constexpr int V4 = kBK * HD / 4;
  for (int i = threadIdx.x; i < V4; i += 256) {
    const int r = i / (HD / 4), c = (i % (HD / 4)) * 4;
    f32x4 v = {0.f, 0.f, 0.f, 0.f};
    if (r0 + r < len) v = *reinterpret_cast<const f32x4*>(src + row_off(b, r0 + r, h, len, heads, HD) + c);
    *reinterpret_cast<f32x4*>(dst + r * LD + c) = v;
  }
  if (LD - 4 > HD) {  // pad columns HD..LD-5 (used when HD < 32)
    for (int i = threadIdx.x; i < kBK * (LD - 4 - HD); i += 256) {
      const int r = i / (LD - 4 - HD), c = HD + i % (LD - 4 - HD);
      dst[r * LD + c] = 0.f;
    }
  }
}

// ------------------------------------------------------------------ forward

template <int HD>
__global__ __launch_bounds__(256) void attn_fwd(AttnGeom g, const float* __restrict__ Q, const float* __restrict__ K,
                                                const float* __restrict__ V, float* __restrict__ O,
                                                float* __restrict__ ml, float* __restrict__ lse, int first, int last) {
  constexpr int HDP = HD < 32 ? 32 : HD;   // output rows padded to the 32-row MFMA tile
  constexpr int LDK = HD + 4, LDV = HDP + 4;
  constexpr int NKB = HD / 8;              // float4 groups of the head dim per half-wave
  constexpr int NEB = HDP / 32;
  __shared__ __attribute__((aligned(16))) float Ks[kBK * LDK];
  __shared__ __attribute__((aligned(16))) float Vs[kBK * LDV];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int half = lane >> 5, l32 = lane & 31;
  const int qblk = gridDim.x - 1 - blockIdx.x;  // heavy (late) query blocks first
  const int bh = blockIdx.y, b = bh / g.heads, h = bh % g.heads;
  const int q0 = qblk * kBQ + wave * 32;        // this wave's first query
  const int q = q0 + l32;                       // this lane's query
  const bool qvalid = q < g.q_len;
  const int64_t qpos = g.q_off + q;

  f32x4 qf[NKB];
  {
    const float qs = g.scale * kLog2e;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      f32x4 v = {0.f, 0.f, 0.f, 0.f};
      if (qvalid) v = *reinterpret_cast<const f32x4*>(Q + row_off(b, q, h, g.q_len, g.heads, HD) + 8 * kb + 4 * half);
      qf[kb] = v * qs;
    }
  }
  f32x16 oacc[NEB];
  float m = -INFINITY, l = 0.f;
  const int64_t st = ((int64_t)b * g.heads + h) * g.q_len + q;
  if (!first && qvalid) {
    m = ml[st * 2];
    l = ml[st * 2 + 1];
  }
#pragma unroll
  for (int eb = 0; eb < NEB; ++eb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int e = eb * 32 + kidx(r, half);
      oacc[eb][r] = (!first && qvalid && e < HD) ? O[row_off(b, q, h, g.q_len, g.heads, HD) + e] : 0.f;
    }

  // keys that any query of this workgroup may see
  const int64_t qmax = g.q_off + min(g.q_len, qblk * kBQ + kBQ) - 1;
  const int kend = (int)max((int64_t)0, min((int64_t)g.k_len, qmax - g.k_off + 1));
  const int64_t wave_qmax = g.q_off + min(g.q_len - 1, q0 + 31);

  for (int k0 = 0; k0 < kend; k0 += kBK) {
    __syncthreads();
    stage_rows<HD, LDK>(Ks, K, b, h, k0, g.k_len, g.heads);
    stage_rows<HD, LDV>(Vs, V, b, h, k0, g.k_len, g.heads);
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < kBK / 32; ++kk) {
      const int kb0 = k0 + kk * 32;
      if (kb0 >= g.k_len || q0 >= g.q_len || g.k_off + kb0 > wave_qmax) continue;  // wave-uniform skip
      f32x16 s;
#pragma unroll
      for (int r = 0; r < 16; ++r) s[r] = 0.f;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        const f32x4 kf = *reinterpret_cast<const f32x4*>(Ks + (kk * 32 + l32) * LDK + 8 * kb + 4 * half);
#pragma unroll
        for (int i = 0; i < 4; ++i) s = mfma(kf[i], qf[kb][i], s);
      }
      float mloc = -INFINITY;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = kb0 + kidx(r, half);
        if (key >= g.k_len || g.k_off + key > qpos) s[r] = -INFINITY;
        mloc = fmaxf(mloc, s[r]);
      }
      mloc = fmaxf(mloc, __shfl_xor(mloc, 32, 64));
      const float mnew = fmaxf(m, mloc);
      const float alpha = mnew == -INFINITY ? 1.f : exp2f(m - mnew);
      float psum = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        s[r] = mnew == -INFINITY ? 0.f : exp2f(s[r] - mnew);
        psum += s[r];
      }
      psum += __shfl_xor(psum, 32, 64);
      l = l * alpha + psum;
      m = mnew;
#pragma unroll
      for (int eb = 0; eb < NEB; ++eb) {
        oacc[eb] *= alpha;
#pragma unroll
        for (int r = 0; r < 16; ++r)
          oacc[eb] = mfma(Vs[(kk * 32 + kidx(r, half)) * LDV + eb * 32 + l32], s[r], oacc[eb]);
      }
    }
  }

  if (!qvalid) return;
  const float inv = last ? 1.f / l : 1.f;
  float* orow = O + row_off(b, q, h, g.q_len, g.heads, HD);
#pragma unroll
  for (int eb = 0; eb < NEB; ++eb)
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
      const int e = eb * 32 + 8 * gq + 4 * half;
      if (e < HD) {
        f32x4 v = {oacc[eb][4 * gq] * inv, oacc[eb][4 * gq + 1] * inv, oacc[eb][4 * gq + 2] * inv,
                   oacc[eb][4 * gq + 3] * inv};
        *reinterpret_cast<f32x4*>(orow + e) = v;
      }
    }
  if (half == 0) {
    if (last) lse[st] = (m + log2f(l)) * kLn2;
    else {
      ml[st * 2] = m;
      ml[st * 2 + 1] = l;
    }
  }
}

// --------------------------------------------------------------- backward

__global__ void attn_prep(int batch, int heads, int q_len, int hd, const float* __restrict__ O,
                          const float* __restrict__ dO, float* __restrict__ Dv) {
  const int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;  // (b, t, h) row
  if (i >= (int64_t)batch * q_len * heads) return;
  const int h = (int)(i % heads);
  const int64_t bt = i / heads;
  const int t = (int)(bt % q_len), b = (int)(bt / q_len);
  const f32x4* o = reinterpret_cast<const f32x4*>(O + i * hd);
  const f32x4* d = reinterpret_cast<const f32x4*>(dO + i * hd);
  float s = 0.f;
  for (int e = 0; e < hd / 4; ++e) {
    const f32x4 a = o[e], c = d[e];
    s += a[0] * c[0] + a[1] * c[1] + a[2] * c[2] + a[3] * c[3];
  }
  Dv[((int64_t)b * heads + h) * q_len + t] = s;
}

// dQ: each wave owns 32 queries; loops over key blocks.
template <int HD>
__global__ __launch_bounds__(256) void attn_bwd_dq(AttnGeom g, const float* __restrict__ Q,
                                                   const float* __restrict__ K, const float* __restrict__ V,
                                                   const float* __restrict__ dO, const float* __restrict__ lse,
                                                   const float* __restrict__ Dv, float* __restrict__ dQ, int acc) {
  constexpr int HDP = HD < 32 ? 32 : HD;
  constexpr int LD = HDP + 4;
  constexpr int NKB = HD / 8, NEB = HDP / 32;
  __shared__ __attribute__((aligned(16))) float Ks[kBK * LD];
  __shared__ __attribute__((aligned(16))) float Vs[kBK * LD];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int half = lane >> 5, l32 = lane & 31;
  const int qblk = gridDim.x - 1 - blockIdx.x;
  const int bh = blockIdx.y, b = bh / g.heads, h = bh % g.heads;
  const int q0 = qblk * kBQ + wave * 32;
  const int q = q0 + l32;
  const bool qvalid = q < g.q_len;
  const int64_t qpos = g.q_off + q;
  const int64_t st = ((int64_t)b * g.heads + h) * g.q_len + q;

  f32x4 qf[NKB], df[NKB];
  const float qs = g.scale * kLog2e;
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb) {
    f32x4 v = {0.f, 0.f, 0.f, 0.f}, w = v;
    if (qvalid) {
      v = *reinterpret_cast<const f32x4*>(Q + row_off(b, q, h, g.q_len, g.heads, HD) + 8 * kb + 4 * half);
      w = *reinterpret_cast<const f32x4*>(dO + row_off(b, q, h, g.q_len, g.heads, HD) + 8 * kb + 4 * half);
    }
    qf[kb] = v * qs;
    df[kb] = w;
  }
  const float lse2 = qvalid ? lse[st] * kLog2e : 0.f;
  const float dq_d = qvalid ? Dv[st] : 0.f;
  f32x16 dacc[NEB];
#pragma unroll
  for (int eb = 0; eb < NEB; ++eb)
#pragma unroll
    for (int r = 0; r < 16; ++r) dacc[eb][r] = 0.f;

  const int64_t qmax = g.q_off + min(g.q_len, qblk * kBQ + kBQ) - 1;
  const int kend = (int)max((int64_t)0, min((int64_t)g.k_len, qmax - g.k_off + 1));
  const int64_t wave_qmax = g.q_off + min(g.q_len - 1, q0 + 31);

  for (int k0 = 0; k0 < kend; k0 += kBK) {
    __syncthreads();
    stage_rows<HD, LD>(Ks, K, b, h, k0, g.k_len, g.heads);
    stage_rows<HD, LD>(Vs, V, b, h, k0, g.k_len, g.heads);
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < kBK / 32; ++kk) {
      const int kb0 = k0 + kk * 32;
      if (kb0 >= g.k_len || q0 >= g.q_len || g.k_off + kb0 > wave_qmax) continue;
      f32x16 s, dp;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        s[r] = 0.f;
        dp[r] = 0.f;
      }
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        const f32x4 kf = *reinterpret_cast<const f32x4*>(Ks + (kk * 32 + l32) * LD + 8 * kb + 4 * half);
        const f32x4 vf = *reinterpret_cast<const f32x4*>(Vs + (kk * 32 + l32) * LD + 8 * kb + 4 * half);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          s = mfma(kf[i], qf[kb][i], s);     // S^T = K Q^T (log2 units)
          dp = mfma(vf[i], df[kb][i], dp);   // dP^T = V dO^T
        }
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = kb0 + kidx(r, half);
        const bool ok = qvalid && key < g.k_len && g.k_off + key <= qpos;
        const float p = ok ? exp2f(s[r] - lse2) : 0.f;
        s[r] = p * (dp[r] - dq_d);           // dS^T
      }
#pragma unroll
      for (int eb = 0; eb < NEB; ++eb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          dacc[eb] = mfma(Ks[(kk * 32 + kidx(r, half)) * LD + eb * 32 + l32], s[r], dacc[eb]);
    }
  }
  if (!qvalid) return;
  float* drow = dQ + row_off(b, q, h, g.q_len, g.heads, HD);
#pragma unroll
  for (int eb = 0; eb < NEB; ++eb)
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
      const int e = eb * 32 + 8 * gq + 4 * half;
      if (e < HD) {
        f32x4 v = {dacc[eb][4 * gq], dacc[eb][4 * gq + 1], dacc[eb][4 * gq + 2], dacc[eb][4 * gq + 3]};
        v *= g.scale;
        if (acc) v += *reinterpret_cast<const f32x4*>(drow + e);
        *reinterpret_cast<f32x4*>(drow + e) = v;
      }
    }
}

// dK, dV: each wave owns 32 keys; loops over query blocks.
template <int HD>
__global__ __launch_bounds__(256) void attn_bwd_dkv(AttnGeom g, const float* __restrict__ Q,
                                                    const float* __restrict__ K, const float* __restrict__ V,
                                                    const float* __restrict__ dO, const float* __restrict__ lse,
                                                    const float* __restrict__ Dv, float* __restrict__ dK,
                                                    float* __restrict__ dV, int acc) {
  constexpr int HDP = HD < 32 ? 32 : HD;
  constexpr int LD = HDP + 4;
  constexpr int NKB = HD / 8, NEB = HDP / 32;
  __shared__ __attribute__((aligned(16))) float Qs[kBK * LD];
  __shared__ __attribute__((aligned(16))) float Ds[kBK * LD];
  __shared__ float Ls[kBK], Dd[kBK];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int half = lane >> 5, l32 = lane & 31;
  const int kblk = blockIdx.x;
  const int bh = blockIdx.y, b = bh / g.heads, h = bh % g.heads;
  const int k0w = kblk * kBQ + wave * 32;     // this wave's first key
  const int key = k0w + l32;                  // this lane's key
  const bool kvalid = key < g.k_len;
  const int64_t kpos = g.k_off + key;

  f32x4 kf[NKB], vf[NKB];
  const float qs = g.scale * kLog2e;
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb) {
    f32x4 v = {0.f, 0.f, 0.f, 0.f}, w = v;
    if (kvalid) {
      v = *reinterpret_cast<const f32x4*>(K + row_off(b, key, h, g.k_len, g.heads, HD) + 8 * kb + 4 * half);
      w = *reinterpret_cast<const f32x4*>(V + row_off(b, key, h, g.k_len, g.heads, HD) + 8 * kb + 4 * half);
    }
    kf[kb] = v * qs;
    vf[kb] = w;
  }
  f32x16 dk[NEB], dv[NEB];
#pragma unroll
  for (int eb = 0; eb < NEB; ++eb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      dk[eb][r] = 0.f;
      dv[eb][r] = 0.f;
    }

  // first query (tile-local) that can see the workgroup's first key
  const int64_t kmin = g.k_off + (int64_t)kblk * kBQ;
  int qstart = (int)max((int64_t)0, kmin - g.q_off);
  qstart = (qstart / kBK) * kBK;
  const bool wave_live = k0w < g.k_len;

  for (int qb = qstart; qb < g.q_len; qb += kBK) {
    __syncthreads();
    stage_rows<HD, LD>(Qs, Q, b, h, qb, g.q_len, g.heads);
    stage_rows<HD, LD>(Ds, dO, b, h, qb, g.q_len, g.heads);
    for (int i = threadIdx.x; i < kBK; i += 256) {
      const int qq = qb + i;
      const int64_t st = ((int64_t)b * g.heads + h) * g.q_len + qq;
      Ls[i] = qq < g.q_len ? lse[st] * kLog2e : 0.f;
      Dd[i] = qq < g.q_len ? Dv[st] : 0.f;
    }
    __syncthreads();
    if (!wave_live) continue;
#pragma unroll
    for (int qq = 0; qq < kBK / 32; ++qq) {
      const int qb0 = qb + qq * 32;
      if (qb0 >= g.q_len || g.q_off + qb0 + 31 < g.k_off + k0w) continue;  // all masked for this wave
      f32x16 s, dp;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        s[r] = 0.f;
        dp[r] = 0.f;
      }
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        const f32x4 qf = *reinterpret_cast<const f32x4*>(Qs + (qq * 32 + l32) * LD + 8 * kb + 4 * half);
        const f32x4 df = *reinterpret_cast<const f32x4*>(Ds + (qq * 32 + l32) * LD + 8 * kb + 4 * half);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          s = mfma(qf[i], kf[kb][i], s);     // S = Q K^T (log2 units); lane owns key column
          dp = mfma(df[i], vf[kb][i], dp);   // dP = dO V^T
        }
      }
      f32x16 p;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int ql = qq * 32 + kidx(r, half);
        const int qg = qb + ql;
        const bool ok = kvalid && qg < g.q_len && kpos <= g.q_off + qg;
        p[r] = ok ? exp2f(s[r] - Ls[ql]) : 0.f;
        s[r] = p[r] * (dp[r] - Dd[ql]);      // dS
      }
#pragma unroll
      for (int eb = 0; eb < NEB; ++eb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int ql = qq * 32 + kidx(r, half);
          dv[eb] = mfma(Ds[ql * LD + eb * 32 + l32], p[r], dv[eb]);   // dV^T += dO^T P
          dk[eb] = mfma(Qs[ql * LD + eb * 32 + l32], s[r], dk[eb]);   // dK^T += Q^T dS
        }
    }
  }
  if (!kvalid) return;
  float* krow = dK + row_off(b, key, h, g.k_len, g.heads, HD);
  float* vrow = dV + row_off(b, key, h, g.k_len, g.heads, HD);
#pragma unroll
  for (int eb = 0; eb < NEB; ++eb)
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
      const int e = eb * 32 + 8 * gq + 4 * half;
      if (e < HD) {
        f32x4 a = {dk[eb][4 * gq], dk[eb][4 * gq + 1], dk[eb][4 * gq + 2], dk[eb][4 * gq + 3]};
        f32x4 c = {dv[eb][4 * gq], dv[eb][4 * gq + 1], dv[eb][4 * gq + 2], dv[eb][4 * gq + 3]};
        a *= g.scale;
        if (acc) {
          a += *reinterpret_cast<const f32x4*>(krow + e);
          c += *reinterpret_cast<const f32x4*>(vrow + e);
        }
        *reinterpret_cast<f32x4*>(krow + e) = a;
        *reinterpret_cast<f32x4*>(vrow + e) = c;
      }
    }
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

int check_geom(const char* who, int64_t batch, int64_t heads, int64_t q_len, int64_t k_len, int64_t hd) {
  if (batch < 0 || heads < 0 || q_len < 0 || k_len < 0) return tt::fail(TT_ERR_ARG, "%s: negative size", who);
  if (hd != 16 && hd != 32 && hd != 64 && hd != 128)
    return tt::fail(TT_ERR_UNSUPPORTED, "%s: head dim %lld not in {16, 32, 64, 128}", who, (long long)hd);
  if (batch * heads > 65535 || q_len > INT32_MAX || k_len > INT32_MAX)
    return tt::fail(TT_ERR_SHAPE, "%s: grid too large", who);
  return TT_OK;
}

}  // namespace

extern "C" int tile_attention_fwd(void* stream, int64_t batch, int64_t heads, int64_t q_len, int64_t k_len, int64_t hd,
                                  int64_t q_off, int64_t k_off, const float* Q, const float* K, const float* V,
                                  float* O, float* ml, float* lse, int first, int last, float scale) {
  if (int rc = check_geom("tile_attention_fwd", batch, heads, q_len, k_len, hd)) return rc;
  if (batch == 0 || heads == 0 || q_len == 0) return TT_OK;
  if (!Q || !O || (k_len > 0 && (!K || !V))) return tt::fail(TT_ERR_ARG, "tile_attention_fwd: null tensor");
  if ((!last && !ml) || (!first && !ml) || (last && !lse)) return tt::fail(TT_ERR_ARG, "tile_attention_fwd: null state");
  if (!aligned16(Q) || !aligned16(O) || (k_len > 0 && (!aligned16(K) || !aligned16(V))))
    return tt::fail(TT_ERR_ARG, "tile_attention_fwd: tensors must be 16-byte aligned");
  AttnGeom g{(int)batch, (int)heads, (int)q_len, (int)k_len, q_off, k_off, scale};
  dim3 grid((unsigned)((q_len + kBQ - 1) / kBQ), (unsigned)(batch * heads)), block(256);
  hipStream_t s = tt::as_stream(stream);
  switch (hd) {
    case 16: hipLaunchKernelGGL(attn_fwd<16>, grid, block, 0, s, g, Q, K, V, O, ml, lse, first, last); break;
    case 32: hipLaunchKernelGGL(attn_fwd<32>, grid, block, 0, s, g, Q, K, V, O, ml, lse, first, last); break;
    case 64: hipLaunchKernelGGL(attn_fwd<64>, grid, block, 0, s, g, Q, K, V, O, ml, lse, first, last); break;
    default: hipLaunchKernelGGL(attn_fwd<128>, grid, block, 0, s, g, Q, K, V, O, ml, lse, first, last); break;
  }
  return tt::launch_status("tile_attention_fwd");
}

extern "C" int tile_attention_bwd(void* stream, int phase, int64_t batch, int64_t heads, int64_t q_len, int64_t k_len,
                                  int64_t hd, int64_t q_off, int64_t k_off, const float* Q, const float* K,
                                  const float* V, const float* O, const float* dO, const float* lse, float* Dvec,
                                  float* dQ, float* dK, float* dV, int acc_dq, int acc_dkv, float scale) {
  if (int rc = check_geom("tile_attention_bwd", batch, heads, q_len, k_len, hd)) return rc;
  if (batch == 0 || heads == 0) return TT_OK;
  hipStream_t s = tt::as_stream(stream);
  if (phase == TT_ATT_PREP) {
    if (q_len == 0) return TT_OK;
    if (!O || !dO || !Dvec) return tt::fail(TT_ERR_ARG, "tile_attention_bwd(PREP): null tensor");
    if (!aligned16(O) || !aligned16(dO)) return tt::fail(TT_ERR_ARG, "tile_attention_bwd: 16-byte alignment required");
    const int64_t rows = batch * q_len * heads;
    hipLaunchKernelGGL(attn_prep, dim3((unsigned)((rows + 255) / 256)), dim3(256), 0, s, (int)batch, (int)heads,
                       (int)q_len, (int)hd, O, dO, Dvec);
    return tt::launch_status("tile_attention_bwd(PREP)");
  }
  if (phase != TT_ATT_GRAD) return tt::fail(TT_ERR_ARG, "tile_attention_bwd: bad phase %d", phase);
  if (q_len == 0 || k_len == 0) return TT_OK;
  if (!Q || !K || !V || !dO || !lse || !Dvec || !dQ || !dK || !dV)
    return tt::fail(TT_ERR_ARG, "tile_attention_bwd(GRAD): null tensor");
  for (const void* p : {(const void*)Q, (const void*)K, (const void*)V, (const void*)dO, (const void*)dQ,
                        (const void*)dK, (const void*)dV})
    if (!aligned16(p)) return tt::fail(TT_ERR_ARG, "tile_attention_bwd: 16-byte alignment required");
  AttnGeom g{(int)batch, (int)heads, (int)q_len, (int)k_len, q_off, k_off, scale};
  dim3 gq((unsigned)((q_len + kBQ - 1) / kBQ), (unsigned)(batch * heads));
  dim3 gk((unsigned)((k_len + kBQ - 1) / kBQ), (unsigned)(batch * heads));
  dim3 block(256);
#define TT_ATT_BWD(HD)                                                                                   \
  hipLaunchKernelGGL(attn_bwd_dq<HD>, gq, block, 0, s, g, Q, K, V, dO, lse, Dvec, dQ, acc_dq);          \
  hipLaunchKernelGGL(attn_bwd_dkv<HD>, gk, block, 0, s, g, Q, K, V, dO, lse, Dvec, dK, dV, acc_dkv)
  switch (hd) {
    case 16: TT_ATT_BWD(16); break;
    case 32: TT_ATT_BWD(32); break;
    case 64: TT_ATT_BWD(64); break;
    default: TT_ATT_BWD(128); break;
  }
#undef TT_ATT_BWD
  return tt::launch_status("tile_attention_bwd(GRAD)");
}
