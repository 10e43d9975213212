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
//
// Work split. A workgroup has 4 waves and owns 64 queries (dK/dV: 64 keys)
// as 2 groups of 32. Each group's row of work (all visible keys; dK/dV: all
// queries that see the key) is shared by 2 waves: the streamed operand
// arrives in LDS stages of 64 rows and wave `part` takes the 32-row half
// `part` of every stage. At the end the two partial results are merged in a
// fixed order (online-softmax states by rescaling to the larger max,
// gradient partials by addition), so the result does not depend on timing.
// Splitting the rows halves the longest wave of a causal tile (the last
// query block sees every key), which bounds the kernel's critical path.
// The grid is (b, h) pairs along x and blocks along y, so the hardware
// dispatches the heaviest block of every (b, h) before any lighter one
// (longest-first list scheduling over the whole launch), and, when the
// pair count is a multiple of 8, every block of one (b, h) lands on the
// same XCD (workgroups go to the XCDs round-robin), so its K and V stay in
// that XCD's L2.
// The next stage's global loads are in flight (in registers) while the
// current stage's MFMAs run -- except in the dK/dV kernel, which keeps its
// keys in LDS and issues the loads after the MFMAs: that frees the
// registers for two workgroups per CU, whose waves cover each other's load
// latency (measured: 497 -> 446 us per GPT2-small layer backward). Per-element causal masking is applied only to
// sub-blocks that straddle the diagonal; sub-blocks wholly above it are
// skipped per wave.
#include "common.hpp"

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kNT = 256;          // threads per workgroup (4 waves)
constexpr int kBQ = 64;           // queries (dK/dV kernel: keys) owned per workgroup
constexpr int kBS = 64;           // streamed rows per LDS stage (2 halves of 32)

// 2^x with the hardware instruction: every argument here is <= 0 up to
// rounding (scores minus a running maximum or the row's logsumexp), and a
// result below 2^-126 is negligible next to the row sum (>= 1), so no
// denormal range handling (measured: forward 3%, backward 2% faster than
// exp2f).
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

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

// Streams blocks of kBS rows x HD floats of one (b, h) through registers into
// an LDS buffer [kBS][LD]; rows >= len read as zero.
template <int HD, int LD>
struct Stager {
  static constexpr int V4 = kBS * HD / 4;
  static constexpr int PT = (V4 + kNT - 1) / kNT;
  f32x4 r[PT];
  __device__ __forceinline__ void load(const float* __restrict__ src, int b, int h, int r0, int len, int heads) {
#pragma unroll
    for (int i = 0; i < PT; ++i) {
      const int idx = threadIdx.x + kNT * i;
      const int row = idx / (HD / 4), c = (idx % (HD / 4)) * 4;
      f32x4 v = {0.f, 0.f, 0.f, 0.f};
      if (idx < V4 && r0 + row < len)
        v = *reinterpret_cast<const f32x4*>(src + row_off(b, r0 + row, h, len, heads, HD) + c);
      r[i] = v;
    }
  }
  __device__ __forceinline__ void store(float* dst) const {
#pragma unroll
    for (int i = 0; i < PT; ++i) {
      const int idx = threadIdx.x + kNT * i;
      if (idx < V4) {
        const int row = idx / (HD / 4), c = (idx % (HD / 4)) * 4;
        *reinterpret_cast<f32x4*>(dst + row * LD + c) = r[i];
      }
    }
  }
};

// zero the pad columns HD..LD-5 of an LDS block (used when HD < 32)
template <int HD, int LD>
__device__ __forceinline__ void zero_pad(float* dst) {
  constexpr int W = LD - 4 - HD;
  if (W > 0)
    for (int i = threadIdx.x; i < kBS * W; i += kNT) dst[(i / W) * LD + HD + i % W] = 0.f;
}

template <int HD>
struct Cfg {
  static constexpr int HDP = HD < 32 ? 32 : HD;   // MFMA output rows padded to 32
  static constexpr int LD = HDP + 4;              // LDS row stride
  static constexpr int NKB = HD / 8;              // 8-wide head-dim groups (4 per half-wave)
  static constexpr int NEB = HDP / 32;            // 32-row blocks of the head dim
  static constexpr int MINW = HD <= 64 ? 2 : 1;   // waves per SIMD the registers must allow
};

// ------------------------------------------------------------------ forward

template <int HD>
__global__ __launch_bounds__(kNT, Cfg<HD>::MINW) void attn_fwd(AttnGeom g, const float* __restrict__ Q,
                                                              const float* __restrict__ K,
                                                              const float* __restrict__ V, float* __restrict__ O,
                                                              float* __restrict__ ml, float* __restrict__ lse,
                                                              int first, int last) {
  using C = Cfg<HD>;
  constexpr int LD = C::LD, NKB = C::NKB, NEB = C::NEB;
  __shared__ __attribute__((aligned(16))) float Ks[kBS * LD];
  __shared__ __attribute__((aligned(16))) float Vs[kBS * LD];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int grp = wave & 1, part = wave >> 1;
  const int half = lane >> 5, l32 = lane & 31;
  const int qblk = gridDim.y - 1 - blockIdx.y;  // heavy (late) query blocks first, over all (b, h)
  const int bh = blockIdx.x, b = bh / g.heads, h = bh % g.heads;
  const int q0 = qblk * kBQ + grp * 32;
  const int q = q0 + l32;
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
  // running state; the previous key tiles' state enters through part 0 only
  f32x16 oacc[NEB];
  float m = -INFINITY, l = 0.f;
  const int64_t st = ((int64_t)b * g.heads + h) * g.q_len + q;
  const bool carry = !first && qvalid && part == 0;
  if (carry) {
    m = ml[st * 2];
    l = ml[st * 2 + 1];
  }
#pragma unroll
  for (int eb = 0; eb < NEB; ++eb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int e = eb * 32 + kidx(r, half);
      oacc[eb][r] = (carry && e < HD) ? O[row_off(b, q, h, g.q_len, g.heads, HD) + e] : 0.f;
    }

  const int64_t qmax = g.q_off + min(g.q_len, qblk * kBQ + kBQ) - 1;
  const int kend = (int)max((int64_t)0, min((int64_t)g.k_len, qmax - g.k_off + 1));
  const int64_t wave_qmin = g.q_off + q0;
  const int64_t wave_qmax = g.q_off + min(g.q_len - 1, q0 + 31);
  const bool wave_live = q0 < g.q_len;

  zero_pad<HD, LD>(Vs);
  Stager<HD, LD> sk, sv;
  if (kend > 0) {
    sk.load(K, b, h, 0, g.k_len, g.heads);
    sv.load(V, b, h, 0, g.k_len, g.heads);
    sk.store(Ks);
    sv.store(Vs);
  }
  __syncthreads();
  for (int k0 = 0; k0 < kend; k0 += kBS) {
    const bool more = k0 + kBS < kend;
    if (more) {
      sk.load(K, b, h, k0 + kBS, g.k_len, g.heads);
      sv.load(V, b, h, k0 + kBS, g.k_len, g.heads);
    }
    const int kb0 = k0 + part * 32;
    const float* ks = Ks + part * 32 * LD;
    const float* vs = Vs + part * 32 * LD;
    if (wave_live && kb0 < g.k_len && g.k_off + kb0 <= wave_qmax) {  // wave-uniform
      f32x16 s;
#pragma unroll
      for (int r = 0; r < 16; ++r) s[r] = 0.f;
      // a wave issuing its products takes priority over the other resident
      // wave of its SIMD, whose softmax arithmetic fills the gaps (head dim
      // 64, two waves per SIMD: 0.922 -> 0.89 ms per GPT2-small step; at 128
      // one wave per SIMD, unchanged; the same in the dK/dV kernel measured
      // no gain)
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        const f32x4 kf = *reinterpret_cast<const f32x4*>(ks + l32 * LD + 8 * kb + 4 * half);
#pragma unroll
        for (int i = 0; i < 4; ++i) s = mfma(kf[i], qf[kb][i], s);
      }
      __builtin_amdgcn_s_setprio(0);
      if (kb0 + 31 >= g.k_len || g.k_off + kb0 + 31 > wave_qmin) {  // straddles the diagonal or the end
        // key kl of this block is visible to the lane's query iff kl <= dlim
        const int dlim = (int)max((int64_t)-1, min((int64_t)32, qpos - g.k_off - kb0));
        const int klim = g.k_len - kb0;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int kl = kidx(r, half);
          s[r] = ((kl < klim) & (kl <= dlim)) ? s[r] : -INFINITY;
        }
      }
      float mloc = s[0];
#pragma unroll
      for (int r = 1; r < 16; ++r) mloc = fmaxf(mloc, s[r]);
      mloc = fmaxf(mloc, __shfl_xor(mloc, 32, 64));
      const float mnew = fmaxf(m, mloc);
      const float alpha = mnew == -INFINITY ? 1.f : exp2_hw(m - mnew);
      float psum = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        s[r] = mnew == -INFINITY ? 0.f : exp2_hw(s[r] - mnew);
        psum += s[r];
      }
      psum += __shfl_xor(psum, 32, 64);
      l = l * alpha + psum;
      m = mnew;
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int eb = 0; eb < NEB; ++eb) {
        oacc[eb] *= alpha;
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[eb] = mfma(vs[kidx(r, half) * LD + eb * 32 + l32], s[r], oacc[eb]);
      }
      __builtin_amdgcn_s_setprio(0);
    }
    __syncthreads();
    if (more) {
      sk.store(Ks);
      sv.store(Vs);
    }
    __syncthreads();
  }

  // merge part 1 into part 0 (LDS reused; the loop ended on a barrier)
  constexpr int STR = 2 + 16 * NEB;
  float* xb = Ks;  // kBS*LD floats >= 2 groups x 64 lanes x STR
  if (part == 1) {
    float* p = xb + (grp * 64 + lane) * STR;
    p[0] = m;
    p[1] = l;
#pragma unroll
    for (int eb = 0; eb < NEB; ++eb)
#pragma unroll
      for (int r = 0; r < 16; ++r) p[2 + 16 * eb + r] = oacc[eb][r];
  }
  __syncthreads();
  if (part == 1 || !qvalid) return;
  {
    const float* p = xb + (grp * 64 + lane) * STR;
    const float m1 = p[0], l1 = p[1];
    const float mm = fmaxf(m, m1);
    const float a0 = m == -INFINITY ? 0.f : exp2_hw(m - mm), a1 = m1 == -INFINITY ? 0.f : exp2_hw(m1 - mm);
    l = l * a0 + l1 * a1;
    m = mm;
#pragma unroll
    for (int eb = 0; eb < NEB; ++eb)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[eb][r] = oacc[eb][r] * a0 + p[2 + 16 * eb + r] * a1;
  }
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

// D[b, h, t] = sum_e dO[b, t, h, e] * O[b, t, h, e]: hd / 4 consecutive lanes
// per (b, t, h) row, one float4 each (a wave reads whole rows, coalesced),
// summed by a fixed butterfly of shuffles
template <int LPR>
__global__ __launch_bounds__(256) void attn_prep(int batch, int heads, int q_len, const float* __restrict__ O,
                                                 const float* __restrict__ dO, float* __restrict__ Dv) {
  const int64_t gid = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  const int64_t i = gid / LPR;  // (b, t, h) row
  const int part = (int)(gid % LPR);
  const bool live = i < (int64_t)batch * q_len * heads;
  float s = 0.f;
  if (live) {
    const f32x4 a = reinterpret_cast<const f32x4*>(O)[i * LPR + part];
    const f32x4 c = reinterpret_cast<const f32x4*>(dO)[i * LPR + part];
    s = a[0] * c[0] + a[1] * c[1] + a[2] * c[2] + a[3] * c[3];
  }
#pragma unroll
  for (int o = LPR / 2; o > 0; o >>= 1) s += __shfl_xor(s, o, LPR);
  if (live && part == 0) {
    const int h = (int)(i % heads);
    const int64_t bt = i / heads;
    const int t = (int)(bt % q_len), b = (int)(bt / q_len);
    Dv[((int64_t)b * heads + h) * q_len + t] = s;
  }
}

// sum of the two parts' register blocks, part 0 + part 1, through LDS
template <int N>
__device__ __forceinline__ void merge_add(float* xb, int grp, int part, int lane, f32x16 (&a)[N]) {
  float* p = xb + (grp * 64 + lane) * (16 * N);
  if (part == 1)
#pragma unroll
    for (int n = 0; n < N; ++n)
#pragma unroll
      for (int r = 0; r < 16; ++r) p[16 * n + r] = a[n][r];
  __syncthreads();
  if (part == 0)
#pragma unroll
    for (int n = 0; n < N; ++n)
#pragma unroll
      for (int r = 0; r < 16; ++r) a[n][r] += p[16 * n + r];
}

// dQ: a group of 32 queries per wave pair; streams key blocks.
template <int HD>
__global__ __launch_bounds__(kNT, Cfg<HD>::MINW) void attn_bwd_dq(AttnGeom g, const float* __restrict__ Q,
                                                                 const float* __restrict__ K,
                                                                 const float* __restrict__ V,
                                                                 const float* __restrict__ dO,
                                                                 const float* __restrict__ lse,
                                                                 const float* __restrict__ Dv, float* __restrict__ dQ,
                                                                 int acc) {
  using C = Cfg<HD>;
  constexpr int LD = C::LD, NKB = C::NKB, NEB = C::NEB;
  __shared__ __attribute__((aligned(16))) float Ks[kBS * LD];
  __shared__ __attribute__((aligned(16))) float Vs[kBS * LD];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int grp = wave & 1, part = wave >> 1;
  const int half = lane >> 5, l32 = lane & 31;
  const int qblk = gridDim.y - 1 - blockIdx.y;
  const int bh = blockIdx.x, b = bh / g.heads, h = bh % g.heads;
  const int q0 = qblk * kBQ + grp * 32;
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
  const int64_t wave_qmin = g.q_off + q0;
  const int64_t wave_qmax = g.q_off + min(g.q_len - 1, q0 + 31);
  const bool wave_live = q0 < g.q_len;

  zero_pad<HD, LD>(Ks);
  Stager<HD, LD> sk, sv;
  if (kend > 0) {
    sk.load(K, b, h, 0, g.k_len, g.heads);
    sv.load(V, b, h, 0, g.k_len, g.heads);
    sk.store(Ks);
    sv.store(Vs);
  }
  __syncthreads();
  for (int k0 = 0; k0 < kend; k0 += kBS) {
    const bool more = k0 + kBS < kend;
    if (more) {
      sk.load(K, b, h, k0 + kBS, g.k_len, g.heads);
      sv.load(V, b, h, k0 + kBS, g.k_len, g.heads);
    }
    const int kb0 = k0 + part * 32;
    const float* ks = Ks + part * 32 * LD;
    const float* vs = Vs + part * 32 * LD;
    if (wave_live && kb0 < g.k_len && g.k_off + kb0 <= wave_qmax) {
      f32x16 s, dp;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        s[r] = 0.f;
        dp[r] = 0.f;
      }
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        const f32x4 kf = *reinterpret_cast<const f32x4*>(ks + l32 * LD + 8 * kb + 4 * half);
        const f32x4 vf = *reinterpret_cast<const f32x4*>(vs + l32 * LD + 8 * kb + 4 * half);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          s = mfma(kf[i], qf[kb][i], s);     // S^T = K Q^T (log2 units)
          dp = mfma(vf[i], df[kb][i], dp);   // dP^T = V dO^T
        }
      }
      const bool edge = kb0 + 31 >= g.k_len || g.k_off + kb0 + 31 > wave_qmin;
      // key kl of this block is visible to the lane's query iff kl <= dlim
      const int dlim = (int)max((int64_t)-1, min((int64_t)32, qpos - g.k_off - kb0));
      const int klim = g.k_len - kb0;  // keys >= klim are past the tile
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kl = kidx(r, half);
        const bool ok = qvalid & (!edge | ((kl < klim) & (kl <= dlim)));
        const float e = exp2_hw(s[r] - lse2);  // computed for every entry; masked ones select 0
        const float p = ok ? e : 0.f;
        s[r] = p * (dp[r] - dq_d);           // dS^T
      }
#pragma unroll
      for (int eb = 0; eb < NEB; ++eb)
#pragma unroll
        for (int r = 0; r < 16; ++r) dacc[eb] = mfma(ks[kidx(r, half) * LD + eb * 32 + l32], s[r], dacc[eb]);
    }
    __syncthreads();
    if (more) {
      sk.store(Ks);
      sv.store(Vs);
    }
    __syncthreads();
  }
  merge_add<NEB>(Ks, grp, part, lane, dacc);
  if (part == 1 || !qvalid) return;
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

// dQ = scale * dS K from the dS blocks the dK/dV kernel stored (5 products
// per tile pair instead of 7: S and dP are not recomputed). Same work split
// as attn_bwd_dq: 32 queries per wave pair, each wave half of every 64-key
// stage. A wave reads its 32 x 32 block of dS straight into registers: lane
// (query l32, half h) takes keys 16h .. 16h + 15 of its query's row (four
// 16-byte loads, issued a stage ahead), and MFMA step j pairs key 16h + j
// of that row with row 16h + j of K in LDS.
template <int HD>
__global__ __launch_bounds__(kNT, Cfg<HD>::MINW) void attn_bwd_dq_ds(AttnGeom g, const float* __restrict__ K,
                                                                    const float* __restrict__ dsw,
                                                                    float* __restrict__ dQ, int acc) {
  using C = Cfg<HD>;
  constexpr int LD = C::LD, NEB = C::NEB;
  __shared__ __attribute__((aligned(16))) float Ks[kBS * LD];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int grp = wave & 1, part = wave >> 1;
  const int half = lane >> 5, l32 = lane & 31;
  const int qblk = gridDim.y - 1 - blockIdx.y;
  const int bh = blockIdx.x, b = bh / g.heads, h = bh % g.heads;
  const int q0 = qblk * kBQ + grp * 32;
  const int q = q0 + l32;
  const bool qvalid = q < g.q_len;
  const int nq32 = (g.q_len + 31) / 32, nk32 = (g.k_len + 31) / 32;

  f32x16 dacc[NEB];
#pragma unroll
  for (int eb = 0; eb < NEB; ++eb)
#pragma unroll
    for (int r = 0; r < 16; ++r) dacc[eb][r] = 0.f;

  const int64_t qmax = g.q_off + min(g.q_len, qblk * kBQ + kBQ) - 1;
  const int kend = (int)max((int64_t)0, min((int64_t)g.k_len, qmax - g.k_off + 1));
  const int64_t wave_qmax = g.q_off + min(g.q_len - 1, q0 + 31);
  const bool wave_live = q0 < g.q_len;
  // the blocks of this wave's 32 queries (query group q0 / 32 < nq32 when live)
  const float* dsrow = dsw + ((int64_t)bh * nq32 + q0 / 32) * nk32 * 1024 + l32 * 32 + 16 * half;
  // a stage's block is live (stored by the dK/dV kernel, which computes every
  // block with a visible pair) when some key of the wave's half sees some query
  auto live = [&](int kb) { return wave_live && kb < g.k_len && g.k_off + kb <= wave_qmax; };
  auto ds_load = [&](int k0, f32x4(&d)[4]) {
    const int kb = k0 + part * 32;
    if (live(kb)) {
      const float* p = dsrow + (int64_t)(kb / 32) * 1024;
#pragma unroll
      for (int i = 0; i < 4; ++i) d[i] = *reinterpret_cast<const f32x4*>(p + 4 * i);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) d[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  };

  zero_pad<HD, LD>(Ks);
  Stager<HD, LD> sk;
  f32x4 dc[4], dn[4];
  if (kend > 0) {
    sk.load(K, b, h, 0, g.k_len, g.heads);
    ds_load(0, dc);
    sk.store(Ks);
  }
  __syncthreads();
  for (int k0 = 0; k0 < kend; k0 += kBS) {
    const bool more = k0 + kBS < kend;
    if (more) {
      sk.load(K, b, h, k0 + kBS, g.k_len, g.heads);
      ds_load(k0 + kBS, dn);
    }
    const float* ks = Ks + (part * 32 + 16 * half) * LD;
    if (live(k0 + part * 32)) {
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const float dsv = dc[j >> 2][j & 3];
#pragma unroll
        for (int eb = 0; eb < NEB; ++eb) dacc[eb] = mfma(ks[j * LD + eb * 32 + l32], dsv, dacc[eb]);
      }
    }
    __syncthreads();
    if (more) {
      sk.store(Ks);
#pragma unroll
      for (int i = 0; i < 4; ++i) dc[i] = dn[i];
    }
    __syncthreads();
  }
  merge_add<NEB>(Ks, grp, part, lane, dacc);
  if (part == 1 || !qvalid) return;
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

// dK, dV: a group of 32 keys per wave pair; streams query blocks (Q, dO, lse, D).
template <int HD, bool STORE_DS>
__global__ __launch_bounds__(kNT, Cfg<HD>::MINW) void attn_bwd_dkv(AttnGeom g, const float* __restrict__ Q,
                                                      const float* __restrict__ K, const float* __restrict__ V,
                                                      const float* __restrict__ dO, const float* __restrict__ lse,
                                                      const float* __restrict__ Dv, float* __restrict__ dK,
                                                      float* __restrict__ dV, int acc, float* __restrict__ dsw) {
  using C = Cfg<HD>;
  constexpr int LD = C::LD, NKB = C::NKB, NEB = C::NEB;
  __shared__ __attribute__((aligned(16))) float Qs[2 * kBS * LD];   // Q stage, then dO stage
  __shared__ __attribute__((aligned(16))) float KVs[2 * kBS * LD];  // the workgroup's keys: K (pre-scaled), V
  __shared__ __attribute__((aligned(16))) float Ls[kBS];
  __shared__ __attribute__((aligned(16))) float Dd[kBS];
  float* Ds = Qs + kBS * LD;

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int grp = wave & 1, part = wave >> 1;
  const int half = lane >> 5, l32 = lane & 31;
  const int kblk = blockIdx.y;   // early keys see the most queries: launched first
  const int bh = blockIdx.x, b = bh / g.heads, h = bh % g.heads;
  const int k0w = kblk * kBQ + grp * 32;
  const int key = k0w + l32;
  const bool kvalid = key < g.k_len;
  const int64_t kpos = g.k_off + key;

  // the workgroup's 64 keys stay in LDS (registers go to the accumulators);
  // K is stored pre-scaled by scale * log2(e)
  float* Kw = KVs;
  float* Vw = KVs + kBS * LD;
  const float qs = g.scale * kLog2e;
  {
    Stager<HD, LD> sk, sv;
    sk.load(K, b, h, kblk * kBQ, g.k_len, g.heads);
    sv.load(V, b, h, kblk * kBQ, g.k_len, g.heads);
#pragma unroll
    for (int i = 0; i < Stager<HD, LD>::PT; ++i) sk.r[i] *= qs;
    sk.store(Kw);
    sv.store(Vw);
  }
  const float* kown = Kw + (grp * 32 + l32) * LD + 4 * half;
  const float* vown = Vw + (grp * 32 + l32) * LD + 4 * half;
  f32x16 dkv[2 * NEB];  // dK blocks, then dV blocks
#pragma unroll
  for (int n = 0; n < 2 * NEB; ++n)
#pragma unroll
    for (int r = 0; r < 16; ++r) dkv[n][r] = 0.f;

  // first (tile-local) query that can see the workgroup's first key
  const int64_t kmin = g.k_off + (int64_t)kblk * kBQ;
  int qstart = (int)max((int64_t)0, kmin - g.q_off);
  qstart = (qstart / kBS) * kBS;
  const bool wave_live = k0w < g.k_len;
  const int64_t wave_kmin = g.k_off + k0w;
  const int64_t wave_kmax = g.k_off + min(g.k_len - 1, k0w + 31);
  // dS blocks of this wave's 32 keys: block (query group qg) at dsk + qg *
  // ds_qstride; the lane's column l32 and its half's rows 4h .. folded in
  const int nk32 = (g.k_len + 31) / 32;
  const int64_t ds_qstride = (int64_t)nk32 * 1024;
  float* const dsk = STORE_DS ? dsw + ((int64_t)bh * ((g.q_len + 31) / 32) * nk32 + k0w / 32) * 1024 + 4 * half * 32 + l32
                              : nullptr;

  zero_pad<HD, LD>(Qs);
  zero_pad<HD, LD>(Ds);
  Stager<HD, LD> sq, sd;
  float pl = 0.f, pd = 0.f;  // lse / D prefetch (threads < kBS)
  auto load_rows = [&](int qb) {
    sq.load(Q, b, h, qb, g.q_len, g.heads);
    sd.load(dO, b, h, qb, g.q_len, g.heads);
    if ((int)threadIdx.x < kBS) {
      const int qq = qb + threadIdx.x;
      const int64_t s2 = ((int64_t)b * g.heads + h) * g.q_len + qq;
      pl = qq < g.q_len ? lse[s2] * kLog2e : 0.f;
      pd = qq < g.q_len ? Dv[s2] : 0.f;
    }
  };
  auto store_rows = [&]() {
    sq.store(Qs);
    sd.store(Ds);
    if ((int)threadIdx.x < kBS) {
      Ls[threadIdx.x] = pl;
      Dd[threadIdx.x] = pd;
    }
  };
  if (qstart < g.q_len) {
    load_rows(qstart);
    store_rows();
  }
  __syncthreads();
  for (int qb = qstart; qb < g.q_len; qb += kBS) {
    const bool more = qb + kBS < g.q_len;
    const int qb0 = qb + part * 32;
    const float* qsb = Qs + part * 32 * LD;
    const float* dsb = Ds + part * 32 * LD;
    const float* lsb = Ls + part * 32;
    const float* ddb = Dd + part * 32;
    if (wave_live && qb0 < g.q_len && g.q_off + qb0 + 31 >= wave_kmin) {  // not all masked
      f32x16 s, dp;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        s[r] = 0.f;
        dp[r] = 0.f;
      }
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        const f32x4 qf = *reinterpret_cast<const f32x4*>(qsb + l32 * LD + 8 * kb + 4 * half);
        const f32x4 df = *reinterpret_cast<const f32x4*>(dsb + l32 * LD + 8 * kb + 4 * half);
        const f32x4 kf = *reinterpret_cast<const f32x4*>(kown + 8 * kb);
        const f32x4 vf = *reinterpret_cast<const f32x4*>(vown + 8 * kb);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          s = mfma(qf[i], kf[i], s);     // S = Q K^T (log2 units); lane owns a key column
          dp = mfma(df[i], vf[i], dp);   // dP = dO V^T
        }
      }
      const bool edge = qb0 + 31 >= g.q_len || g.q_off + qb0 < wave_kmax;
      // lse (log2 units) and D of the 16 query rows held by this lane's
      // registers: rows 8*(r/4) + 4*half + r%4, i.e. four 16-byte reads each
      // (D read only after the dV products, so the two are not live together)
      f32x4 lv[4], dv[4];
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) lv[g4] = *reinterpret_cast<const f32x4*>(lsb + 8 * g4 + 4 * half);
      // query row ql of this block sees the lane's key iff ql >= dlim
      const int dlim = (int)max((int64_t)-1, min((int64_t)32, kpos - g.q_off - qb0));
      const int qlim = g.q_len - qb0;  // rows >= qlim are past the tile
#pragma unroll
      for (int r = 0; r < 16; ++r) {         // P, in place of S (branch-free: masked entries select 0)
        const int ql = kidx(r, half);
        const bool ok = kvalid & (!edge | ((ql < qlim) & (ql >= dlim)));
        const float p = exp2_hw(s[r] - lv[r >> 2][r & 3]);
        s[r] = ok ? p : 0.f;
      }
#pragma unroll
      for (int eb = 0; eb < NEB; ++eb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          dkv[NEB + eb] = mfma(dsb[kidx(r, half) * LD + eb * 32 + l32], s[r], dkv[NEB + eb]);  // dV^T += dO^T P
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) dv[g4] = *reinterpret_cast<const f32x4*>(ddb + 8 * g4 + 4 * half);
#pragma unroll
      for (int r = 0; r < 16; ++r) s[r] *= dp[r] - dv[r >> 2][r & 3];  // dS, in place of P
      if constexpr (STORE_DS) {  // the 32 x 32 block of dS for the dQ kernel, row-major by query (two 128-byte rows per store)
        float* blk = dsk + (int64_t)(qb0 / 32) * ds_qstride;
#pragma unroll
        for (int r = 0; r < 16; ++r) blk[(8 * (r >> 2) + (r & 3)) * 32] = s[r];
      }
#pragma unroll
      for (int eb = 0; eb < NEB; ++eb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          dkv[eb] = mfma(qsb[kidx(r, half) * LD + eb * 32 + l32], s[r], dkv[eb]);  // dK^T += Q^T dS
    }
    // the next stage's loads are issued after the MFMAs, so the staging
    // registers are not live across them (two workgroups fit per CU; the
    // other one's MFMAs cover this load's latency)
    if (more) load_rows(qb + kBS);
    __syncthreads();
    if (more) store_rows();
    __syncthreads();
  }
  merge_add<2 * NEB>(Qs, grp, part, lane, dkv);
  if (part == 1 || !kvalid) return;
  float* krow = dK + row_off(b, key, h, g.k_len, g.heads, HD);
  float* vrow = dV + row_off(b, key, h, g.k_len, g.heads, HD);
#pragma unroll
  for (int eb = 0; eb < NEB; ++eb)
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
      const int e = eb * 32 + 8 * gq + 4 * half;
      if (e < HD) {
        f32x4 a = {dkv[eb][4 * gq], dkv[eb][4 * gq + 1], dkv[eb][4 * gq + 2], dkv[eb][4 * gq + 3]};
        f32x4 c = {dkv[NEB + eb][4 * gq], dkv[NEB + eb][4 * gq + 1], dkv[NEB + eb][4 * gq + 2],
                   dkv[NEB + eb][4 * gq + 3]};
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
  // grid: x = (batch, head) pairs, y = 64-row blocks of the query (key) axis
  if (batch * heads > INT32_MAX || (q_len + kBQ - 1) / kBQ > 65535 || (k_len + kBQ - 1) / kBQ > 65535)
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
  dim3 grid((unsigned)(batch * heads), (unsigned)((q_len + kBQ - 1) / kBQ)), block(kNT);
  hipStream_t s = tt::as_stream(stream);
  switch (hd) {
    case 16: hipLaunchKernelGGL(attn_fwd<16>, grid, block, 0, s, g, Q, K, V, O, ml, lse, first, last); break;
    case 32: hipLaunchKernelGGL(attn_fwd<32>, grid, block, 0, s, g, Q, K, V, O, ml, lse, first, last); break;
    case 64: hipLaunchKernelGGL(attn_fwd<64>, grid, block, 0, s, g, Q, K, V, O, ml, lse, first, last); break;
    default: hipLaunchKernelGGL(attn_fwd<128>, grid, block, 0, s, g, Q, K, V, O, ml, lse, first, last); break;
  }
  return tt::launch_status("tile_attention_fwd");
}

extern "C" size_t tile_attention_bwd_workspace(int64_t batch, int64_t heads, int64_t q_len, int64_t k_len) {
  if (batch <= 0 || heads <= 0 || q_len <= 0 || k_len <= 0) return 0;
  return (size_t)(batch * heads) * (size_t)((q_len + 31) / 32) * (size_t)((k_len + 31) / 32) * 1024 * sizeof(float);
}

extern "C" int tile_attention_bwd_ws(void* stream, int phase, int64_t batch, int64_t heads, int64_t q_len,
                                     int64_t k_len, int64_t hd, int64_t q_off, int64_t k_off, const float* Q,
                                     const float* K, const float* V, const float* O, const float* dO, const float* lse,
                                     float* Dvec, float* dQ, float* dK, float* dV, int acc_dq, int acc_dkv,
                                     float scale, void* workspace, size_t workspace_bytes) {
  if (int rc = check_geom("tile_attention_bwd", batch, heads, q_len, k_len, hd)) return rc;
  if (batch == 0 || heads == 0) return TT_OK;
  hipStream_t s = tt::as_stream(stream);
  if (phase == TT_ATT_PREP) {
    if (q_len == 0) return TT_OK;
    if (!O || !dO || !Dvec) return tt::fail(TT_ERR_ARG, "tile_attention_bwd(PREP): null tensor");
    if (!aligned16(O) || !aligned16(dO)) return tt::fail(TT_ERR_ARG, "tile_attention_bwd: 16-byte alignment required");
    const int64_t rows = batch * q_len * heads;
    const dim3 grid((unsigned)((rows * (hd / 4) + 255) / 256)), block(256);
    switch (hd) {
      case 16: hipLaunchKernelGGL(attn_prep<4>, grid, block, 0, s, (int)batch, (int)heads, (int)q_len, O, dO, Dvec); break;
      case 32: hipLaunchKernelGGL(attn_prep<8>, grid, block, 0, s, (int)batch, (int)heads, (int)q_len, O, dO, Dvec); break;
      case 64: hipLaunchKernelGGL(attn_prep<16>, grid, block, 0, s, (int)batch, (int)heads, (int)q_len, O, dO, Dvec); break;
      default: hipLaunchKernelGGL(attn_prep<32>, grid, block, 0, s, (int)batch, (int)heads, (int)q_len, O, dO, Dvec); break;
    }
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
  dim3 gq((unsigned)(batch * heads), (unsigned)((q_len + kBQ - 1) / kBQ));
  dim3 gk((unsigned)(batch * heads), (unsigned)((k_len + kBQ - 1) / kBQ));
  dim3 block(kNT);
  const bool stored = workspace && aligned16(workspace) &&
                      workspace_bytes >= tile_attention_bwd_workspace(batch, heads, q_len, k_len);
  float* dsw = stored ? (float*)workspace : nullptr;
  // with a workspace the dK/dV kernel stores dS and the dQ kernel reads it;
  // without, the dQ kernel recomputes S and dP
#define TT_ATT_BWD(HD)                                                                                          \
  if (stored) {                                                                                                 \
    hipLaunchKernelGGL((attn_bwd_dkv<HD, true>), gk, block, 0, s, g, Q, K, V, dO, lse, Dvec, dK, dV, acc_dkv, dsw); \
    hipLaunchKernelGGL(attn_bwd_dq_ds<HD>, gq, block, 0, s, g, K, (const float*)dsw, dQ, acc_dq);               \
  } else {                                                                                                      \
    hipLaunchKernelGGL(attn_bwd_dq<HD>, gq, block, 0, s, g, Q, K, V, dO, lse, Dvec, dQ, acc_dq);               \
    hipLaunchKernelGGL((attn_bwd_dkv<HD, false>), gk, block, 0, s, g, Q, K, V, dO, lse, Dvec, dK, dV, acc_dkv,    \
                       nullptr);                                                                                \
  }
  switch (hd) {
    case 16: TT_ATT_BWD(16); break;
    case 32: TT_ATT_BWD(32); break;
    case 64: TT_ATT_BWD(64); break;
    default: TT_ATT_BWD(128); break;
  }
#undef TT_ATT_BWD
  return tt::launch_status("tile_attention_bwd(GRAD)");
}

extern "C" int tile_attention_bwd(void* stream, int phase, int64_t batch, int64_t heads, int64_t q_len, int64_t k_len,
                                  int64_t hd, int64_t q_off, int64_t k_off, const float* Q, const float* K,
                                  const float* V, const float* O, const float* dO, const float* lse, float* Dvec,
                                  float* dQ, float* dK, float* dV, int acc_dq, int acc_dkv, float scale) {
  return tile_attention_bwd_ws(stream, phase, batch, heads, q_len, k_len, hd, q_off, k_off, Q, K, V, O, dO, lse, Dvec,
                               dQ, dK, dV, acc_dq, acc_dkv, scale, nullptr, 0);
}
