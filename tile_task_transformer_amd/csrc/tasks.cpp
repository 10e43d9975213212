// Task-level tile ops (tt_submit): each op's tile list, access modes,
// shape checks and launch. The GPT2 step submits its tasks through the
// same submit_op, so the public interface and the model share one code path.
#include "tasks.hpp"

#include <algorithm>
#include <cstring>

namespace tt {

namespace {

float* Fp(const TileArg& a) { return (float*)a.t->dev(a.lin); }
const int32_t* Ip(const TileArg& a) { return (const int32_t*)a.t->dev(a.lin); }
void matv(const TileArg& a, int64_t* r, int64_t* c) { a.t->mat(a.lin, r, c); }
int64_t elems(const TileArg& a) { return a.t->tile_elems(a.lin); }
Access acc_of(const TileArg& a, int mode) { return Access{TileRef{a.t, a.lin}, mode}; }

constexpr size_t kAlign = 256;
size_t align_up(size_t b) { return (b + kAlign - 1) & ~(kAlign - 1); }
constexpr size_t kSplitCap = size_t(256) << 20;  // split-K partials per stream workspace

int need_f32(const TileArg* t, int n, const char* op) {
  for (int i = 0; i < n; ++i)
    if (t[i].t->dtype != TT_F32) return fail(TT_ERR_ARG, "%s: tile %d must be f32", op, i);
  return TT_OK;
}

int need_i32(const TileArg& t, const char* op, const char* what) {
  if (t.t->dtype != TT_I32) return fail(TT_ERR_ARG, "%s: %s must be i32", op, what);
  return TT_OK;
}

template <class S>
int scal(const void* p, size_t size, const char* op, S* out) {
  if (!p || size != sizeof(S)) return fail(TT_ERR_ARG, "%s: scalars must be a %zu-byte struct", op, sizeof(S));
  memcpy(out, p, sizeof(S));
  return TT_OK;
}

// vocab offset of a logits tile: its index along the last axis times the tile size
int64_t last_axis_offset(const TileArg& a) {
  const tt_tensor* t = a.t;
  int64_t l = a.lin, idx = 0;
  for (int d = 0; d < t->ndim; ++d) {
    idx = l % t->grid[d];
    l /= t->grid[d];
  }
  return idx * t->tshape[t->ndim - 1];
}

// ---------------------------------------------------------------- GEMM

int op_gemm(tt_ctx* ctx, const TileArg* T, int n, const tt_op_gemm& q, const char* label, bool grow) {
  const char* nm = "TT_OP_GEMM";
  const int epi = q.epilogue;
  if (epi & ~(TT_EPI_BIAS | TT_EPI_RES | TT_EPI_GELU | TT_EPI_GELU_BWD))
    return fail(TT_ERR_ARG, "%s: unknown epilogue bits", nm);
  if ((epi & TT_EPI_GELU) && (epi & TT_EPI_GELU_BWD)) return fail(TT_ERR_ARG, "%s: GELU and GELU_BWD", nm);
  const bool has_bias = epi & TT_EPI_BIAS, has_res = epi & TT_EPI_RES;
  const bool has_aux = epi & (TT_EPI_GELU | TT_EPI_GELU_BWD), gelu = epi & TT_EPI_GELU;
  const int want = 3 + has_bias + has_res + has_aux;
  if (n != want) return fail(TT_ERR_ARG, "%s: %d tiles given, the epilogue needs %d", nm, n, want);
  if (int rc = need_f32(T, n, nm)) return rc;
  int64_t ar, ac, br, bc, cr, cc;
  matv(T[0], &ar, &ac);
  matv(T[1], &br, &bc);
  matv(T[2], &cr, &cc);
  const int64_t m = q.transA ? ac : ar, k = q.transA ? ar : ac;
  const int64_t kb = q.transB ? bc : br, nn = q.transB ? br : bc;
  if (k != kb || m != cr || nn != cc)
    return fail(TT_ERR_SHAPE, "%s: op(A) %lldx%lld, op(B) %lldx%lld, C %lldx%lld", nm, (long long)m, (long long)k,
                (long long)kb, (long long)nn, (long long)cr, (long long)cc);
  int at = 3;
  TileArg bias, res, aux;
  if (has_bias) {
    bias = T[at++];
    if (elems(bias) != nn) return fail(TT_ERR_SHAPE, "%s: bias has %lld elements, C has %lld columns", nm,
                                       (long long)elems(bias), (long long)nn);
  }
  int64_t ldr = 0, ldaux = 0;
  if (has_res) {
    res = T[at++];
    int64_t r, c;
    matv(res, &r, &c);
    if (r != m || c != nn) return fail(TT_ERR_SHAPE, "%s: residual tile is not %lldx%lld", nm, (long long)m,
                                       (long long)nn);
    ldr = c;
  }
  if (has_aux) {
    aux = T[at++];
    int64_t r, c;
    matv(aux, &r, &c);
    if (r != m || c != nn) return fail(TT_ERR_SHAPE, "%s: aux tile is not %lldx%lld", nm, (long long)m, (long long)nn);
    ldaux = c;
  }
  std::vector<Access> acc = {acc_of(T[0], TT_R), acc_of(T[1], TT_R),
                             acc_of(T[2], (q.beta == 0.f || gelu) ? TT_W : TT_RW)};
  if (has_bias) acc.push_back(acc_of(bias, TT_R));
  if (has_res) acc.push_back(acc_of(res, TT_R));
  if (has_aux) acc.push_back(acc_of(aux, gelu ? (q.beta == 0.f ? TT_W : TT_RW) : TT_R));
  if (q.split_k && grow)
    if (int rc = ctx->ensure_workspace(std::min(kSplitCap, tile_gemm_workspace(m, nn, k)))) return rc;
  const TileArg A = T[0], B = T[1], C = T[2];
  const tt_op_gemm p = q;
  return ctx->submit(label ? label : "gemm", std::move(acc), [=](hipStream_t s, void* ws) {
    const bool split = p.split_k && ws;
    return tile_gemm_ws(s, p.transA, p.transB, m, nn, k, p.alpha, Fp(A), ac, Fp(B), bc, p.beta, Fp(C), cc,
                        p.epilogue, has_bias ? Fp(bias) : nullptr, has_res ? Fp(res) : nullptr, ldr,
                        has_aux ? Fp(aux) : nullptr, ldaux, split ? ws : nullptr, split ? ctx->workspace_bytes : 0);
  }, 2.0 * m * nn * k);
}

int op_gemm_batch_xstats(tt_ctx* ctx, const TileArg* T, int n, const tt_op_gemm& q, const char* label);

int op_gemm_batch(tt_ctx* ctx, const TileArg* T, int n, const tt_op_gemm& q, const char* label, bool grow) {
  const char* nm = "TT_OP_GEMM_BATCH";
  if (q.epilogue == TT_EPI_XSTATS) return op_gemm_batch_xstats(ctx, T, n, q, label);
  if (n < 3 || n % 3) return fail(TT_ERR_ARG, "%s: needs (A, B, C) triples", nm);
  if (q.epilogue != TT_EPI_NONE) return fail(TT_ERR_ARG, "%s: no epilogue", nm);
  if (int rc = need_f32(T, n, nm)) return rc;
  const int cnt = n / 3;
  std::vector<int64_t> m(cnt), nn(cnt), lda(cnt), ldb(cnt), ldc(cnt);
  int64_t k = -1;
  std::vector<Access> acc;
  double flops = 0;
  for (int u = 0; u < cnt; ++u) {
    int64_t ar, ac, br, bc, cr, cc;
    matv(T[3 * u], &ar, &ac);
    matv(T[3 * u + 1], &br, &bc);
    matv(T[3 * u + 2], &cr, &cc);
    const int64_t mu = q.transA ? ac : ar, ku = q.transA ? ar : ac;
    const int64_t kb = q.transB ? bc : br, nu = q.transB ? br : bc;
    if (ku != kb || mu != cr || nu != cc || (k >= 0 && ku != k))
      return fail(TT_ERR_SHAPE, "%s: product %d: op(A) %lldx%lld, op(B) %lldx%lld, C %lldx%lld (K must be shared)", nm,
                  u, (long long)mu, (long long)ku, (long long)kb, (long long)nu, (long long)cr, (long long)cc);
    k = ku;
    m[u] = mu;
    nn[u] = nu;
    lda[u] = ac;
    ldb[u] = bc;
    ldc[u] = cc;
    acc.push_back(acc_of(T[3 * u], TT_R));
    acc.push_back(acc_of(T[3 * u + 1], TT_R));
    acc.push_back(acc_of(T[3 * u + 2], q.beta == 0.f ? TT_W : TT_RW));
    flops += 2.0 * mu * nu * ku;
  }
  for (int u = 0; u < cnt; ++u)
    for (int w = u + 1; w < cnt; ++w)
      if (T[3 * u + 2].t == T[3 * w + 2].t && T[3 * u + 2].lin == T[3 * w + 2].lin)
        return fail(TT_ERR_ARG, "%s: products %d and %d write the same C tile", nm, u, w);
  if (q.split_k && grow)
    if (int rc = ctx->ensure_workspace(std::min(kSplitCap, tile_gemm_batch_workspace(cnt, m.data(), nn.data(), k))))
      return rc;
  std::vector<TileArg> tl(T, T + n);
  const tt_op_gemm p = q;
  return ctx->submit(label ? label : "gemm_batch", std::move(acc), [=](hipStream_t s, void* ws) {
    std::vector<const float*> A(cnt), B(cnt);
    std::vector<float*> C(cnt);
    for (int u = 0; u < cnt; ++u) {
      A[u] = Fp(tl[3 * u]);
      B[u] = Fp(tl[3 * u + 1]);
      C[u] = Fp(tl[3 * u + 2]);
    }
    const bool split = p.split_k && ws;
    return tile_gemm_batch_ws(s, cnt, p.transA, p.transB, m.data(), nn.data(), k, p.alpha, A.data(), lda.data(),
                              B.data(), ldb.data(), p.beta, C.data(), ldc.data(), split ? ws : nullptr,
                              split ? ctx->workspace_bytes : 0);
  }, flops);
}

// the tied head's vocab-tile products with the cross-entropy statistics in
// the epilogue: tiles (A, B, C) per product, labels, then one partials tile
// per product (tile_gemm_batch_xstats)
int op_gemm_batch_xstats(tt_ctx* ctx, const TileArg* T, int n, const tt_op_gemm& q, const char* label) {
  const char* nm = "TT_OP_GEMM_BATCH (TT_EPI_XSTATS)";
  if (n < 5 || n % 4 != 1) return fail(TT_ERR_ARG, "%s: needs (A, B, C) triples, labels, one partials tile each", nm);
  const int cnt = (n - 1) / 4;
  if (q.transA) return fail(TT_ERR_ARG, "%s: transA must be 0", nm);
  if (int rc = need_f32(T, 3 * cnt, nm)) return rc;
  if (int rc = need_i32(T[3 * cnt], nm, "labels")) return rc;
  if (int rc = need_f32(T + 3 * cnt + 1, cnt, nm)) return rc;
  const tt_tensor* zt = T[2].t;
  const int64_t v_tile = zt->tshape[zt->ndim - 1], v_off0 = last_axis_offset(T[2]);
  std::vector<int64_t> nn(cnt), lda(cnt), ldb(cnt), ldc(cnt);
  int64_t m = -1, k = -1;
  std::vector<Access> acc;
  double flops = 0;
  const int64_t groups = (v_tile + 63) / 64;
  for (int u = 0; u < cnt; ++u) {
    const TileArg &A = T[3 * u], &B = T[3 * u + 1], &C = T[3 * u + 2], &P = T[3 * cnt + 1 + u];
    int64_t ar, ac, br, bc, cr, cc;
    matv(A, &ar, &ac);
    matv(B, &br, &bc);
    matv(C, &cr, &cc);
    const int64_t kb = q.transB ? bc : br, nu = q.transB ? br : bc;
    if (ac != kb || nu != cc || ar != cr || (m >= 0 && (ar != m || ac != k)))
      return fail(TT_ERR_SHAPE, "%s: product %d does not match (shared m and K)", nm, u);
    if (C.t != zt || last_axis_offset(C) != v_off0 + u * v_tile)
      return fail(TT_ERR_ARG, "%s: C tiles must be consecutive vocab tiles of one tensor", nm);
    if (elems(P) < groups * ar * 3)
      return fail(TT_ERR_SHAPE, "%s: partials tile %d holds %lld floats, %lld needed", nm, u, (long long)elems(P),
                  (long long)(groups * ar * 3));
    m = ar;
    k = ac;
    nn[u] = nu;
    lda[u] = ac;
    ldb[u] = bc;
    ldc[u] = cc;
    acc.push_back(acc_of(A, TT_R));
    acc.push_back(acc_of(B, TT_R));
    acc.push_back(acc_of(C, q.beta == 0.f ? TT_W : TT_RW));
    acc.push_back(acc_of(P, TT_W));
    flops += 2.0 * ar * nu * ac;
  }
  if (elems(T[3 * cnt]) < m) return fail(TT_ERR_SHAPE, "%s: labels tile smaller than the rows", nm);
  acc.push_back(acc_of(T[3 * cnt], TT_R));
  std::vector<TileArg> tl(T, T + n);
  const tt_op_gemm p = q;
  return ctx->submit(label ? label : "gemm_batch_xstats", std::move(acc), [=](hipStream_t s, void*) {
    std::vector<const float*> A(cnt), B(cnt);
    std::vector<float*> C(cnt);
    for (int u = 0; u < cnt; ++u) {
      A[u] = Fp(tl[3 * u]);
      B[u] = Fp(tl[3 * u + 1]);
      C[u] = Fp(tl[3 * u + 2]);
    }
    float* p0 = Fp(tl[3 * cnt + 1]);
    const int64_t stride = cnt > 1 ? Fp(tl[3 * cnt + 2]) - p0 : groups * m * 3;
    for (int u = 0; u < cnt; ++u)
      if (Fp(tl[3 * cnt + 1 + u]) != p0 + u * stride)
        return fail(TT_ERR_SHAPE, "%s: the partials tiles are not equally spaced", "TT_OP_GEMM_BATCH (TT_EPI_XSTATS)");
    return tile_gemm_batch_xstats(s, cnt, p.transB, m, nn.data(), k, p.alpha, A.data(), lda.data(), B.data(),
                                  ldb.data(), p.beta, C.data(), ldc.data(),
                                  (const int32_t*)tl[3 * cnt].t->dev(tl[3 * cnt].lin), v_off0, v_tile, p0, stride);
  }, flops);
}

int op_gemm_ksum(tt_ctx* ctx, const TileArg* T, int n, const tt_op_gemm& q, const char* label, bool grow) {
  const char* nm = "TT_OP_GEMM_KSUM";
  const int epi = q.epilogue;
  if (q.transA) return fail(TT_ERR_ARG, "%s: transA must be 0", nm);
  if (epi & ~(TT_EPI_BIAS | TT_EPI_RES | TT_EPI_GELU | TT_EPI_GELU_BWD))
    return fail(TT_ERR_ARG, "%s: unknown epilogue bits", nm);
  if ((epi & TT_EPI_GELU) && (epi & TT_EPI_GELU_BWD)) return fail(TT_ERR_ARG, "%s: GELU and GELU_BWD", nm);
  const bool has_bias = epi & TT_EPI_BIAS, has_res = epi & TT_EPI_RES;
  const bool has_aux = epi & (TT_EPI_GELU | TT_EPI_GELU_BWD), gelu = epi & TT_EPI_GELU;
  const int ne = 1 + has_bias + has_res + has_aux;
  if (n < ne + 2 || (n - ne) % 2) return fail(TT_ERR_ARG, "%s: needs C, the epilogue's tiles and (A, B) pairs", nm);
  if (int rc = need_f32(T, n, nm)) return rc;
  const int cnt = (n - ne) / 2;
  int64_t dr, dc;
  matv(T[0], &dr, &dc);
  int at = 1;
  TileArg bias, res, aux;
  int64_t ldr = 0, ldaux = 0;
  if (has_bias) {
    bias = T[at++];
    if (elems(bias) != dc) return fail(TT_ERR_SHAPE, "%s: bias has %lld elements, C has %lld columns", nm,
                                       (long long)elems(bias), (long long)dc);
  }
  if (has_res) {
    res = T[at++];
    int64_t r, c;
    matv(res, &r, &c);
    if (r != dr || c != dc) return fail(TT_ERR_SHAPE, "%s: residual tile is not %lldx%lld", nm, (long long)dr,
                                        (long long)dc);
    ldr = c;
  }
  if (has_aux) {
    aux = T[at++];
    int64_t r, c;
    matv(aux, &r, &c);
    if (r != dr || c != dc) return fail(TT_ERR_SHAPE, "%s: aux tile is not %lldx%lld", nm, (long long)dr,
                                        (long long)dc);
    ldaux = c;
  }
  std::vector<int64_t> ks(cnt), lda(cnt), ldb(cnt);
  std::vector<Access> acc;
  double flops = 0;
  for (int u = 0; u < cnt; ++u) {
    int64_t ar, ac, br, bc;
    matv(T[ne + 2 * u], &ar, &ac);
    matv(T[ne + 1 + 2 * u], &br, &bc);
    const int64_t kb = q.transB ? bc : br, nb = q.transB ? br : bc;
    if (ar != dr || kb != ac || nb != dc)
      return fail(TT_ERR_SHAPE, "%s: pair %d (%lldx%lld, %lldx%lld) does not match C %lldx%lld", nm, u, (long long)ar,
                  (long long)ac, (long long)br, (long long)bc, (long long)dr, (long long)dc);
    ks[u] = ac;
    lda[u] = ac;
    ldb[u] = bc;
    acc.push_back(acc_of(T[ne + 2 * u], TT_R));
    acc.push_back(acc_of(T[ne + 1 + 2 * u], TT_R));
    flops += 2.0 * dr * dc * ac;
  }
  acc.push_back(acc_of(T[0], (q.beta == 0.f || gelu) ? TT_W : TT_RW));
  if (has_bias) acc.push_back(acc_of(bias, TT_R));
  if (has_res) acc.push_back(acc_of(res, TT_R));
  if (has_aux) acc.push_back(acc_of(aux, gelu ? (q.beta == 0.f ? TT_W : TT_RW) : TT_R));
  if (q.split_k && grow)
    if (int rc = ctx->ensure_workspace(std::min(kSplitCap, tile_gemm_ksum_workspace(dr, dc)))) return rc;
  std::vector<TileArg> tl(T, T + n);
  const tt_op_gemm p = q;
  return ctx->submit(label ? label : "gemm_ksum", std::move(acc), [=](hipStream_t s, void* ws) {
    std::vector<const float*> A(cnt), B(cnt);
    for (int u = 0; u < cnt; ++u) {
      A[u] = Fp(tl[ne + 2 * u]);
      B[u] = Fp(tl[ne + 1 + 2 * u]);
    }
    float* bp = has_bias ? Fp(bias) : nullptr;
    float* rp = has_res ? Fp(res) : nullptr;
    float* xp = has_aux ? Fp(aux) : nullptr;
    const bool split = p.split_k && ws;
    const int rc = tile_gemm_ksum_ws(s, cnt, p.transB, dr, dc, ks.data(), p.alpha, A.data(), lda.data(), B.data(),
                                     ldb.data(), p.beta, Fp(tl[0]), dc, p.epilogue, bp, rp, ldr, xp, ldaux,
                                     split ? ws : nullptr, split ? ctx->workspace_bytes : 0);
    if (rc != TT_ERR_UNSUPPORTED) return rc;
    // the epilogue could not be fused into one long-K launch: a chain of
    // accumulating products inside this task, the residual with the first,
    // bias and activation with the last (the GELU chain accumulates the
    // pre-activation in aux)
    clear_error();
    const size_t wsb = p.split_k && ws ? ctx->workspace_bytes : 0;
    for (int u = 0; u < cnt; ++u) {
      const bool first = u == 0, last = u == cnt - 1;
      const int ep = (first ? (p.epilogue & TT_EPI_RES) : 0) |
                     (last ? (p.epilogue & (TT_EPI_BIAS | TT_EPI_GELU | TT_EPI_GELU_BWD)) : 0);
      const bool to_aux = gelu && !last;
      float* tgt = to_aux ? xp : Fp(tl[0]);
      const int64_t ldt = to_aux ? ldaux : dc;
      if (int rc2 = tile_gemm_ws(s, 0, p.transB, dr, dc, ks[u], p.alpha, A[u], lda[u], B[u], ldb[u],
                                 first ? p.beta : 1.f, tgt, ldt, ep, bp, rp, ldr, xp, ldaux, wsb ? ws : nullptr, wsb))
        return rc2;
    }
    return TT_OK;
  }, flops);
}

// ------------------------------------------------------------ LayerNorm

// the one-pass multi-tile kernels take tiles as wide as the first but a
// narrower last one, widths multiples of 4, at most 16384 features
bool ln_one_pass(const std::vector<int64_t>& cols) {
  int64_t total = 0;
  for (size_t e = 0; e < cols.size(); ++e) {
    if (cols[e] < 4 || cols[e] % 4 || cols[e] > cols[0] || (e + 1 < cols.size() && cols[e] != cols[0])) return false;
    total += cols[e];
  }
  return cols.size() >= 2 && cols.size() <= 16 && total <= 16384;
}

bool all_aligned(const std::vector<const void*>& ps) {
  for (const void* p : ps)
    if (reinterpret_cast<uintptr_t>(p) & 15) return false;
  return true;
}

int op_ln_fwd(tt_ctx* ctx, const TileArg* T, int n, const tt_op_layernorm& q, const char* label, bool grow) {
  const char* nm = "TT_OP_LAYERNORM_FWD";
  if (n < 5 || (n - 1) % 4) return fail(TT_ERR_ARG, "%s: needs 4n+1 tiles", nm);
  if (int rc = need_f32(T, n, nm)) return rc;
  const int ne = (n - 1) / 4;
  const TileArg* X = T;
  const TileArg* Gm = T + ne;
  const TileArg* Bt = T + 2 * ne;
  const TileArg stats = T[3 * ne];
  const TileArg* Y = T + 3 * ne + 1;
  int64_t rows = -1, total = 0;
  std::vector<int64_t> cols(ne);
  std::vector<Access> acc;
  for (int e = 0; e < ne; ++e) {
    int64_t r, c, yr, yc;
    matv(X[e], &r, &c);
    matv(Y[e], &yr, &yc);
    if ((rows >= 0 && r != rows) || yr != r || yc != c || elems(Gm[e]) != c || elems(Bt[e]) != c)
      return fail(TT_ERR_SHAPE, "%s: feature tile %d: x %lldx%lld, y %lldx%lld, gamma %lld, beta %lld", nm, e,
                  (long long)r, (long long)c, (long long)yr, (long long)yc, (long long)elems(Gm[e]),
                  (long long)elems(Bt[e]));
    rows = r;
    cols[e] = c;
    total += c;
    acc.push_back(acc_of(X[e], TT_R));
    acc.push_back(acc_of(Gm[e], TT_R));
    acc.push_back(acc_of(Bt[e], TT_R));
    acc.push_back(acc_of(Y[e], TT_W));
  }
  if (elems(stats) < 2 * rows) return fail(TT_ERR_SHAPE, "%s: stats tile holds fewer than 2*rows floats", nm);
  acc.push_back(acc_of(stats, TT_W));
  const size_t need = layernorm_fwd_workspace(ne, rows);
  if (need && grow)
    if (int rc = ctx->ensure_workspace(need)) return rc;
  std::vector<TileArg> tl(T, T + n);
  const float eps = q.eps;
  return ctx->submit(label ? label : "ln_fwd", std::move(acc), [=](hipStream_t s, void* ws) {
    const TileArg* x = tl.data();
    const TileArg* gm = x + ne;
    const TileArg* bt = x + 2 * ne;
    const TileArg st = x[3 * ne];
    const TileArg* y = x + 3 * ne + 1;
    if (ne == 1)
      return tile_layernorm_fwd(s, TT_LN_FUSED, rows, cols[0], Fp(x[0]), cols[0], Fp(gm[0]), Fp(bt[0]), nullptr, 0,
                                0, Fp(st), Fp(y[0]), cols[0], eps);
    if (ln_one_pass(cols)) {
      std::vector<const float*> xs(ne), gs(ne), bs(ne);
      std::vector<float*> ys(ne);
      std::vector<const void*> all;
      for (int e = 0; e < ne; ++e) {
        xs[e] = Fp(x[e]);
        gs[e] = Fp(gm[e]);
        bs[e] = Fp(bt[e]);
        ys[e] = Fp(y[e]);
        all.insert(all.end(), {xs[e], gs[e], bs[e], ys[e]});
      }
      if (all_aligned(all))
        return tile_layernorm_fwd_multi(s, ne, rows, cols.data(), xs.data(), gs.data(), bs.data(), Fp(st), ys.data(),
                                        eps);
    }
    if (!ws || ctx->workspace_bytes < need)
      return fail(TT_ERR_STATE, "layernorm: the stream workspace holds %zu bytes, %zu needed", ctx->workspace_bytes,
                  need);
    float* parts = (float*)ws;
    for (int e = 0; e < ne; ++e)
      if (int rc = tile_layernorm_fwd(s, TT_LN_PARTIAL, rows, cols[e], Fp(x[e]), cols[e], nullptr, nullptr,
                                      parts + (size_t)e * rows * 3, 0, 0, nullptr, nullptr, 0, eps))
        return rc;
    if (int rc = tile_layernorm_fwd(s, TT_LN_MERGE, rows, 0, nullptr, 0, nullptr, nullptr, parts, ne, rows * 3,
                                    Fp(st), nullptr, 0, eps))
      return rc;
    for (int e = 0; e < ne; ++e)
      if (int rc = tile_layernorm_fwd(s, TT_LN_APPLY, rows, cols[e], Fp(x[e]), cols[e], Fp(gm[e]), Fp(bt[e]), nullptr,
                                      0, 0, Fp(st), Fp(y[e]), cols[e], eps))
        return rc;
    return TT_OK;
  });
}

int op_ln_bwd(tt_ctx* ctx, const TileArg* T, int n, const tt_op_layernorm& q, const char* label, bool grow) {
  const char* nm = "TT_OP_LAYERNORM_BWD";
  if (n < 7 || (n - 1) % 6) return fail(TT_ERR_ARG, "%s: needs 6n+1 tiles", nm);
  if (int rc = need_f32(T, n, nm)) return rc;
  const int ne = (n - 1) / 6;
  const TileArg* DY = T;
  const TileArg* X = T + ne;
  const TileArg* Gm = T + 2 * ne;
  const TileArg stats = T[3 * ne];
  const TileArg* DX = T + 3 * ne + 1;
  const TileArg* DG = T + 4 * ne + 1;
  const TileArg* DB = T + 5 * ne + 1;
  int64_t rows = -1, total = 0, widest = 0;
  std::vector<int64_t> cols(ne);
  std::vector<Access> acc;
  for (int e = 0; e < ne; ++e) {
    int64_t r, c, dyr, dyc, dxr, dxc;
    matv(X[e], &r, &c);
    matv(DY[e], &dyr, &dyc);
    matv(DX[e], &dxr, &dxc);
    if ((rows >= 0 && r != rows) || dyr != r || dyc != c || dxr != r || dxc != c || elems(Gm[e]) != c ||
        elems(DG[e]) != c || elems(DB[e]) != c)
      return fail(TT_ERR_SHAPE, "%s: feature tile %d: shapes of dy, x, dx, gamma, dgamma, dbeta disagree", nm, e);
    rows = r;
    cols[e] = c;
    total += c;
    widest = std::max(widest, c);
    acc.push_back(acc_of(DY[e], TT_R));
    acc.push_back(acc_of(X[e], TT_R));
    acc.push_back(acc_of(Gm[e], TT_R));
    acc.push_back(acc_of(DX[e], q.dx_acc ? TT_RW : TT_W));
    acc.push_back(acc_of(DG[e], TT_RW));
    acc.push_back(acc_of(DB[e], TT_RW));
  }
  if (elems(stats) < 2 * rows) return fail(TT_ERR_SHAPE, "%s: stats tile holds fewer than 2*rows floats", nm);
  acc.push_back(acc_of(stats, TT_R));
  const size_t need = layernorm_bwd_workspace(ne, rows, widest);
  if (grow)
    if (int rc = ctx->ensure_workspace(need)) return rc;
  std::vector<TileArg> tl(T, T + n);
  const int dx_acc = q.dx_acc;
  return ctx->submit(label ? label : "ln_bwd", std::move(acc), [=](hipStream_t s, void* ws) {
    const TileArg* dy = tl.data();
    const TileArg* x = dy + ne;
    const TileArg* gm = dy + 2 * ne;
    const TileArg st = dy[3 * ne];
    const TileArg* dx = dy + 3 * ne + 1;
    const TileArg* dg = dy + 4 * ne + 1;
    const TileArg* db = dy + 5 * ne + 1;
    if (!ws || ctx->workspace_bytes < need)
      return fail(TT_ERR_STATE, "layernorm backward: the stream workspace holds %zu bytes, %zu needed",
                  ctx->workspace_bytes, need);
    if (ne == 1)
      return tile_layernorm_bwd(s, TT_LN_FUSED, rows, cols[0], total, Fp(dy[0]), cols[0], Fp(x[0]), cols[0],
                                Fp(gm[0]), Fp(st), nullptr, 0, 0, Fp(dx[0]), cols[0], dx_acc, Fp(dg[0]), Fp(db[0]),
                                ws);
    if (ln_one_pass(cols)) {
      std::vector<const float*> dys(ne), xs(ne), gs(ne);
      std::vector<float*> dxs(ne), dgs(ne), dbs(ne);
      std::vector<const void*> all = {ws};
      for (int e = 0; e < ne; ++e) {
        dys[e] = Fp(dy[e]);
        xs[e] = Fp(x[e]);
        gs[e] = Fp(gm[e]);
        dxs[e] = Fp(dx[e]);
        dgs[e] = Fp(dg[e]);
        dbs[e] = Fp(db[e]);
        all.insert(all.end(), {dys[e], xs[e], gs[e], dxs[e]});
      }
      if (all_aligned(all))
        return tile_layernorm_bwd_multi(s, ne, rows, cols.data(), dys.data(), xs.data(), gs.data(), Fp(st),
                                        dxs.data(), dx_acc, dgs.data(), dbs.data(), ws, ctx->workspace_bytes);
    }
    float* parts = (float*)ws;
    void* cws = (char*)ws + align_up((size_t)ne * rows * 2 * sizeof(float));
    for (int e = 0; e < ne; ++e)
      if (int rc = tile_layernorm_bwd(s, TT_LN_PARTIAL, rows, cols[e], total, Fp(dy[e]), cols[e], Fp(x[e]), cols[e],
                                      Fp(gm[e]), Fp(st), parts + (size_t)e * rows * 2, 0, 0, nullptr, 0, 0, nullptr,
                                      nullptr, nullptr))
        return rc;
    for (int e = 0; e < ne; ++e)
      if (int rc = tile_layernorm_bwd(s, TT_LN_APPLY, rows, cols[e], total, Fp(dy[e]), cols[e], Fp(x[e]), cols[e],
                                      Fp(gm[e]), Fp(st), parts, ne, rows * 2, Fp(dx[e]), cols[e], dx_acc, Fp(dg[e]),
                                      Fp(db[e]), cws))
        return rc;
    return TT_OK;
  });
}

// ------------------------------------------------------------ attention

struct AttGeo {
  int64_t batch, q_len, k_len, heads, hd;
};

int att_geo(const TileArg& Q, const TileArg& K, const char* nm, AttGeo* g) {
  if (Q.t->ndim != 4 || K.t->ndim != 4) return fail(TT_ERR_SHAPE, "%s: Q and K tiles must be 4-D", nm);
  int64_t eq[TT_MAX_DIMS], ek[TT_MAX_DIMS];
  Q.t->extent(Q.lin, eq);
  K.t->extent(K.lin, ek);
  if (eq[0] != ek[0] || eq[2] != ek[2] || eq[3] != ek[3])
    return fail(TT_ERR_SHAPE, "%s: Q and K tiles disagree on batch, heads or head dim", nm);
  *g = AttGeo{eq[0], eq[1], ek[1], eq[2], eq[3]};
  if (g->hd != 16 && g->hd != 32 && g->hd != 64 && g->hd != 128)
    return fail(TT_ERR_SHAPE, "%s: head dim %lld not in {16, 32, 64, 128}", nm, (long long)g->hd);
  return TT_OK;
}

int same_extent(const TileArg& a, const TileArg& b) {
  if (a.t->ndim != b.t->ndim) return 0;
  int64_t ea[TT_MAX_DIMS], eb[TT_MAX_DIMS];
  a.t->extent(a.lin, ea);
  b.t->extent(b.lin, eb);
  for (int d = 0; d < a.t->ndim; ++d)
    if (ea[d] != eb[d]) return 0;
  return 1;
}

double visible_pairs(int64_t q_len, int64_t k_len, int64_t q_off, int64_t k_off) {
  double p = 0;
  for (int64_t t = 0; t < q_len; ++t) p += (double)std::max<int64_t>(0, std::min(k_len, q_off + t - k_off + 1));
  return p;
}

int op_att_fwd(tt_ctx* ctx, const TileArg* T, int n, const tt_op_attention& q, const char* label) {
  const char* nm = "TT_OP_ATTENTION_FWD";
  if (n != 6) return fail(TT_ERR_ARG, "%s: tiles Q, K, V, O, ml, lse", nm);
  if (int rc = need_f32(T, n, nm)) return rc;
  AttGeo g;
  if (int rc = att_geo(T[0], T[1], nm, &g)) return rc;
  if (!same_extent(T[1], T[2]) || !same_extent(T[0], T[3]))
    return fail(TT_ERR_SHAPE, "%s: V must match K and O must match Q", nm);
  const int64_t nq = g.batch * g.heads * g.q_len;
  if ((!(q.first && q.last) && elems(T[4]) < 2 * nq) || (q.last && elems(T[5]) < nq))
    return fail(TT_ERR_SHAPE, "%s: ml needs %lld floats and lse %lld", nm, (long long)(2 * nq), (long long)nq);
  std::vector<Access> acc = {acc_of(T[0], TT_R), acc_of(T[1], TT_R), acc_of(T[2], TT_R),
                             acc_of(T[3], q.first ? TT_W : TT_RW)};
  if (!(q.first && q.last)) acc.push_back(acc_of(T[4], q.first ? TT_W : TT_RW));
  if (q.last) acc.push_back(acc_of(T[5], TT_W));
  const TileArg Q = T[0], K = T[1], V = T[2], O = T[3], ml = T[4], lse = T[5];
  const tt_op_attention p = q;
  const double flops = 4.0 * g.batch * g.heads * g.hd * visible_pairs(g.q_len, g.k_len, q.q_off, q.k_off);
  return ctx->submit(label ? label : "attn_fwd", std::move(acc), [=](hipStream_t s, void*) {
    return tile_attention_fwd(s, g.batch, g.heads, g.q_len, g.k_len, g.hd, p.q_off, p.k_off, Fp(Q), Fp(K), Fp(V),
                              Fp(O), (p.first && p.last) ? nullptr : Fp(ml), p.last ? Fp(lse) : nullptr, p.first,
                              p.last, p.scale);
  }, flops);
}

int op_att_prep(tt_ctx* ctx, const TileArg* T, int n, const tt_op_attention& q, const char* label) {
  const char* nm = "TT_OP_ATTENTION_PREP";
  if (n != 3) return fail(TT_ERR_ARG, "%s: tiles O, dO, Dvec", nm);
  if (int rc = need_f32(T, n, nm)) return rc;
  AttGeo g;
  if (int rc = att_geo(T[0], T[1], nm, &g)) return rc;
  if (!same_extent(T[0], T[1])) return fail(TT_ERR_SHAPE, "%s: dO must match O", nm);
  if (elems(T[2]) < g.batch * g.heads * g.q_len) return fail(TT_ERR_SHAPE, "%s: Dvec too small", nm);
  const TileArg O = T[0], dO = T[1], D = T[2];
  const float scale = q.scale;
  return ctx->submit(label ? label : "attn_prep", {acc_of(O, TT_R), acc_of(dO, TT_R), acc_of(D, TT_W)},
                     [=](hipStream_t s, void*) {
                       return tile_attention_bwd(s, TT_ATT_PREP, g.batch, g.heads, g.q_len, g.q_len, g.hd, 0, 0,
                                                 nullptr, nullptr, nullptr, Fp(O), Fp(dO), nullptr, Fp(D), nullptr,
                                                 nullptr, nullptr, 0, 0, scale);
                     });
}

int op_att_bwd(tt_ctx* ctx, const TileArg* T, int n, const tt_op_attention& q, const char* label, bool grow) {
  const char* nm = "TT_OP_ATTENTION_BWD";
  if (n != 9) return fail(TT_ERR_ARG, "%s: tiles Q, K, V, dO, lse, Dvec, dQ, dK, dV", nm);
  if (int rc = need_f32(T, n, nm)) return rc;
  AttGeo g;
  if (int rc = att_geo(T[0], T[1], nm, &g)) return rc;
  if (!same_extent(T[1], T[2]) || !same_extent(T[0], T[3]) || !same_extent(T[0], T[6]) ||
      !same_extent(T[1], T[7]) || !same_extent(T[1], T[8]))
    return fail(TT_ERR_SHAPE, "%s: V, dK, dV must match K; dO, dQ must match Q", nm);
  const int64_t nq = g.batch * g.heads * g.q_len;
  if (elems(T[4]) < nq || elems(T[5]) < nq) return fail(TT_ERR_SHAPE, "%s: lse and Dvec need %lld floats", nm,
                                                        (long long)nq);
  std::vector<Access> acc = {acc_of(T[0], TT_R), acc_of(T[1], TT_R), acc_of(T[2], TT_R),
                             acc_of(T[3], TT_R), acc_of(T[4], TT_R), acc_of(T[5], TT_R),
                             acc_of(T[6], q.acc_dq ? TT_RW : TT_W), acc_of(T[7], q.acc_dkv ? TT_RW : TT_W),
                             acc_of(T[8], q.acc_dkv ? TT_RW : TT_W)};
  std::vector<TileArg> tl(T, T + n);
  const tt_op_attention p = q;
  const double flops = 10.0 * g.batch * g.heads * g.hd * visible_pairs(g.q_len, g.k_len, q.q_off, q.k_off);
  // dS goes through the stream workspace (5 products per tile pair instead of 7)
  const size_t need = tile_attention_bwd_workspace(g.batch, g.heads, g.q_len, g.k_len);
  if (grow)
    if (int rc = ctx->ensure_workspace(need)) return rc;
  return ctx->submit(label ? label : "attn_bwd", std::move(acc), [=](hipStream_t s, void* ws) {
    return tile_attention_bwd_ws(s, TT_ATT_GRAD, g.batch, g.heads, g.q_len, g.k_len, g.hd, p.q_off, p.k_off,
                                 Fp(tl[0]), Fp(tl[1]), Fp(tl[2]), nullptr, Fp(tl[3]), Fp(tl[4]), Fp(tl[5]), Fp(tl[6]),
                                 Fp(tl[7]), Fp(tl[8]), p.acc_dq, p.acc_dkv, p.scale, ws,
                                 ws ? ctx->workspace_bytes : 0);
  }, flops);
}

// -------------------------------------------------------- cross-entropy

int op_xe_stats(tt_ctx* ctx, const TileArg* T, int n, const char* label) {
  const char* nm = "TT_OP_XENTROPY_STATS";
  if (n < 3 || (n - 1) % 2) return fail(TT_ERR_ARG, "%s: tiles labels, z_0..z_{n-1}, parts_0..parts_{n-1}", nm);
  if (int rc = need_i32(T[0], nm, "labels")) return rc;
  if (int rc = need_f32(T + 1, n - 1, nm)) return rc;
  const int nv = (n - 1) / 2;
  int64_t rows = elems(T[0]);
  std::vector<Access> acc = {acc_of(T[0], TT_R)};
  std::vector<int64_t> lens(nv), offs(nv);
  for (int j = 0; j < nv; ++j) {
    int64_t r, c;
    matv(T[1 + j], &r, &c);
    if (r != rows || c > 2048 || elems(T[1 + nv + j]) < 3 * rows)
      return fail(TT_ERR_SHAPE, "%s: logits tile %d is %lldx%lld (rows must equal the labels' %lld, width <= 2048) "
                  "or its partials tile is too small", nm, j, (long long)r, (long long)c, (long long)rows);
    lens[j] = c;
    offs[j] = last_axis_offset(T[1 + j]);
    acc.push_back(acc_of(T[1 + j], TT_R));
    acc.push_back(acc_of(T[1 + nv + j], TT_W));
  }
  std::vector<TileArg> tl(T, T + n);
  return ctx->submit(label ? label : "ce_stats", std::move(acc), [=](hipStream_t s, void*) {
    std::vector<float*> zs(nv);
    float* p0 = Fp(tl[1 + nv]);
    const int64_t stride = nv > 1 ? Fp(tl[2 + nv]) - p0 : rows * 3;
    for (int j = 0; j < nv; ++j) {
      zs[j] = Fp(tl[1 + j]);
      if (Fp(tl[1 + nv + j]) != p0 + j * stride || stride < rows * 3)
        return fail(TT_ERR_SHAPE, "cross-entropy statistics: the partials tiles are not equally spaced");
    }
    std::vector<int64_t> ld(lens);
    return tile_xentropy_multi(s, TT_XE_STATS, nv, rows, lens.data(), offs.data(), Ip(tl[0]), zs.data(), ld.data(), p0,
                               stride, nullptr, 1.f);
  });
}

int op_xe_merge(tt_ctx* ctx, const TileArg* T, int n, const tt_op_xe_groups* grp, const char* label) {
  const char* nm = "TT_OP_XENTROPY_MERGE";
  if (n < 3) return fail(TT_ERR_ARG, "%s: tiles lse, row_loss, parts_0..parts_{n-1}", nm);
  if (int rc = need_f32(T, n, nm)) return rc;
  const int np = n - 2;
  const int64_t rows = elems(T[0]);
  if (elems(T[1]) < rows) return fail(TT_ERR_SHAPE, "%s: row_loss smaller than lse", nm);
  // group mode: partials tile j holds the 64-column groups of vocab tile j
  std::vector<int64_t> vlen;
  if (grp) {
    if (grp->group < 1 || grp->v_tile < 1 || grp->vocab < 1 || (grp->vocab + grp->v_tile - 1) / grp->v_tile != np)
      return fail(TT_ERR_ARG, "%s: groups need group >= 1 and one partials tile per vocab tile", nm);
    for (int j = 0; j < np; ++j) vlen.push_back(std::min(grp->v_tile, grp->vocab - j * grp->v_tile));
  }
  std::vector<Access> acc;
  for (int j = 0; j < np; ++j) {
    const int64_t need = 3 * rows * (grp ? (vlen[j] + grp->group - 1) / grp->group : 1);
    if (elems(T[2 + j]) < need) return fail(TT_ERR_SHAPE, "%s: partials tile %d too small", nm, j);
    acc.push_back(acc_of(T[2 + j], TT_R));
  }
  acc.push_back(acc_of(T[0], TT_W));
  acc.push_back(acc_of(T[1], TT_W));
  std::vector<TileArg> tl(T, T + n);
  const int group = grp ? grp->group : 0;
  return ctx->submit(label ? label : "ce_merge", std::move(acc), [=](hipStream_t s, void*) {
    float* p0 = Fp(tl[2]);
    const int64_t least = group ? 3 * rows * ((vlen[0] + group - 1) / group) : rows * 3;
    const int64_t stride = np > 1 ? Fp(tl[3]) - p0 : least;
    for (int j = 0; j < np; ++j)
      if (Fp(tl[2 + j]) != p0 + j * stride || stride < least)
        return fail(TT_ERR_SHAPE, "cross-entropy merge: the partials tiles are not equally spaced");
    if (group)
      return tile_xentropy_merge_groups(s, rows, np, vlen.data(), group, p0, stride, Fp(tl[0]), Fp(tl[1]));
    return tile_softmax(s, TT_SM_MERGE, rows, 0, 0, 0, 1.f, 0, nullptr, 0, nullptr, p0, np, stride, Fp(tl[0]),
                        Fp(tl[1]), nullptr, 0, 1.f);
  });
}

int op_xe_loss(tt_ctx* ctx, const TileArg* T, int n, const tt_op_xentropy& q, const char* label) {
  const char* nm = "TT_OP_XENTROPY_LOSS";
  if (n != 2) return fail(TT_ERR_ARG, "%s: tiles row_loss, loss", nm);
  if (int rc = need_f32(T, n, nm)) return rc;
  const int64_t rows = elems(T[0]);
  const TileArg rl = T[0], loss = T[1];
  const int accumulate = q.accumulate;
  const float inv_n = q.inv_n;
  return ctx->submit(label ? label : "ce_loss", {acc_of(rl, TT_R), acc_of(loss, accumulate ? TT_RW : TT_W)},
                     [=](hipStream_t s, void*) {
                       return tile_xentropy(s, TT_XE_LOSS, rows, 0, 0, nullptr, nullptr, 0, nullptr, Fp(rl), Fp(loss),
                                            accumulate, inv_n);
                     });
}

int op_xe_grad(tt_ctx* ctx, const TileArg* T, int n, const tt_op_xentropy& q, const char* label) {
  const char* nm = "TT_OP_XENTROPY_GRAD";
  if (n < 3) return fail(TT_ERR_ARG, "%s: tiles labels, lse, z_0..z_{n-1}", nm);
  if (int rc = need_i32(T[0], nm, "labels")) return rc;
  if (int rc = need_f32(T + 1, n - 1, nm)) return rc;
  const int nv = n - 2;
  const int64_t rows = elems(T[0]);
  if (elems(T[1]) < rows) return fail(TT_ERR_SHAPE, "%s: lse smaller than the labels", nm);
  std::vector<Access> acc = {acc_of(T[0], TT_R), acc_of(T[1], TT_R)};
  std::vector<int64_t> lens(nv), offs(nv);
  for (int j = 0; j < nv; ++j) {
    int64_t r, c;
    matv(T[2 + j], &r, &c);
    if (r != rows || c > 2048)
      return fail(TT_ERR_SHAPE, "%s: logits tile %d is %lldx%lld (rows %lld, width <= 2048)", nm, j, (long long)r,
                  (long long)c, (long long)rows);
    lens[j] = c;
    offs[j] = last_axis_offset(T[2 + j]);
    acc.push_back(acc_of(T[2 + j], TT_RW));
  }
  std::vector<TileArg> tl(T, T + n);
  const float inv_n = q.inv_n;
  return ctx->submit(label ? label : "ce_grad", std::move(acc), [=](hipStream_t s, void*) {
    std::vector<float*> zs(nv);
    for (int j = 0; j < nv; ++j) zs[j] = Fp(tl[2 + j]);
    std::vector<int64_t> ld(lens);
    return tile_xentropy_multi(s, TT_XE_GRAD, nv, rows, lens.data(), offs.data(), Ip(tl[0]), zs.data(), ld.data(),
                               nullptr, 0, Fp(tl[1]), inv_n);
  });
}

// ------------------------------------------------------------ optimisers

int op_adamw(tt_ctx* ctx, const TileArg* T, int n, const tt_op_optim& q, const char* label) {
  const char* nm = "TT_OP_ADAMW";
  if (n < 5 || (n - 1) % 4 || (n - 1) / 4 > TT_ADAMW_MAX_TILES)
    return fail(TT_ERR_ARG, "%s: tiles bias_corr, then 1..%d (p, g, m, v) quadruples", nm, TT_ADAMW_MAX_TILES);
  if (int rc = need_f32(T, n, nm)) return rc;
  if (elems(T[0]) < 2) return fail(TT_ERR_SHAPE, "%s: bias_corr holds 2 floats", nm);
  const int cnt = (n - 1) / 4;
  std::vector<Access> acc;
  for (int i = 0; i < cnt; ++i) {
    const TileArg* t = T + 1 + 4 * i;
    const int64_t e = elems(t[0]);
    if (elems(t[1]) != e || elems(t[2]) != e || elems(t[3]) != e)
      return fail(TT_ERR_SHAPE, "%s: p, g, m, v of tile %d differ in size", nm, i);
    acc.push_back(acc_of(t[0], TT_RW));
    acc.push_back(acc_of(t[1], TT_R));
    acc.push_back(acc_of(t[2], TT_RW));
    acc.push_back(acc_of(t[3], TT_RW));
  }
  acc.push_back(acc_of(T[0], TT_R));
  std::vector<TileArg> tl(T, T + n);
  const tt_op_optim h = q;
  return ctx->submit(label ? label : "adamw", std::move(acc), [=](hipStream_t s, void*) {
    float *pp[TT_ADAMW_MAX_TILES], *mm[TT_ADAMW_MAX_TILES], *vv[TT_ADAMW_MAX_TILES];
    const float* gg[TT_ADAMW_MAX_TILES];
    int64_t nn[TT_ADAMW_MAX_TILES];
    for (int i = 0; i < cnt; ++i) {
      const TileArg* t = tl.data() + 1 + 4 * i;
      pp[i] = Fp(t[0]);
      gg[i] = Fp(t[1]);
      mm[i] = Fp(t[2]);
      vv[i] = Fp(t[3]);
      nn[i] = elems(t[0]);
    }
    return tile_fused_adamw_multi(s, cnt, pp, gg, mm, vv, nn, h.lr, h.beta1, h.beta2, h.eps, h.weight_decay,
                                  Fp(tl[0]));
  });
}

int op_adamw_advance(tt_ctx* ctx, const TileArg* T, int n, const tt_op_optim& q, const char* label) {
  const char* nm = "TT_OP_ADAMW_ADVANCE";
  if (n != 2) return fail(TT_ERR_ARG, "%s: tiles step, bias_corr", nm);
  if (int rc = need_i32(T[0], nm, "step")) return rc;
  if (int rc = need_f32(T + 1, 1, nm)) return rc;
  if (elems(T[1]) < 2) return fail(TT_ERR_SHAPE, "%s: bias_corr holds 2 floats", nm);
  const TileArg st = T[0], bc = T[1];
  const float b1 = q.beta1, b2 = q.beta2;
  return ctx->submit(label ? label : "adam_step", {acc_of(st, TT_RW), acc_of(bc, TT_W)}, [=](hipStream_t s, void*) {
    return tile_adamw_advance(s, (int32_t*)st.t->dev(st.lin), Fp(bc), b1, b2);
  });
}

int op_sgd(tt_ctx* ctx, const TileArg* T, int n, const tt_op_optim& q, const char* label) {
  const char* nm = "TT_OP_SGD";
  if (n < 2 || n % 2 || n / 2 > TT_SGD_MAX_TILES)
    return fail(TT_ERR_ARG, "%s: tiles 1..%d (p, g) pairs", nm, TT_SGD_MAX_TILES);
  if (int rc = need_f32(T, n, nm)) return rc;
  const int cnt = n / 2;
  std::vector<Access> acc;
  for (int i = 0; i < cnt; ++i) {
    if (elems(T[2 * i]) != elems(T[2 * i + 1])) return fail(TT_ERR_SHAPE, "%s: p and g of tile %d differ", nm, i);
    acc.push_back(acc_of(T[2 * i], TT_RW));
    acc.push_back(acc_of(T[2 * i + 1], TT_R));
  }
  std::vector<TileArg> tl(T, T + n);
  const float lr = q.lr;
  return ctx->submit(label ? label : "sgd", std::move(acc), [=](hipStream_t s, void*) {
    float* pp[TT_SGD_MAX_TILES];
    const float* gg[TT_SGD_MAX_TILES];
    int64_t nn[TT_SGD_MAX_TILES];
    for (int i = 0; i < cnt; ++i) {
      pp[i] = Fp(tl[2 * i]);
      gg[i] = Fp(tl[2 * i + 1]);
      nn[i] = elems(tl[2 * i]);
    }
    return tile_sgd_multi(s, cnt, pp, gg, nn, lr);
  });
}

// ------------------------------------------------------------- embedding

// consecutive vocab tiles of one embd column of the token table (all of
// them when `all`), in vocab order; v_first = the first one's vocab tile index
int vocab_column(const TileArg* W, int nv, int64_t cols, const char* nm, bool all, int64_t* vocab, int64_t* vt,
                 int64_t* v_first) {
  const tt_tensor* t = W[0].t;
  if (t->ndim != 2) return fail(TT_ERR_SHAPE, "%s: the token table must be 2-D", nm);
  *vocab = t->shape[0];
  *vt = t->tshape[0];
  *v_first = W[0].lin % t->grid[0];
  if (all && (nv != t->grid[0] || *v_first != 0))
    return fail(TT_ERR_ARG, "%s: %d vocab tiles given, the table has %lld", nm, nv, (long long)t->grid[0]);
  if (*v_first + nv > t->grid[0]) return fail(TT_ERR_ARG, "%s: vocab tiles past the end of the table", nm);
  for (int v = 0; v < nv; ++v) {
    int64_t r, c;
    W[v].t->mat(W[v].lin, &r, &c);
    if (W[v].t != t || W[v].lin != W[0].lin + v || c != cols)
      return fail(TT_ERR_ARG, "%s: wte tiles must be consecutive vocab tiles of one embd column, in order", nm);
  }
  return TT_OK;
}

bool contiguous_column(const TileArg* W, int nv) {
  if (W[0].t->home != TT_HOME_DEVICE) return false;
  for (int v = 1; v < nv; ++v)
    if ((char*)W[v].t->dev(W[v].lin) != (char*)W[0].t->dev(W[0].lin) + W[0].t->tile_off[W[v].lin] * 4 -
                                            W[0].t->tile_off[W[0].lin] * 4)
      return false;
  return true;
}

// pos: the tile list has a position-table tile after ids (TT_OP_EMBEDDING_FWD);
// without it (TT_OP_EMBEDDING_TOKEN_FWD) out = wte[id]
int op_emb_fwd(tt_ctx* ctx, const TileArg* T, int n, const tt_op_embedding& q, const char* label, bool pos) {
  const char* nm = pos ? "TT_OP_EMBEDDING_FWD" : "TT_OP_EMBEDDING_TOKEN_FWD";
  const int np = pos ? 1 : 0;
  if (n < 3 + np) return fail(TT_ERR_ARG, "%s: tiles ids, %sout, wte_0..wte_{n-1}", nm, pos ? "wpe, " : "");
  if (int rc = need_i32(T[0], nm, "ids")) return rc;
  if (int rc = need_f32(T + 1, n - 1, nm)) return rc;
  const int nv = n - 2 - np;
  int64_t rows, cols, pr = 0, pc = 0;
  matv(T[1 + np], &rows, &cols);
  if (pos) matv(T[1], &pr, &pc);
  else pr = q.seq_len, pc = cols;
  if (elems(T[0]) != rows || pc != cols || q.seq_len < 1 || q.seq_len > pr || rows % q.seq_len)
    return fail(TT_ERR_SHAPE, "%s: ids %lld, out %lldx%lld, wpe %lldx%lld, seq_len %lld disagree", nm,
                (long long)elems(T[0]), (long long)rows, (long long)cols, (long long)pr, (long long)pc,
                (long long)q.seq_len);
  int64_t vocab, vt, v_first;
  if (int rc = vocab_column(T + 2 + np, nv, cols, nm, true, &vocab, &vt, &v_first)) return rc;
  std::vector<Access> acc = {acc_of(T[0], TT_R), acc_of(T[1 + np], TT_W)};
  if (pos) acc.push_back(acc_of(T[1], TT_R));
  for (int v = 0; v < nv; ++v) acc.push_back(acc_of(T[2 + np + v], TT_R));
  std::vector<TileArg> tl(T, T + n);
  const int64_t sl = q.seq_len;
  return ctx->submit(label ? label : "emb_fwd", std::move(acc), [=](hipStream_t s, void*) {
    const TileArg *ids = &tl[0], *out = &tl[1 + np], *W = &tl[2 + np];
    float* wpe = pos ? Fp(tl[1]) : nullptr;
    if (contiguous_column(W, nv))  // device home: the column is one [vocab, cols] slab
      return tile_embedding_fwd(s, rows, cols, Ip(*ids), vocab, 0, vocab, Fp(W[0]), cols, wpe, cols, sl, 0,
                                Fp(*out), cols);
    for (int v = 0; v < nv; ++v) {
      const int64_t v_off = v * vt;
      if (int rc = tile_embedding_fwd(s, rows, cols, Ip(*ids), vocab, v_off, std::min(vt, vocab - v_off), Fp(W[v]),
                                      cols, wpe, cols, sl, 0, Fp(*out), cols))
        return rc;
    }
    return TT_OK;
  });
}

int op_emb_index(tt_ctx* ctx, const TileArg* T, int n, const char* label) {
  const char* nm = "TT_OP_EMBEDDING_INDEX";
  if (n != 3) return fail(TT_ERR_ARG, "%s: tiles ids, sorted, perm", nm);
  for (int i = 0; i < 3; ++i)
    if (int rc = need_i32(T[i], nm, "every tile")) return rc;
  const int64_t rows = elems(T[0]);
  if (elems(T[1]) != rows || elems(T[2]) != rows || rows > 65536)
    return fail(TT_ERR_SHAPE, "%s: sorted and perm must match ids (at most 65536)", nm);
  const TileArg ids = T[0], so = T[1], pe = T[2];
  return ctx->submit(label ? label : "emb_index", {acc_of(ids, TT_R), acc_of(so, TT_W), acc_of(pe, TT_W)},
                     [=](hipStream_t s, void*) {
                       return tile_embedding_index(s, rows, Ip(ids), (int32_t*)so.t->dev(so.lin),
                                                   (int32_t*)pe.t->dev(pe.lin));
                     });
}

int op_emb_bwd(tt_ctx* ctx, const TileArg* T, int n, const tt_op_embedding& q, const char* label) {
  const char* nm = "TT_OP_EMBEDDING_BWD";
  if (n < 4) return fail(TT_ERR_ARG, "%s: tiles dh, sorted, perm, dwte_0..dwte_{n-1}", nm);
  if (int rc = need_i32(T[1], nm, "sorted")) return rc;
  if (int rc = need_i32(T[2], nm, "perm")) return rc;
  if (int rc = need_f32(T, 1, nm)) return rc;
  if (int rc = need_f32(T + 3, n - 3, nm)) return rc;
  const int nv = n - 3;
  int64_t rows, cols;
  matv(T[0], &rows, &cols);
  if (elems(T[1]) != rows || elems(T[2]) != rows) return fail(TT_ERR_SHAPE, "%s: sorted/perm must match dh's rows", nm);
  int64_t vocab, vt, v_first;
  if (int rc = vocab_column(T + 3, nv, cols, nm, false, &vocab, &vt, &v_first)) return rc;
  std::vector<Access> acc = {acc_of(T[0], TT_R), acc_of(T[1], TT_R), acc_of(T[2], TT_R)};
  for (int v = 0; v < nv; ++v) acc.push_back(acc_of(T[3 + v], TT_RW));
  std::vector<TileArg> tl(T, T + n);
  const int64_t sl = std::max<int64_t>(1, q.seq_len);
  return ctx->submit(label ? label : "emb_dw", std::move(acc), [=](hipStream_t s, void*) {
    const TileArg *dh = &tl[0], *so = &tl[1], *pe = &tl[2], *W = &tl[3];
    if (v_first == 0 && nv * vt >= vocab && contiguous_column(W, nv))
      return tile_embedding_bwd(s, TT_EMB_TOKEN, rows, cols, Ip(*so), Ip(*pe), 0, vocab, sl, Fp(*dh), cols, Fp(W[0]),
                                cols);
    for (int v = 0; v < nv; ++v) {
      const int64_t v_off = (v_first + v) * vt;
      if (int rc = tile_embedding_bwd(s, TT_EMB_TOKEN, rows, cols, Ip(*so), Ip(*pe), v_off,
                                      std::min(vt, vocab - v_off), sl, Fp(*dh), cols, Fp(W[v]), cols))
        return rc;
    }
    return TT_OK;
  });
}

int op_emb_pos_bwd(tt_ctx* ctx, const TileArg* T, int n, const tt_op_embedding& q, const char* label) {
  const char* nm = "TT_OP_EMBEDDING_POS_BWD";
  if (n != 2) return fail(TT_ERR_ARG, "%s: tiles dh, dwpe", nm);
  if (int rc = need_f32(T, n, nm)) return rc;
  int64_t rows, cols, pr, pc;
  matv(T[0], &rows, &cols);
  matv(T[1], &pr, &pc);
  if (pc != cols || q.seq_len < 1 || q.seq_len > pr || rows % q.seq_len)
    return fail(TT_ERR_SHAPE, "%s: dh %lldx%lld, dwpe %lldx%lld, seq_len %lld disagree", nm, (long long)rows,
                (long long)cols, (long long)pr, (long long)pc, (long long)q.seq_len);
  const TileArg dh = T[0], dw = T[1];
  const int64_t sl = q.seq_len;
  return ctx->submit(label ? label : "emb_dpos", {acc_of(dh, TT_R), acc_of(dw, TT_RW)}, [=](hipStream_t s, void*) {
    return tile_embedding_bwd(s, TT_EMB_POS, rows, cols, nullptr, nullptr, 0, 0, sl, Fp(dh), cols, Fp(dw), cols);
  });
}

// ------------------------------------------------------------ the rest

int op_reduce(tt_ctx* ctx, const TileArg* T, int n, const tt_op_reduce& q, const char* label, bool grow) {
  const char* nm = "TT_OP_REDUCE_ROWS";
  if (n < 2 || n % 2 || n / 2 > 16) return fail(TT_ERR_ARG, "%s: tiles 1..16 (X, out) pairs", nm);
  if (int rc = need_f32(T, n, nm)) return rc;
  const int cnt = n / 2;
  int64_t rows = -1;
  std::vector<int64_t> cols(cnt);
  std::vector<Access> acc;
  size_t need = 0;
  for (int u = 0; u < cnt; ++u) {
    int64_t r, c;
    matv(T[2 * u], &r, &c);
    if ((rows >= 0 && r != rows) || elems(T[2 * u + 1]) != c)
      return fail(TT_ERR_SHAPE, "%s: pair %d: X %lldx%lld, out %lld (rows must be equal)", nm, u, (long long)r,
                  (long long)c, (long long)elems(T[2 * u + 1]));
    rows = r;
    cols[u] = c;
    need += tile_reduce_rows_workspace(r, c);
    acc.push_back(acc_of(T[2 * u], TT_R));
    acc.push_back(acc_of(T[2 * u + 1], q.beta ? TT_RW : TT_W));
  }
  if (grow)
    if (int rc = ctx->ensure_workspace(need)) return rc;
  std::vector<TileArg> tl(T, T + n);
  const int beta = q.beta;
  return ctx->submit(label ? label : "colsum", std::move(acc), [=](hipStream_t s, void* ws) {
    if (cnt == 1) return tile_reduce_rows(s, rows, cols[0], Fp(tl[0]), cols[0], Fp(tl[1]), beta, ws);
    std::vector<const float*> X(cnt);
    std::vector<float*> O(cnt);
    for (int u = 0; u < cnt; ++u) {
      X[u] = Fp(tl[2 * u]);
      O[u] = Fp(tl[2 * u + 1]);
    }
    std::vector<int64_t> ld(cols);
    return tile_reduce_rows_multi(s, cnt, rows, cols.data(), X.data(), ld.data(), O.data(), beta, ws,
                                  ctx->workspace_bytes);
  });
}

int op_split(tt_ctx* ctx, const TileArg* T, int n, const char* label) {
  const char* nm = "TT_OP_SPLIT_TOKENS";
  if (n != 3) return fail(TT_ERR_ARG, "%s: tiles tokens, ids, labels", nm);
  for (int i = 0; i < 3; ++i)
    if (int rc = need_i32(T[i], nm, "every tile")) return rc;
  const tt_tensor *tok = T[0].t, *ids = T[1].t;
  if (tok->ndim != 2 || tok->ntiles != 1 || ids->ndim != 2 || T[2].t->ndim != 2 || !same_extent(T[1], T[2]) ||
      tok->shape[0] != ids->shape[0] || tok->shape[1] != ids->shape[1] + 1 || T[2].t->shape[0] != ids->shape[0] ||
      T[2].t->shape[1] != ids->shape[1])
    return fail(TT_ERR_SHAPE, "%s: tokens must be one [B, T+1] tile, ids and labels [B, T]", nm);
  int64_t ext[TT_MAX_DIMS];
  ids->extent(T[1].lin, ext);
  const int64_t bi = T[1].lin % ids->grid[0], si = T[1].lin / ids->grid[0];
  const int64_t b0 = bi * ids->tshape[0], s0 = si * ids->tshape[1], bt = ext[0], sq = ext[1];
  const int64_t win = tok->shape[1];
  const TileArg t0 = T[0], ti = T[1], tl = T[2];
  return ctx->submit(label ? label : "split", {acc_of(t0, TT_R), acc_of(ti, TT_W), acc_of(tl, TT_W)},
                     [=](hipStream_t s, void*) {
                       for (int64_t b = 0; b < bt; ++b) {  // one launch per window of the tile
                         const int32_t* src = Ip(t0) + (b0 + b) * win + s0;
                         if (int rc = tile_split_tokens(s, 1, sq, src, (int32_t*)ti.t->dev(ti.lin) + b * sq,
                                                        (int32_t*)tl.t->dev(tl.lin) + b * sq))
                           return rc;
                       }
                       return TT_OK;
                     });
}

int op_copy_in(tt_ctx* ctx, const TileArg* T, int n, const tt_op_copy& q, const char* label) {
  const char* nm = "TT_OP_COPY_IN";
  if (n != 1) return fail(TT_ERR_ARG, "%s: one tile", nm);
  if (!q.src && !ctx->dryrun) return fail(TT_ERR_ARG, "%s: null source", nm);
  const TileArg d = T[0];
  const size_t bytes = (size_t)elems(d) * d.t->esize();
  const void* src = q.src;
  return ctx->submit(label ? label : "copy_in", {acc_of(d, TT_W)}, [=](hipStream_t s, void*) {
    TT_HIP_TRY(hipMemcpyAsync(d.t->dev(d.lin), src, bytes, hipMemcpyDeviceToDevice, s));
    return TT_OK;
  });
}

int op_fill(tt_ctx* ctx, const TileArg* T, int n, const tt_op_fill& q, const char* label) {
  const char* nm = "TT_OP_FILL";
  if (n < 1 || n > TT_FILL_MAX_TILES) return fail(TT_ERR_ARG, "%s: 1..%d tiles", nm, TT_FILL_MAX_TILES);
  if (int rc = need_f32(T, n, nm)) return rc;
  std::vector<Access> acc;
  for (int i = 0; i < n; ++i) acc.push_back(acc_of(T[i], TT_W));
  std::vector<TileArg> tl(T, T + n);
  const float v = q.value;
  return ctx->submit(label ? label : "fill", std::move(acc), [=](hipStream_t s, void*) {
    float* dst[TT_FILL_MAX_TILES];
    int64_t nn[TT_FILL_MAX_TILES];
    for (int i = 0; i < n; ++i) {
      dst[i] = Fp(tl[i]);
      nn[i] = elems(tl[i]);
    }
    return tile_fill_multi(s, n, dst, nn, v);
  });
}

// ------------------------------------------------------- LLaMA block ops

// rows and per-tile widths of an RMSNorm tile list (x_e and the tiles that
// must match them), checked against the one-pass kernels' limits
int rms_cols(const char* nm, const TileArg* X, int ne, int64_t* rows, std::vector<int64_t>* cols) {
  *rows = -1;
  cols->assign(ne, 0);
  for (int e = 0; e < ne; ++e) {
    int64_t r, c;
    matv(X[e], &r, &c);
    if (*rows >= 0 && r != *rows) return fail(TT_ERR_SHAPE, "%s: feature tiles have different row counts", nm);
    *rows = r;
    (*cols)[e] = c;
  }
  int64_t total = 0;
  for (int e = 0; e < ne; ++e) {
    const int64_t c = (*cols)[e];
    if (c < 4 || c % 4 || c > (*cols)[0] || (e + 1 < ne && c != (*cols)[0]))
      return fail(TT_ERR_SHAPE, "%s: tile widths must be multiples of 4, equal but for a narrower last tile", nm);
    total += c;
  }
  if (total > 16384) return fail(TT_ERR_SHAPE, "%s: %lld features exceed 16384", nm, (long long)total);
  return TT_OK;
}

int op_rms_fwd(tt_ctx* ctx, const TileArg* T, int n, const tt_op_layernorm& q, const char* label) {
  const char* nm = "TT_OP_RMSNORM_FWD";
  if (n < 4 || (n - 1) % 3 || (n - 1) / 3 > 16) return fail(TT_ERR_ARG, "%s: needs 3n+1 tiles, n <= 16", nm);
  if (int rc = need_f32(T, n, nm)) return rc;
  const int ne = (n - 1) / 3;
  const TileArg *X = T, *Gm = T + ne, *Y = T + 2 * ne + 1;
  const TileArg rs = T[2 * ne];
  int64_t rows;
  std::vector<int64_t> cols;
  if (int rc = rms_cols(nm, X, ne, &rows, &cols)) return rc;
  std::vector<Access> acc;
  for (int e = 0; e < ne; ++e) {
    int64_t yr, yc;
    matv(Y[e], &yr, &yc);
    if (yr != rows || yc != cols[e] || elems(Gm[e]) != cols[e])
      return fail(TT_ERR_SHAPE, "%s: feature tile %d: shapes of x, gamma, y disagree", nm, e);
    acc.push_back(acc_of(X[e], TT_R));
    acc.push_back(acc_of(Gm[e], TT_R));
    acc.push_back(acc_of(Y[e], TT_W));
  }
  if (elems(rs) < rows) return fail(TT_ERR_SHAPE, "%s: rstd tile holds fewer than rows floats", nm);
  acc.push_back(acc_of(rs, TT_W));
  std::vector<TileArg> tl(T, T + n);
  const float eps = q.eps;
  return ctx->submit(label ? label : "rms_fwd", std::move(acc), [=](hipStream_t s, void*) {
    std::vector<const float*> xs(ne), gs(ne);
    std::vector<float*> ys(ne);
    for (int e = 0; e < ne; ++e) {
      xs[e] = Fp(tl[e]);
      gs[e] = Fp(tl[ne + e]);
      ys[e] = Fp(tl[2 * ne + 1 + e]);
    }
    return tile_rmsnorm_fwd(s, ne, rows, cols.data(), xs.data(), gs.data(), Fp(tl[2 * ne]), ys.data(), eps);
  });
}

int op_rms_bwd(tt_ctx* ctx, const TileArg* T, int n, const tt_op_layernorm& q, const char* label, bool grow) {
  const char* nm = "TT_OP_RMSNORM_BWD";
  if (n < 6 || (n - 1) % 5 || (n - 1) / 5 > 16) return fail(TT_ERR_ARG, "%s: needs 5n+1 tiles, n <= 16", nm);
  if (int rc = need_f32(T, n, nm)) return rc;
  const int ne = (n - 1) / 5;
  const TileArg *DY = T, *X = T + ne, *Gm = T + 2 * ne, *DX = T + 3 * ne + 1, *DG = T + 4 * ne + 1;
  const TileArg rs = T[3 * ne];
  int64_t rows;
  std::vector<int64_t> cols;
  if (int rc = rms_cols(nm, X, ne, &rows, &cols)) return rc;
  std::vector<Access> acc;
  int64_t total = 0;
  for (int e = 0; e < ne; ++e) {
    int64_t dyr, dyc, dxr, dxc;
    matv(DY[e], &dyr, &dyc);
    matv(DX[e], &dxr, &dxc);
    if (dyr != rows || dyc != cols[e] || dxr != rows || dxc != cols[e] || elems(Gm[e]) != cols[e] ||
        elems(DG[e]) != cols[e])
      return fail(TT_ERR_SHAPE, "%s: feature tile %d: shapes of dy, x, dx, gamma, dgamma disagree", nm, e);
    total += cols[e];
    acc.push_back(acc_of(DY[e], TT_R));
    acc.push_back(acc_of(X[e], TT_R));
    acc.push_back(acc_of(Gm[e], TT_R));
    acc.push_back(acc_of(DX[e], q.dx_acc ? TT_RW : TT_W));
    acc.push_back(acc_of(DG[e], TT_RW));
  }
  if (elems(rs) < rows) return fail(TT_ERR_SHAPE, "%s: rstd tile holds fewer than rows floats", nm);
  acc.push_back(acc_of(rs, TT_R));
  const size_t need = tile_rmsnorm_bwd_workspace(rows, total);
  if (grow)
    if (int rc = ctx->ensure_workspace(need)) return rc;
  std::vector<TileArg> tl(T, T + n);
  const int dx_acc = q.dx_acc;
  return ctx->submit(label ? label : "rms_bwd", std::move(acc), [=](hipStream_t s, void* ws) {
    std::vector<const float*> dys(ne), xs(ne), gs(ne);
    std::vector<float*> dxs(ne), dgs(ne);
    for (int e = 0; e < ne; ++e) {
      dys[e] = Fp(tl[e]);
      xs[e] = Fp(tl[ne + e]);
      gs[e] = Fp(tl[2 * ne + e]);
      dxs[e] = Fp(tl[3 * ne + 1 + e]);
      dgs[e] = Fp(tl[4 * ne + 1 + e]);
    }
    return tile_rmsnorm_bwd(s, ne, rows, cols.data(), dys.data(), xs.data(), gs.data(), Fp(tl[3 * ne]), dxs.data(),
                            dx_acc, dgs.data(), ws, ctx->workspace_bytes);
  });
}

int op_rope(tt_ctx* ctx, const TileArg* T, int n, const tt_op_rope& q, const char* label) {
  const char* nm = "TT_OP_ROPE";
  if (n < 2 || n > 5) return fail(TT_ERR_ARG, "%s: tiles x_0..x_{n-1} (1..4), table", nm);
  if (int rc = need_f32(T, n, nm)) return rc;
  int64_t ext[TT_MAX_DIMS];
  const TileArg& x0 = T[0];
  if (x0.t->ndim != 4) return fail(TT_ERR_SHAPE, "%s: x tiles must be 4-D [batch, len, heads, hd]", nm);
  x0.t->extent(x0.lin, ext);
  const int64_t len = ext[1], heads = ext[2], hd = ext[3], rows = ext[0] * ext[1];
  std::vector<Access> acc;
  for (int i = 0; i < n - 1; ++i) {
    int64_t e2[TT_MAX_DIMS];
    if (T[i].t->ndim != 4) return fail(TT_ERR_SHAPE, "%s: x tiles must be 4-D", nm);
    T[i].t->extent(T[i].lin, e2);
    if (e2[0] != ext[0] || e2[1] != len || e2[2] != heads || e2[3] != hd)
      return fail(TT_ERR_SHAPE, "%s: x tiles must have equal extents", nm);
    acc.push_back(acc_of(T[i], TT_RW));
  }
  const TileArg tab = T[n - 1];
  int64_t tr, tc;
  matv(tab, &tr, &tc);
  if (tc != hd || q.pos_off < 0 || q.pos_off + len > tr)
    return fail(TT_ERR_SHAPE, "%s: table %lldx%lld does not cover positions %lld..%lld of head dim %lld", nm,
                (long long)tr, (long long)tc, (long long)q.pos_off, (long long)(q.pos_off + len - 1), (long long)hd);
  acc.push_back(acc_of(tab, TT_R));
  std::vector<TileArg> tl(T, T + n);
  const int64_t off = q.pos_off;
  const int inv = q.inverse;
  return ctx->submit(label ? label : "rope", std::move(acc), [=](hipStream_t s, void*) {
    float* xs[4];
    for (int i = 0; i < n - 1; ++i) xs[i] = Fp(tl[i]);
    return tile_rope_multi(s, n - 1, xs, rows, heads, hd, len, off, Fp(tl[n - 1]), tr, inv);
  });
}

int op_rope_table(tt_ctx* ctx, const TileArg* T, int n, const tt_op_rope& q, const char* label) {
  const char* nm = "TT_OP_ROPE_TABLE";
  if (n != 1) return fail(TT_ERR_ARG, "%s: one tile (the table)", nm);
  if (int rc = need_f32(T, n, nm)) return rc;
  int64_t r, c;
  matv(T[0], &r, &c);
  if (c != 16 && c != 32 && c != 64 && c != 128) return fail(TT_ERR_SHAPE, "%s: head dim %lld", nm, (long long)c);
  if (!(q.base > 1.0)) return fail(TT_ERR_ARG, "%s: base must exceed 1", nm);
  const TileArg t = T[0];
  const double base = q.base;
  return ctx->submit(label ? label : "rope_table", {acc_of(t, TT_W)},
                     [=](hipStream_t s, void*) { return tile_rope_table(s, r, c, base, Fp(t)); });
}

int op_swiglu(tt_ctx* ctx, const TileArg* T, int n, const char* label, bool bwd) {
  const char* nm = bwd ? "TT_OP_SWIGLU_BWD" : "TT_OP_SWIGLU_FWD";
  if (n < 3 || n % 3 || n / 3 > 16) return fail(TT_ERR_ARG, "%s: 1..16 tile triples", nm);
  if (int rc = need_f32(T, n, nm)) return rc;
  std::vector<Access> acc;
  for (int i = 0; i < n; i += 3) {
    if (elems(T[i]) != elems(T[i + 1]) || elems(T[i]) != elems(T[i + 2]))
      return fail(TT_ERR_SHAPE, "%s: triple %d: element counts differ", nm, i / 3);
    if (bwd) {  // dh, a, b: a and b replaced by their gradients
      acc.push_back(acc_of(T[i], TT_R));
      acc.push_back(acc_of(T[i + 1], TT_RW));
      acc.push_back(acc_of(T[i + 2], TT_RW));
    } else {    // a, b, h
      acc.push_back(acc_of(T[i], TT_R));
      acc.push_back(acc_of(T[i + 1], TT_R));
      acc.push_back(acc_of(T[i + 2], TT_W));
    }
  }
  std::vector<TileArg> tl(T, T + n);
  return ctx->submit(label ? label : (bwd ? "swiglu_bwd" : "swiglu"), std::move(acc), [=](hipStream_t s, void*) {
    for (int i = 0; i < n; i += 3) {
      const int64_t cnt = elems(tl[i]);
      const int rc = bwd ? tile_swiglu_bwd(s, cnt, Fp(tl[i]), Fp(tl[i + 1]), Fp(tl[i + 2]), Fp(tl[i + 1]),
                                           Fp(tl[i + 2]))
                         : tile_swiglu_fwd(s, cnt, Fp(tl[i]), Fp(tl[i + 1]), Fp(tl[i + 2]));
      if (rc) return rc;
    }
    return TT_OK;
  });
}

}  // namespace

size_t layernorm_fwd_workspace(int64_t n, int64_t rows) {
  return n > 1 ? align_up((size_t)n * rows * 3 * sizeof(float)) : 0;
}

size_t layernorm_bwd_workspace(int64_t n, int64_t rows, int64_t cols) {
  const size_t phases = (n > 1 ? align_up((size_t)n * rows * 2 * sizeof(float)) : 0) +
                        tile_layernorm_bwd_workspace(rows, cols);
  return n > 1 ? std::max(phases, tile_layernorm_bwd_multi_workspace(rows, n * cols)) : phases;
}

int submit_op(tt_ctx* ctx, int op, const TileArg* T, int n, const void* sc, size_t size, const char* label,
              bool grow) {
  if (!ctx) return fail(TT_ERR_ARG, "tt_submit: null context");
  if (n < 0 || (n > 0 && !T)) return fail(TT_ERR_ARG, "tt_submit: bad tile list");
  for (int i = 0; i < n; ++i)
    if (!T[i].t || T[i].t->ctx != ctx || T[i].lin < 0 || T[i].lin >= T[i].t->ntiles)
      return fail(TT_ERR_ARG, "tt_submit: tile %d is null, out of range or of another context", i);
  switch (op) {
    case TT_OP_FILL: {
      tt_op_fill q;
      if (int rc = scal(sc, size, "TT_OP_FILL", &q)) return rc;
      return op_fill(ctx, T, n, q, label);
    }
    case TT_OP_GEMM:
    case TT_OP_GEMM_BATCH:
    case TT_OP_GEMM_KSUM: {
      tt_op_gemm q;
      if (int rc = scal(sc, size, "TT_OP_GEMM*", &q)) return rc;
      if (op == TT_OP_GEMM) return op_gemm(ctx, T, n, q, label, grow);
      if (op == TT_OP_GEMM_BATCH) return op_gemm_batch(ctx, T, n, q, label, grow);
      return op_gemm_ksum(ctx, T, n, q, label, grow);
    }
    case TT_OP_LAYERNORM_FWD:
    case TT_OP_LAYERNORM_BWD: {
      tt_op_layernorm q;
      if (int rc = scal(sc, size, "TT_OP_LAYERNORM*", &q)) return rc;
      return op == TT_OP_LAYERNORM_FWD ? op_ln_fwd(ctx, T, n, q, label, grow) : op_ln_bwd(ctx, T, n, q, label, grow);
    }
    case TT_OP_ATTENTION_FWD:
    case TT_OP_ATTENTION_PREP:
    case TT_OP_ATTENTION_BWD: {
      tt_op_attention q;
      if (int rc = scal(sc, size, "TT_OP_ATTENTION*", &q)) return rc;
      if (op == TT_OP_ATTENTION_FWD) return op_att_fwd(ctx, T, n, q, label);
      if (op == TT_OP_ATTENTION_PREP) return op_att_prep(ctx, T, n, q, label);
      return op_att_bwd(ctx, T, n, q, label, grow);
    }
    case TT_OP_XENTROPY_STATS:
      return op_xe_stats(ctx, T, n, label);
    case TT_OP_XENTROPY_MERGE:
      if (sc || size) {
        tt_op_xe_groups q;
        if (int rc = scal(sc, size, "TT_OP_XENTROPY_MERGE", &q)) return rc;
        return op_xe_merge(ctx, T, n, &q, label);
      }
      return op_xe_merge(ctx, T, n, nullptr, label);
    case TT_OP_XENTROPY_LOSS:
    case TT_OP_XENTROPY_GRAD: {
      tt_op_xentropy q;
      if (int rc = scal(sc, size, "TT_OP_XENTROPY*", &q)) return rc;
      return op == TT_OP_XENTROPY_LOSS ? op_xe_loss(ctx, T, n, q, label) : op_xe_grad(ctx, T, n, q, label);
    }
    case TT_OP_ADAMW:
    case TT_OP_ADAMW_ADVANCE:
    case TT_OP_SGD: {
      tt_op_optim q;
      if (int rc = scal(sc, size, "TT_OP_ADAMW/SGD", &q)) return rc;
      if (op == TT_OP_ADAMW) return op_adamw(ctx, T, n, q, label);
      if (op == TT_OP_ADAMW_ADVANCE) return op_adamw_advance(ctx, T, n, q, label);
      return op_sgd(ctx, T, n, q, label);
    }
    case TT_OP_EMBEDDING_FWD:
    case TT_OP_EMBEDDING_TOKEN_FWD:
    case TT_OP_EMBEDDING_BWD:
    case TT_OP_EMBEDDING_POS_BWD: {
      tt_op_embedding q;
      if (int rc = scal(sc, size, "TT_OP_EMBEDDING*", &q)) return rc;
      if (op == TT_OP_EMBEDDING_FWD || op == TT_OP_EMBEDDING_TOKEN_FWD)
        return op_emb_fwd(ctx, T, n, q, label, op == TT_OP_EMBEDDING_FWD);
      if (op == TT_OP_EMBEDDING_BWD) return op_emb_bwd(ctx, T, n, q, label);
      return op_emb_pos_bwd(ctx, T, n, q, label);
    }
    case TT_OP_EMBEDDING_INDEX:
      return op_emb_index(ctx, T, n, label);
    case TT_OP_REDUCE_ROWS: {
      tt_op_reduce q;
      if (int rc = scal(sc, size, "TT_OP_REDUCE_ROWS", &q)) return rc;
      return op_reduce(ctx, T, n, q, label, grow);
    }
    case TT_OP_SPLIT_TOKENS:
      return op_split(ctx, T, n, label);
    case TT_OP_RMSNORM_FWD:
    case TT_OP_RMSNORM_BWD: {
      tt_op_layernorm q;
      if (int rc = scal(sc, size, "TT_OP_RMSNORM*", &q)) return rc;
      return op == TT_OP_RMSNORM_FWD ? op_rms_fwd(ctx, T, n, q, label) : op_rms_bwd(ctx, T, n, q, label, grow);
    }
    case TT_OP_ROPE:
    case TT_OP_ROPE_TABLE: {
      tt_op_rope q;
      if (int rc = scal(sc, size, "TT_OP_ROPE*", &q)) return rc;
      return op == TT_OP_ROPE ? op_rope(ctx, T, n, q, label) : op_rope_table(ctx, T, n, q, label);
    }
    case TT_OP_SWIGLU_FWD:
    case TT_OP_SWIGLU_BWD:
      return op_swiglu(ctx, T, n, label, op == TT_OP_SWIGLU_BWD);
    case TT_OP_COPY_IN: {
      tt_op_copy q;
      if (int rc = scal(sc, size, "TT_OP_COPY_IN", &q)) return rc;
      return op_copy_in(ctx, T, n, q, label);
    }
    default:
      return fail(TT_ERR_ARG, "tt_submit: unknown op %d", op);
  }
}

}  // namespace tt

extern "C" int tt_submit(tt_ctx* ctx, int op, const tt_tile* tiles, int ntiles, const void* scalars,
                         size_t scalars_size) {
  tt::clear_error();
  if (!ctx || ntiles < 0 || (ntiles > 0 && !tiles)) return tt::fail(TT_ERR_ARG, "tt_submit: bad argument");
  std::vector<tt::TileArg> T(ntiles);
  for (int i = 0; i < ntiles; ++i) {
    tt_tensor* t = tiles[i].tensor;
    if (!t) return tt::fail(TT_ERR_ARG, "tt_submit: tile %d has a null tensor", i);
    for (int d = 0; d < t->ndim; ++d)
      if (tiles[i].tile[d] < 0 || tiles[i].tile[d] >= t->grid[d])
        return tt::fail(TT_ERR_ARG, "tt_submit: tile %d index %lld out of range on axis %d", i,
                        (long long)tiles[i].tile[d], d);
    T[i] = tt::TileArg{t, t->lin(tiles[i].tile)};
  }
  return tt::submit_op(ctx, op, T.data(), ntiles, scalars, scalars_size, nullptr, true);
}
