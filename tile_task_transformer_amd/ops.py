"""Tile ops of libtiletask with the C names; arguments marshalled only.

Buffers: torch tensors on the GPU (or raw device addresses). Streams:
torch.cuda.Stream, a raw hipStream_t, or None for the default stream. See
include/tiletask.h for the meaning, layout and error behaviour of every
argument; each call raises TTError on a non-zero return code.
"""
from __future__ import annotations

from ._lib import (TT_EPI_NONE, check, lib, ptr, stream_handle, TT_EPI_BIAS, TT_EPI_RES, TT_EPI_GELU,  # noqa: F401
                   TT_EPI_GELU_BWD, TT_LN_PARTIAL, TT_LN_MERGE, TT_LN_APPLY, TT_LN_FUSED, TT_SM_STATS,
                   TT_SM_MERGE, TT_SM_APPLY, TT_XE_LOSS, TT_XE_GRAD, TT_XE_STATS, TT_ATT_PREP, TT_ATT_GRAD,
                   TT_EMB_TOKEN, TT_EMB_POS, TT_EPI_XSTATS, TT_PROBE_READ, TT_PROBE_WRITE, TT_PROBE_COPY, TT_PROBE_NONTEMPORAL)

__all__ = [
    "tile_gemm", "tile_gemm_ws", "tile_gemm_workspace", "tile_gemm_ksum", "tile_gemm_batch", "tile_gemm_batch_ws",
    "tile_gemm_batch_workspace", "tile_gemm_ksum_ex", "tile_layernorm_fwd",
    "tile_layernorm_bwd", "tile_layernorm_bwd_workspace", "tile_softmax",
    "tile_xentropy", "tile_xentropy_multi", "tile_attention_fwd", "tile_attention_bwd",
    "tile_attention_bwd_workspace", "tile_attention_bwd_ws", "tile_gemm_ksum_workspace", "tt_probe_hbm", "tile_gemm_batch_xstats",
    "tile_xentropy_merge_groups", "TT_EPI_XSTATS",
    "TT_PROBE_READ", "TT_PROBE_WRITE", "TT_PROBE_COPY", "TT_PROBE_NONTEMPORAL", "tile_fused_adamw",
    "tile_fused_adamw_multi",
    "tile_adamw_advance", "tile_sgd", "tile_sgd_multi",
    "tile_embedding_fwd", "tile_embedding_index", "tile_embedding_bwd", "tile_reduce_rows",
    "tile_reduce_rows_workspace", "tile_reduce_rows_multi", "tile_fill", "tile_fill_multi", "tile_split_tokens",
    "tt_probe_mfma_f32", "tile_layernorm_fwd_multi", "tile_layernorm_bwd_multi",
    "tile_layernorm_bwd_multi_workspace", "tile_rmsnorm_fwd", "tile_rmsnorm_bwd", "tile_rmsnorm_bwd_workspace",
    "tile_rope_table", "tile_rope", "tile_rope_multi", "tile_swiglu_fwd", "tile_swiglu_bwd",
    "TT_EPI_NONE", "TT_EPI_BIAS", "TT_EPI_RES", "TT_EPI_GELU", "TT_EPI_GELU_BWD", "TT_LN_PARTIAL",
    "TT_LN_MERGE", "TT_LN_APPLY", "TT_LN_FUSED", "TT_SM_STATS", "TT_SM_MERGE", "TT_SM_APPLY", "TT_XE_LOSS",
    "TT_XE_GRAD", "TT_XE_STATS", "TT_ATT_PREP", "TT_ATT_GRAD", "TT_EMB_TOKEN", "TT_EMB_POS",
]


def tile_gemm(stream, transA, transB, m, n, k, alpha, A, lda, B, ldb, beta, C, ldc, epilogue=TT_EPI_NONE,
              bias=None, res=None, ldr=0, aux=None, ldaux=0):
    return check(lib.tile_gemm(stream_handle(stream), transA, transB, m, n, k, alpha, ptr(A), lda, ptr(B), ldb,
                               beta, ptr(C), ldc, epilogue, ptr(bias), ptr(res), ldr, ptr(aux), ldaux))


def tile_gemm_ws(stream, transA, transB, m, n, k, alpha, A, lda, B, ldb, beta, C, ldc, epilogue=TT_EPI_NONE,
                 bias=None, res=None, ldr=0, aux=None, ldaux=0, workspace=None, workspace_bytes=0):
    return check(lib.tile_gemm_ws(stream_handle(stream), transA, transB, m, n, k, alpha, ptr(A), lda, ptr(B), ldb,
                                  beta, ptr(C), ldc, epilogue, ptr(bias), ptr(res), ldr, ptr(aux), ldaux,
                                  ptr(workspace), workspace_bytes))


def tile_gemm_workspace(m, n, k):
    return lib.tile_gemm_workspace(m, n, k)


def tile_gemm_ksum(stream, m, n, ks, alpha, As, ldas, Bs, ldbs, beta, C, ldc, transB=0):
    """C = alpha * sum_t A_t op(B_t) + beta * C; pairs given as equal-length lists."""
    import ctypes as C_
    cnt = len(As)
    i64 = lambda xs: (C_.c_int64 * max(cnt, 1))(*[int(x) for x in xs])  # noqa: E731
    ptrs = lambda xs: (C_.c_void_p * max(cnt, 1))(*[ptr(x) for x in xs])  # noqa: E731
    return check(lib.tile_gemm_ksum(stream_handle(stream), cnt, transB, m, n, i64(ks), alpha, ptrs(As), i64(ldas),
                                    ptrs(Bs), i64(ldbs), beta, ptr(C), ldc))


def tile_gemm_ksum_ex(stream, m, n, ks, alpha, As, ldas, Bs, ldbs, beta, C, ldc, transB=0, epilogue=TT_EPI_NONE,
                      bias=None, res=None, ldr=0, aux=None, ldaux=0, workspace=None, workspace_bytes=0):
    """tile_gemm_ksum followed by tile_gemm's epilogue on the whole sum;
    with a workspace, tile_gemm_ksum_ws (split K for outputs of few blocks)."""
    import ctypes as C_
    cnt = len(As)
    i64 = lambda xs: (C_.c_int64 * max(cnt, 1))(*[int(x) for x in xs])  # noqa: E731
    ptrs = lambda xs: (C_.c_void_p * max(cnt, 1))(*[ptr(x) for x in xs])  # noqa: E731
    args = (stream_handle(stream), cnt, transB, m, n, i64(ks), alpha, ptrs(As), i64(ldas), ptrs(Bs), i64(ldbs), beta,
            ptr(C), ldc, epilogue, ptr(bias), ptr(res), ldr, ptr(aux), ldaux)
    if workspace is None:
        return check(lib.tile_gemm_ksum_ex(*args))
    return check(lib.tile_gemm_ksum_ws(*args, ptr(workspace), workspace_bytes))


def tile_gemm_ksum_workspace(m, n):
    return lib.tile_gemm_ksum_workspace(m, n)


def _batch_args(ms, ns, As, ldas, Bs, ldbs, Cs, ldcs):
    import ctypes as C_
    cnt = len(Cs)
    per = lambda x: list(x) if isinstance(x, (list, tuple)) else [x] * cnt  # noqa: E731
    i64 = lambda xs: (C_.c_int64 * max(cnt, 1))(*[int(x) for x in per(xs)])  # noqa: E731
    ptrs = lambda xs: (C_.c_void_p * max(cnt, 1))(*[ptr(x) for x in xs])  # noqa: E731
    return cnt, i64(ms), i64(ns), ptrs(As), i64(ldas), ptrs(Bs), i64(ldbs), ptrs(Cs), i64(ldcs)


def tile_gemm_batch(stream, transA, transB, ms, ns, k, alpha, As, ldas, Bs, ldbs, beta, Cs, ldcs):
    """C_t = alpha op(A_t) op(B_t) + beta C_t; per-product sizes and leading
    dimensions as equal-length lists (an int is used for every product)."""
    cnt, m, n, a, la, b, lb, c, lc = _batch_args(ms, ns, As, ldas, Bs, ldbs, Cs, ldcs)
    return check(lib.tile_gemm_batch(stream_handle(stream), cnt, transA, transB, m, n, k, alpha, a, la, b, lb, beta,
                                     c, lc))


def tile_gemm_batch_ws(stream, transA, transB, ms, ns, k, alpha, As, ldas, Bs, ldbs, beta, Cs, ldcs, workspace,
                       workspace_bytes):
    cnt, m, n, a, la, b, lb, c, lc = _batch_args(ms, ns, As, ldas, Bs, ldbs, Cs, ldcs)
    return check(lib.tile_gemm_batch_ws(stream_handle(stream), cnt, transA, transB, m, n, k, alpha, a, la, b, lb,
                                        beta, c, lc, ptr(workspace), workspace_bytes))


def tile_gemm_batch_xstats(stream, transB, m, ns, k, alpha, As, ldas, Bs, ldbs, beta, Cs, ldcs, labels, v_off0,
                           v_tile, parts, part_stride):
    """Batched head products with the cross-entropy statistics of each
    64-column group of every C in the epilogue."""
    cnt, _, n, a, la, b, lb, c, lc = _batch_args([m] * len(Cs), ns, As, ldas, Bs, ldbs, Cs, ldcs)
    return check(lib.tile_gemm_batch_xstats(stream_handle(stream), cnt, transB, m, n, k, alpha, a, la, b, lb, beta, c,
                                            lc, ptr(labels), v_off0, v_tile, ptr(parts), part_stride))


def tile_xentropy_merge_groups(stream, rows, v_lens, group, parts, part_stride, lse, row_loss=None):
    import ctypes as C_
    cnt = len(v_lens)
    arr = (C_.c_int64 * max(cnt, 1))(*[int(x) for x in v_lens])
    return check(lib.tile_xentropy_merge_groups(stream_handle(stream), rows, cnt, arr, group, ptr(parts), part_stride,
                                                ptr(lse), ptr(row_loss)))


def tile_gemm_batch_workspace(ms, ns, k):
    import ctypes as C_
    cnt = len(ms)
    i64 = lambda xs: (C_.c_int64 * max(cnt, 1))(*[int(x) for x in xs])  # noqa: E731
    return lib.tile_gemm_batch_workspace(cnt, i64(ms), i64(ns), k)


def tile_layernorm_fwd(stream, phase, rows, cols, x, ldx, gamma, beta, parts, n_parts, part_stride, stats, y,
                       ldy, eps):
    return check(lib.tile_layernorm_fwd(stream_handle(stream), phase, rows, cols, ptr(x), ldx, ptr(gamma),
                                        ptr(beta), ptr(parts), n_parts, part_stride, ptr(stats), ptr(y), ldy, eps))


def tile_layernorm_bwd(stream, phase, rows, cols, n_total, dy, lddy, x, ldx, gamma, stats, parts, n_parts,
                       part_stride, dx, lddx, dx_acc, dgamma, dbeta, workspace):
    return check(lib.tile_layernorm_bwd(stream_handle(stream), phase, rows, cols, n_total, ptr(dy), lddy, ptr(x),
                                        ldx, ptr(gamma), ptr(stats), ptr(parts), n_parts, part_stride, ptr(dx),
                                        lddx, dx_acc, ptr(dgamma), ptr(dbeta), ptr(workspace)))


def tile_layernorm_bwd_workspace(rows, cols):
    return lib.tile_layernorm_bwd_workspace(rows, cols)


def tile_softmax(stream, phase, rows, cols, row_offset, col_offset, scale, causal, X, ldx, labels, parts,
                 n_parts, part_stride, lse, row_loss, Y, ldy, grad_scale):
    return check(lib.tile_softmax(stream_handle(stream), phase, rows, cols, row_offset, col_offset, scale, causal,
                                  ptr(X), ldx, ptr(labels), ptr(parts), n_parts, part_stride, ptr(lse),
                                  ptr(row_loss), ptr(Y), ldy, grad_scale))


def tile_xentropy(stream, phase, rows, v_len, v_off, labels, logits, ldz, lse, row_loss, loss, accumulate, inv_n):
    return check(lib.tile_xentropy(stream_handle(stream), phase, rows, v_len, v_off, ptr(labels), ptr(logits), ldz,
                                   ptr(lse), ptr(row_loss), ptr(loss), accumulate, inv_n))


def tile_xentropy_multi(stream, phase, rows, v_lens, v_offs, labels, logits, ldzs, parts=None, part_stride=0,
                        lse=None, inv_n=1.0):
    """STATS or GRAD of several vocab tiles (equal-length lists) in one launch."""
    import ctypes as C_
    cnt = len(logits)
    i64 = lambda xs: (C_.c_int64 * max(cnt, 1))(*[int(x) for x in xs])  # noqa: E731
    ptrs = (C_.c_void_p * max(cnt, 1))(*[ptr(x) for x in logits])
    return check(lib.tile_xentropy_multi(stream_handle(stream), phase, cnt, rows, i64(v_lens), i64(v_offs),
                                         ptr(labels), ptrs, i64(ldzs), ptr(parts), part_stride, ptr(lse), inv_n))


def tile_attention_fwd(stream, batch, heads, q_len, k_len, hd, q_off, k_off, Q, K, V, O, ml, lse, first, last,
                       scale):
    return check(lib.tile_attention_fwd(stream_handle(stream), batch, heads, q_len, k_len, hd, q_off, k_off, ptr(Q),
                                        ptr(K), ptr(V), ptr(O), ptr(ml), ptr(lse), first, last, scale))


def tile_attention_bwd(stream, phase, batch, heads, q_len, k_len, hd, q_off, k_off, Q, K, V, O, dO, lse, Dvec, dQ,
                       dK, dV, acc_dq, acc_dkv, scale):
    return check(lib.tile_attention_bwd(stream_handle(stream), phase, batch, heads, q_len, k_len, hd, q_off, k_off,
                                        ptr(Q), ptr(K), ptr(V), ptr(O), ptr(dO), ptr(lse), ptr(Dvec), ptr(dQ),
                                        ptr(dK), ptr(dV), acc_dq, acc_dkv, scale))


def tile_attention_bwd_workspace(batch, heads, q_len, k_len):
    return lib.tile_attention_bwd_workspace(batch, heads, q_len, k_len)


def tile_attention_bwd_ws(stream, phase, batch, heads, q_len, k_len, hd, q_off, k_off, Q, K, V, O, dO, lse, Dvec, dQ,
                          dK, dV, acc_dq, acc_dkv, scale, workspace, workspace_bytes):
    return check(lib.tile_attention_bwd_ws(stream_handle(stream), phase, batch, heads, q_len, k_len, hd, q_off, k_off,
                                           ptr(Q), ptr(K), ptr(V), ptr(O), ptr(dO), ptr(lse), ptr(Dvec), ptr(dQ),
                                           ptr(dK), ptr(dV), acc_dq, acc_dkv, scale, ptr(workspace),
                                           workspace_bytes))


def tile_fused_adamw(stream, n, p, g, m, v, lr, beta1, beta2, eps, weight_decay, bias_corr):
    return check(lib.tile_fused_adamw(stream_handle(stream), n, ptr(p), ptr(g), ptr(m), ptr(v), lr, beta1, beta2,
                                      eps, weight_decay, ptr(bias_corr)))


def tile_fused_adamw_multi(stream, ps, gs, ms, vs, lr, beta1, beta2, eps, weight_decay, bias_corr):
    """Tiles given as lists of equal length (torch tensors or device addresses)."""
    import ctypes as C
    k = len(ps)
    arr = lambda xs: (C.c_void_p * max(k, 1))(*[ptr(x) for x in xs])  # noqa: E731
    ns = (C.c_int64 * max(k, 1))(*[int(x.numel()) for x in ps])
    return check(lib.tile_fused_adamw_multi(stream_handle(stream), k, arr(ps), arr(gs), arr(ms), arr(vs), ns, lr,
                                            beta1, beta2, eps, weight_decay, ptr(bias_corr)))


def tile_sgd(stream, n, p, g, lr):
    return check(lib.tile_sgd(stream_handle(stream), n, ptr(p), ptr(g), lr))


def tile_sgd_multi(stream, ps, gs, lr):
    """Tiles given as lists of equal length (torch tensors or device addresses)."""
    import ctypes as C
    k = len(ps)
    arr = lambda xs: (C.c_void_p * max(k, 1))(*[ptr(x) for x in xs])  # noqa: E731
    ns = (C.c_int64 * max(k, 1))(*[int(x.numel()) for x in ps])
    return check(lib.tile_sgd_multi(stream_handle(stream), k, arr(ps), arr(gs), ns, lr))


def tile_adamw_advance(stream, step, bias_corr, beta1, beta2):
    return check(lib.tile_adamw_advance(stream_handle(stream), ptr(step), ptr(bias_corr), beta1, beta2))


def tile_embedding_fwd(stream, rows, cols, ids, vocab, v_off, v_len, wte, ld_wte, wpe, ld_wpe, seq_len, pos_offset,
                       out, ldo):
    return check(lib.tile_embedding_fwd(stream_handle(stream), rows, cols, ptr(ids), vocab, v_off, v_len, ptr(wte), ld_wte,
                                        ptr(wpe), ld_wpe, seq_len, pos_offset, ptr(out), ldo))


def tile_embedding_index(stream, rows, ids, sorted_ids, perm):
    return check(lib.tile_embedding_index(stream_handle(stream), rows, ptr(ids), ptr(sorted_ids), ptr(perm)))


def tile_embedding_bwd(stream, phase, rows, cols, sorted_ids, perm, v_off, v_len, seq_len, dh, lddh, dst, ld_dst):
    return check(lib.tile_embedding_bwd(stream_handle(stream), phase, rows, cols, ptr(sorted_ids), ptr(perm), v_off,
                                        v_len, seq_len, ptr(dh), lddh, ptr(dst), ld_dst))


def tile_reduce_rows(stream, rows, cols, X, ldx, out, beta, workspace):
    return check(lib.tile_reduce_rows(stream_handle(stream), rows, cols, ptr(X), ldx, ptr(out), beta, ptr(workspace)))


def tile_reduce_rows_workspace(rows, cols):
    return lib.tile_reduce_rows_workspace(rows, cols)


def tile_reduce_rows_multi(stream, rows, cols, Xs, ldxs, outs, beta, workspace, workspace_bytes):
    """Column sums of several tiles (equal-length lists) in one pair of launches."""
    import ctypes as C_
    cnt = len(outs)
    i64 = lambda xs: (C_.c_int64 * max(cnt, 1))(*[int(x) for x in xs])  # noqa: E731
    ptrs = lambda xs: (C_.c_void_p * max(cnt, 1))(*[ptr(x) for x in xs])  # noqa: E731
    return check(lib.tile_reduce_rows_multi(stream_handle(stream), cnt, rows, i64(cols), ptrs(Xs), i64(ldxs),
                                            ptrs(outs), beta, ptr(workspace), workspace_bytes))


def tile_fill(stream, n, dst, value):
    return check(lib.tile_fill(stream_handle(stream), n, ptr(dst), value))


def tile_fill_multi(stream, dsts, value):
    """Tiles given as a list of torch tensors (or (address, count) pairs)."""
    import ctypes as C
    k = len(dsts)
    ptrs = (C.c_void_p * max(k, 1))(*[ptr(x[0] if isinstance(x, tuple) else x) for x in dsts])
    ns = (C.c_int64 * max(k, 1))(*[int(x[1] if isinstance(x, tuple) else x.numel()) for x in dsts])
    return check(lib.tile_fill_multi(stream_handle(stream), k, ptrs, ns, value))


def tile_split_tokens(stream, batch, seq, tokens, ids, labels):
    return check(lib.tile_split_tokens(stream_handle(stream), batch, seq, ptr(tokens), ptr(ids), ptr(labels)))


def tt_probe_mfma_f32(stream, blocks, iters, out):
    """Launch the fp32 matrix-core peak probe; returns its flop count."""
    import ctypes as C
    f = C.c_double()
    check(lib.tt_probe_mfma_f32(stream_handle(stream), blocks, iters, ptr(out), C.byref(f)))
    return f.value


def tt_probe_hbm(stream, mode, src, dst, n, blocks):
    """Launch the HBM bandwidth probe; returns the bytes it moves."""
    import ctypes as C
    f = C.c_double()
    check(lib.tt_probe_hbm(stream_handle(stream), mode, ptr(src), ptr(dst), n, blocks, C.byref(f)))
    return f.value


def _arrs(n, *lists):
    import ctypes as C
    return [(C.c_void_p * max(n, 1))(*[ptr(x) for x in lst]) for lst in lists]


def tile_layernorm_fwd_multi(stream, rows, cols, xs, gammas, betas, stats, ys, eps=1e-5):
    """LayerNorm of a row block over several feature tiles in one pass."""
    import ctypes as C
    n = len(xs)
    c = (C.c_int64 * n)(*[int(v) for v in cols])
    x, g, b, y = _arrs(n, xs, gammas, betas, ys)
    return check(lib.tile_layernorm_fwd_multi(stream_handle(stream), n, rows, c, x, g, b, ptr(stats), y, eps))


def tile_layernorm_bwd_multi(stream, rows, cols, dys, xs, gammas, stats, dxs, dx_acc, dgammas, dbetas, workspace,
                             workspace_bytes):
    import ctypes as C
    n = len(xs)
    c = (C.c_int64 * n)(*[int(v) for v in cols])
    dy, x, g, dx, dg, db = _arrs(n, dys, xs, gammas, dxs, dgammas, dbetas)
    return check(lib.tile_layernorm_bwd_multi(stream_handle(stream), n, rows, c, dy, x, g, ptr(stats), dx, dx_acc,
                                              dg, db, ptr(workspace), workspace_bytes))


def tile_layernorm_bwd_multi_workspace(rows, total_cols):
    return lib.tile_layernorm_bwd_multi_workspace(rows, total_cols)


def tile_rmsnorm_fwd(stream, rows, cols, xs, gammas, rstd, ys, eps=1e-5):
    """RMSNorm of a row block over 1..16 feature tiles (the LLaMA block)."""
    import ctypes as C
    n = len(xs)
    c = (C.c_int64 * n)(*[int(v) for v in cols])
    x, g, y = _arrs(n, xs, gammas, ys)
    return check(lib.tile_rmsnorm_fwd(stream_handle(stream), n, rows, c, x, g, ptr(rstd), y, eps))


def tile_rmsnorm_bwd(stream, rows, cols, dys, xs, gammas, rstd, dxs, dx_acc, dgammas, workspace, workspace_bytes):
    import ctypes as C
    n = len(xs)
    c = (C.c_int64 * n)(*[int(v) for v in cols])
    dy, x, g, dx, dg = _arrs(n, dys, xs, gammas, dxs, dgammas)
    return check(lib.tile_rmsnorm_bwd(stream_handle(stream), n, rows, c, dy, x, g, ptr(rstd), dx, dx_acc, dg,
                                      ptr(workspace), workspace_bytes))


def tile_rmsnorm_bwd_workspace(rows, total_cols):
    return lib.tile_rmsnorm_bwd_workspace(rows, total_cols)


def tile_rope_table(stream, seq, hd, base, table):
    return check(lib.tile_rope_table(stream_handle(stream), seq, hd, float(base), ptr(table)))


def tile_rope(stream, x, rows, heads, hd, seq_len, pos_off, table, table_rows, inverse=False):
    """Rotary embedding of a [rows, heads, hd] q or k tile, in place."""
    return check(lib.tile_rope(stream_handle(stream), ptr(x), rows, heads, hd, seq_len, pos_off, ptr(table),
                               table_rows, int(inverse)))


def tile_rope_multi(stream, xs, rows, heads, hd, seq_len, pos_off, table, table_rows, inverse=False):
    """tile_rope on 1..4 equal tiles in one launch."""
    (x,) = _arrs(len(xs), xs)
    return check(lib.tile_rope_multi(stream_handle(stream), len(xs), x, rows, heads, hd, seq_len, pos_off,
                                     ptr(table), table_rows, int(inverse)))


def tile_swiglu_fwd(stream, n, a, b, h):
    return check(lib.tile_swiglu_fwd(stream_handle(stream), n, ptr(a), ptr(b), ptr(h)))


def tile_swiglu_bwd(stream, n, dh, a, b, da, db):
    return check(lib.tile_swiglu_bwd(stream_handle(stream), n, ptr(dh), ptr(a), ptr(b), ptr(da), ptr(db)))
