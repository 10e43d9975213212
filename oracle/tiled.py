"""Float64 tile decompositions of the GPT2 layers (part of the oracle).

TEST INFRASTRUCTURE: only tests/, the smoke check and the benchmark's
CPU-baseline leg may use this module.

The pith.science review of NNTile ("What carries the argument") describes
the method: every tensor is split into tiles along all of its axes and each
layer becomes tasks that read and write a few tiles; tile placement does not
change the mathematical result ("Core claim"). When a reduction axis is
split, each layer therefore needs a rule that combines per-tile partial
results into the untiled answer. This module writes each rule out plainly
so tests can check, in float64, that it reproduces the untiled layer of
``oracle.gpt2`` across many tile shapes (ragged last tiles included):

  * matmul split along K: partial products summed tile by tile;
  * LayerNorm statistics split along the feature axis: per-tile
    (count, mean, sum of squared deviations) merged pairwise with the
    parallel-variance update of Chan, Golub and LeVeque;
  * LayerNorm backward split along the feature axis: the two row sums
    sum(dxhat) and sum(dxhat * xhat) added over tiles;
  * softmax / cross-entropy split along the class axis: per-tile (row max,
    sum of exp(x - max)) merged by rescaling to the larger max;
  * causal attention split along query and key tiles: for each query tile a
    running (max, sum, unnormalised output) updated key tile by key tile
    (online softmax), key tiles that lie wholly above the diagonal skipped;
    the backward recomputes P from the saved logsumexp per tile pair and uses
    D = rowsum(dO * O) in place of rowsum(P * dP);
  * embedding backward split along vocab and token tiles: each vocab tile
    sums, in token order, the rows of dh whose id falls in the tile.
"""
from __future__ import annotations

import math
from typing import List, Tuple

import numpy as np


def tiles(n: int, t: int) -> List[Tuple[int, int]]:
    """[start, stop) of each tile of size t along an axis of length n; the
    last tile is ragged when t does not divide n."""
    return [(s, min(s + t, n)) for s in range(0, n, t)]


def matmul_ksplit(a: np.ndarray, b: np.ndarray, kt: int) -> np.ndarray:
    """C = A @ B with K split into tiles of kt, accumulated in tile order."""
    c = np.zeros((a.shape[0], b.shape[1]))
    for k0, k1 in tiles(a.shape[1], kt):
        c = c + a[:, k0:k1] @ b[k0:k1, :]
    return c


def ln_partial(x: np.ndarray):
    """Per-row (count, mean, M2) of one feature tile."""
    n = x.shape[-1]
    mean = x.mean(axis=-1)
    m2 = ((x - mean[..., None]) ** 2).sum(axis=-1)
    return float(n), mean, m2


def chan_merge(a, b):
    """Merge two (count, mean, M2) summaries of disjoint parts of a row."""
    na, ma, m2a = a
    nb, mb, m2b = b
    n = na + nb
    delta = mb - ma
    return n, ma + delta * (nb / n), m2a + m2b + delta * delta * (na * nb / n)


def ln_stats_tiled(x: np.ndarray, et: int, eps: float = 1e-5):
    """(mean, rstd) per row from feature tiles of width et."""
    acc = None
    for c0, c1 in tiles(x.shape[-1], et):
        part = ln_partial(x[..., c0:c1])
        acc = part if acc is None else chan_merge(acc, part)
    n, mean, m2 = acc
    return mean, 1.0 / np.sqrt(m2 / n + eps)


def ln_fwd_tiled(x, g, b, et: int, eps: float = 1e-5):
    mean, rstd = ln_stats_tiled(x, et, eps)
    y = np.empty_like(x)
    for c0, c1 in tiles(x.shape[-1], et):
        y[..., c0:c1] = (x[..., c0:c1] - mean[..., None]) * rstd[..., None] * g[c0:c1] + b[c0:c1]
    return y, (mean, rstd)


def ln_bwd_tiled(dy, x, g, mean, rstd, et: int, row_tile: int):
    """LayerNorm backward with features split in et and rows in row_tile.

    Phase 1 per feature tile: s1 = sum dxhat, s2 = sum dxhat*xhat (added over
    tiles). Phase 2 per feature tile: dx from the merged sums. dg and db are
    accumulated over row tiles in order."""
    d = x.shape[-1]
    xs = x.reshape(-1, d)
    dys = dy.reshape(-1, d)
    mu, rs = mean.reshape(-1), rstd.reshape(-1)
    dx = np.empty_like(xs)
    dg = np.zeros(d)
    db = np.zeros(d)
    for r0, r1 in tiles(xs.shape[0], row_tile):
        s1 = np.zeros(r1 - r0)
        s2 = np.zeros(r1 - r0)
        for c0, c1 in tiles(d, et):
            xhat = (xs[r0:r1, c0:c1] - mu[r0:r1, None]) * rs[r0:r1, None]
            dxhat = dys[r0:r1, c0:c1] * g[c0:c1]
            s1 += dxhat.sum(axis=-1)
            s2 += (dxhat * xhat).sum(axis=-1)
        for c0, c1 in tiles(d, et):
            xhat = (xs[r0:r1, c0:c1] - mu[r0:r1, None]) * rs[r0:r1, None]
            dxhat = dys[r0:r1, c0:c1] * g[c0:c1]
            dx[r0:r1, c0:c1] = rs[r0:r1, None] * (dxhat - s1[:, None] / d - xhat * (s2[:, None] / d))
            dg[c0:c1] += (dys[r0:r1, c0:c1] * xhat).sum(axis=0)
            db[c0:c1] += dys[r0:r1, c0:c1].sum(axis=0)
    return dx.reshape(x.shape), dg, db


def softmax_partial(x: np.ndarray):
    """Per-row (max, sum exp(x - max)) of one class tile."""
    m = x.max(axis=-1)
    return m, np.exp(x - m[..., None]).sum(axis=-1)


def softmax_merge(a, b):
    ma, sa = a
    mb, sb = b
    m = np.maximum(ma, mb)
    return m, sa * np.exp(ma - m) + sb * np.exp(mb - m)


def logsumexp_tiled(z: np.ndarray, vt: int) -> np.ndarray:
    acc = None
    for c0, c1 in tiles(z.shape[-1], vt):
        part = softmax_partial(z[..., c0:c1])
        acc = part if acc is None else softmax_merge(acc, part)
    m, s = acc
    return m + np.log(s)


def cross_entropy_tiled(z: np.ndarray, y: np.ndarray, vt: int, row_tile: int):
    """Mean cross-entropy and its gradient from class tiles of width vt.

    Per class tile: partial stats and, for rows whose label falls in the
    tile, the target logit. Then lse per row, the loss, and per class tile
    dz = (exp(z - lse) - onehot) / N."""
    n = z.shape[0]
    lse = logsumexp_tiled(z, vt)
    zy = np.zeros(n)
    dz = np.empty_like(z)
    for c0, c1 in tiles(z.shape[1], vt):
        inside = (y >= c0) & (y < c1)
        rows = np.nonzero(inside)[0]
        zy[rows] = z[rows, y[rows]]
        blk = np.exp(z[:, c0:c1] - lse[:, None])
        blk[rows, y[rows] - c0] -= 1.0
        dz[:, c0:c1] = blk / n
    row_loss = lse - zy
    total = 0.0
    for r0, r1 in tiles(n, row_tile):
        total += row_loss[r0:r1].sum()
    return total / n, dz, lse


def attention_fwd_tiled(q, k, v, qt: int, kt: int):
    """Causal attention for one head, q/k/v [T, hd], query tiles of qt and
    key tiles of kt, by the online softmax. Returns O [T, hd], lse [T]."""
    t, hd = q.shape
    scale = 1.0 / math.sqrt(hd)
    o = np.zeros((t, hd))
    lse = np.zeros(t)
    for q0, q1 in tiles(t, qt):
        m = np.full(q1 - q0, -np.inf)
        l = np.zeros(q1 - q0)
        acc = np.zeros((q1 - q0, hd))
        for k0, k1 in tiles(t, kt):
            if k0 > q1 - 1:          # key tile entirely in the masked future
                break
            s = (q[q0:q1] @ k[k0:k1].T) * scale
            qi = np.arange(q0, q1)[:, None]
            kj = np.arange(k0, k1)[None, :]
            s = np.where(kj > qi, -np.inf, s)
            m_new = np.maximum(m, s.max(axis=1))
            alpha = np.exp(m - m_new)
            p = np.exp(s - m_new[:, None])
            l = l * alpha + p.sum(axis=1)
            acc = acc * alpha[:, None] + p @ v[k0:k1]
            m = m_new
        o[q0:q1] = acc / l[:, None]
        lse[q0:q1] = m + np.log(l)
    return o, lse


def attention_bwd_tiled(do, q, k, v, o, lse, qt: int, kt: int):
    """Backward of attention_fwd_tiled by tile pairs: P recomputed from lse,
    D = rowsum(dO * O) replaces rowsum(P * dP)."""
    t, hd = q.shape
    scale = 1.0 / math.sqrt(hd)
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    dvec = (do * o).sum(axis=1)
    for q0, q1 in tiles(t, qt):
        for k0, k1 in tiles(t, kt):
            if k0 > q1 - 1:
                break
            s = (q[q0:q1] @ k[k0:k1].T) * scale
            qi = np.arange(q0, q1)[:, None]
            kj = np.arange(k0, k1)[None, :]
            p = np.where(kj > qi, 0.0, np.exp(s - lse[q0:q1, None]))
            dv[k0:k1] += p.T @ do[q0:q1]
            dp = do[q0:q1] @ v[k0:k1].T
            ds = p * (dp - dvec[q0:q1, None])
            dq[q0:q1] += (ds @ k[k0:k1]) * scale
            dk[k0:k1] += (ds.T @ q[q0:q1]) * scale
    return dq, dk, dv


def embedding_bwd_tiled(dh: np.ndarray, ids: np.ndarray, vocab: int, vt: int, et: int,
                        row_tile: int) -> np.ndarray:
    """dwte[v] = sum of dh rows whose id is v, built per (vocab tile, embd
    tile, token tile), rows added in token order."""
    n, d = dh.shape
    out = np.zeros((vocab, d))
    for v0, v1 in tiles(vocab, vt):
        for c0, c1 in tiles(d, et):
            for r0, r1 in tiles(n, row_tile):
                for r in range(r0, r1):
                    if v0 <= ids[r] < v1:
                        out[ids[r], c0:c1] += dh[r, c0:c1]
    return out
