"""Untiled float64 LLaMA-style forward, backward and optimiser step (the oracle).

TEST INFRASTRUCTURE: only tests/, the smoke check and the benchmark's
CPU-baseline leg may use this module.

What it follows. The NNTile README ("Minimal working GPT example" and the
notebook list under it) names LLaMa as the second model its examples train,
next to GPT2, and the pith.science review ("Editorial extensions") notes that
the same tile tasks can be assembled into other architectures. The pages
give no definition of the LLaMa block; the readings below take the published
LLaMA architecture (Touvron et al., 2023: pre-normalisation with RMSNorm,
SwiGLU feed-forward, rotary position embeddings, no biases) in its plainest
form:

  L1 block = pre-norm: h += Attn(RMS1(h)); h += MLP(RMS2(h)); final RMSNorm.
  L2 RMSNorm: y = x / sqrt(mean(x^2) + eps) * g over the embedding axis, a
     gain and no bias, eps 1e-5 inside the square root.
  L3 rotary embedding on q and k of every head after the projection, at the
     token's absolute position t in its sequence: for i < hd/2 the pair
     (x_i, x_{i + hd/2}) is rotated by the angle t * base^(-2i/hd), base
     10000 (the half-split pairing; pairing adjacent elements instead is the
     same model up to a fixed permutation of each head's q and k columns).
  L4 MLP: SwiGLU, (silu(n W_gate) * (n W_up)) W_down, silu(a) = a sigmoid(a),
     the hidden width from the config.
  L5 no biases on any linear layer; no position-embedding table.
  L6 LM head untied: its own [V, d] weight, logits = nf w_head^T.
  L7 attention (causal, 1/sqrt(hd)), the mean next-token loss, and the
     AdamW / SGD update as for GPT2 (``oracle.gpt2`` R6-R9), decay on every
     parameter.

The arithmetic below is the plain definition of each layer; the only
library primitive used is numpy's matmul (and exp/log/sin/cos/sqrt).
"""
from __future__ import annotations

from typing import Dict, List, Tuple

import numpy as np

from . import gpt2 as _g

ROPE_BASE = 10000.0


# --------------------------------------------------------------------- layers

def rmsnorm_fwd(x: np.ndarray, g: np.ndarray, eps: float = 1e-5):
    """y = x / sqrt(mean(x^2) + eps) * g over the last axis (L2).

    Returns y and rstd per row, the statistic the backward needs."""
    rstd = 1.0 / np.sqrt((x * x).mean(axis=-1, keepdims=True) + eps)
    return x * rstd * g, rstd[..., 0]


def rmsnorm_bwd(dy: np.ndarray, x: np.ndarray, g: np.ndarray, rstd: np.ndarray):
    """Gradient of rmsnorm_fwd: returns dx, dg.

    With n = x * rstd and dn = dy * g (rstd depends on every x of the row):
      dx = rstd * (dn - n * mean(dn * n)),   dg = sum over rows of dy * n."""
    n = x * rstd[..., None]
    dn = dy * g
    dx = rstd[..., None] * (dn - n * (dn * n).mean(axis=-1, keepdims=True))
    axes = tuple(range(dy.ndim - 1))
    return dx, (dy * n).sum(axis=axes)


def rope_angles(seq: int, hd: int, base: float = ROPE_BASE) -> np.ndarray:
    """[seq, hd/2] rotation angles t * base^(-2i/hd) (L3)."""
    i = np.arange(hd // 2, dtype=np.float64)
    theta = base ** (-2.0 * i / hd)
    return np.arange(seq, dtype=np.float64)[:, None] * theta[None, :]


def rope_fwd(x: np.ndarray, ang: np.ndarray) -> np.ndarray:
    """Rotate the pairs (x_i, x_{i+hd/2}) of the last axis by ang[t, i], t
    being the second-to-last axis (L3)."""
    h = x.shape[-1] // 2
    c, s = np.cos(ang), np.sin(ang)
    x1, x2 = x[..., :h], x[..., h:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def rope_bwd(dy: np.ndarray, ang: np.ndarray) -> np.ndarray:
    """Gradient of rope_fwd: each 2x2 rotation is orthogonal, so its
    transpose is the rotation by the opposite angle."""
    return rope_fwd(dy, -ang)


def silu(a: np.ndarray) -> np.ndarray:
    return a / (1.0 + np.exp(-a))


def silu_grad(a: np.ndarray) -> np.ndarray:
    """d silu / da = s (1 + a (1 - s)) with s = sigmoid(a)."""
    s = 1.0 / (1.0 + np.exp(-a))
    return s * (1.0 + a * (1.0 - s))


def swiglu_fwd(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """silu(a) * b (L4): a = n W_gate, b = n W_up."""
    return silu(a) * b


def swiglu_bwd(dh: np.ndarray, a: np.ndarray, b: np.ndarray):
    """Gradient of swiglu_fwd: (da, db) = (dh * b * silu'(a), dh * silu(a))."""
    return dh * b * silu_grad(a), dh * silu(a)


# ---------------------------------------------------------------------- model

def param_names(n_layer: int) -> List[str]:
    """Parameter order: wte, per block (attn_norm_g, w_qkv, w_o, mlp_norm_g,
    w_gate, w_up, w_down), then norm_f_g and w_head."""
    names = ["wte"]
    for l in range(n_layer):
        p = f"h{l}."
        names += [p + s for s in ("attn_norm_g", "w_qkv", "w_o", "mlp_norm_g", "w_gate", "w_up", "w_down")]
    return names + ["norm_f_g", "w_head"]


def forward(params: Dict[str, np.ndarray], x: np.ndarray, y: np.ndarray, n_layer: int,
            n_head: int, eps: float = 1e-5, rope_base: float = ROPE_BASE):
    """LLaMA-style forward + loss (L1-L7). params are promoted to float64.

    Returns (loss, cache) where cache holds every activation the backward
    needs, plus the logits and the per-row logsumexp."""
    P = {k: np.asarray(v, np.float64) for k, v in params.items()}
    B, T = x.shape
    d = P["wte"].shape[1]
    hd = d // n_head
    ang = rope_angles(T, hd, rope_base)
    cache = {"x": x, "y": y, "P": P, "blocks": [], "ang": ang}
    h = P["wte"][x]
    for l in range(n_layer):
        p = f"h{l}."
        c = {"h_in": h}
        n1, r1 = rmsnorm_fwd(h, P[p + "attn_norm_g"], eps)
        qkv = n1 @ P[p + "w_qkv"]
        q, k, v = (_g._heads(qkv[..., i * d:(i + 1) * d], n_head) for i in range(3))
        qr, kr = rope_fwd(q, ang), rope_fwd(k, ang)
        o, pr = _g.causal_attention_fwd(qr, kr, v)
        om = _g._merge_heads(o)
        h_mid = h + om @ P[p + "w_o"]
        n2, r2 = rmsnorm_fwd(h_mid, P[p + "mlp_norm_g"], eps)
        a = n2 @ P[p + "w_gate"]
        b = n2 @ P[p + "w_up"]
        hh = swiglu_fwd(a, b)
        h = h_mid + hh @ P[p + "w_down"]
        c.update(n1=n1, r1=r1, qr=qr, kr=kr, v=v, p=pr, om=om, h_mid=h_mid, n2=n2, r2=r2, a=a, b=b, hh=hh)
        cache["blocks"].append(c)
    cache["h_last"] = h
    nf, rf = rmsnorm_fwd(h, P["norm_f_g"], eps)
    z = nf.reshape(B * T, d) @ P["w_head"].T
    loss, dz, lse = _g.cross_entropy(z, y.reshape(-1))
    cache.update(nf=nf, rf=rf, z=z, dz=dz, lse=lse, loss=loss)
    return loss, cache


def row_losses(params, x, y, n_layer: int, n_head: int, eps: float = 1e-5) -> np.ndarray:
    """Per-token next-token losses [B, T] (the terms whose mean is the loss)."""
    _, cache = forward(params, x, y, n_layer, n_head, eps)
    z, lse = cache["z"], cache["lse"]
    return (lse - z[np.arange(z.shape[0]), y.reshape(-1)]).reshape(x.shape)


def backward(cache, n_layer: int, n_head: int) -> Dict[str, np.ndarray]:
    """Analytic gradients of the mean loss w.r.t. every parameter (float64)."""
    P, x, ang = cache["P"], cache["x"], cache["ang"]
    B, T = x.shape
    d = P["wte"].shape[1]
    G: Dict[str, np.ndarray] = {}
    dz = cache["dz"]
    G["w_head"] = dz.T @ cache["nf"].reshape(B * T, d)
    dnf = (dz @ P["w_head"]).reshape(B, T, d)
    dh, G["norm_f_g"] = rmsnorm_bwd(dnf, cache["h_last"], P["norm_f_g"], cache["rf"])
    for l in reversed(range(n_layer)):
        p = f"h{l}."
        c = cache["blocks"][l]
        # MLP branch: h = h_mid + swiglu(n2 W_gate, n2 W_up) W_down
        inner = c["hh"].shape[-1]
        G[p + "w_down"] = c["hh"].reshape(-1, inner).T @ dh.reshape(-1, d)
        dhh = dh @ P[p + "w_down"].T
        da, db = swiglu_bwd(dhh, c["a"], c["b"])
        n2 = c["n2"].reshape(-1, d)
        G[p + "w_gate"] = n2.T @ da.reshape(-1, inner)
        G[p + "w_up"] = n2.T @ db.reshape(-1, inner)
        dn2 = da @ P[p + "w_gate"].T + db @ P[p + "w_up"].T
        dx2, G[p + "mlp_norm_g"] = rmsnorm_bwd(dn2, c["h_mid"], P[p + "mlp_norm_g"], c["r2"])
        dh = dh + dx2
        # attention branch: h_mid = h_in + merge(attn(rope(q), rope(k), v)) W_o
        G[p + "w_o"] = c["om"].reshape(-1, d).T @ dh.reshape(-1, d)
        do = _g._heads(dh @ P[p + "w_o"].T, n_head)
        dqr, dkr, dv = _g.causal_attention_bwd(do, c["qr"], c["kr"], c["v"], c["p"])
        dq, dk = rope_bwd(dqr, ang), rope_bwd(dkr, ang)
        dqkv = np.concatenate([_g._merge_heads(dq), _g._merge_heads(dk), _g._merge_heads(dv)], axis=-1)
        G[p + "w_qkv"] = c["n1"].reshape(-1, d).T @ dqkv.reshape(-1, 3 * d)
        dn1 = dqkv @ P[p + "w_qkv"].T
        dx1, G[p + "attn_norm_g"] = rmsnorm_bwd(dn1, c["h_in"], P[p + "attn_norm_g"], c["r1"])
        dh = dh + dx1
    # embedding: h0 = wte[x]
    G["wte"] = np.zeros_like(P["wte"])
    np.add.at(G["wte"], x.reshape(-1), dh.reshape(-1, d))
    return G


def step(params: Dict[str, np.ndarray], tokens: np.ndarray, n_layer: int, n_head: int,
         lr: float = 3e-4, beta1: float = 0.9, beta2: float = 0.999, eps: float = 1e-8,
         wd: float = 0.1, t: int = 1, norm_eps: float = 1e-5, state=None, optimizer: str = "adamw"):
    """One training step: forward, loss, backward, then AdamW (or SGD) on
    every parameter (L7), as ``oracle.gpt2.step``.

    tokens: int [B, T+1] window; inputs are tokens[:, :-1], labels tokens[:, 1:].
    Returns (loss, grads, new_params, new_state)."""
    if optimizer not in ("adamw", "sgd"):
        raise ValueError(f"unknown optimizer {optimizer!r}")
    tok = np.asarray(tokens, np.int64)
    x, y = tok[:, :-1], tok[:, 1:]
    loss, cache = forward(params, x, y, n_layer, n_head, norm_eps)
    grads = backward(cache, n_layer, n_head)
    new_p, new_s = {}, {}
    for name, p in params.items():
        p64 = np.asarray(p, np.float64)
        if optimizer == "sgd":
            new_p[name] = _g.sgd(p64, grads[name], lr)
            if state and name in state:
                new_s[name] = state[name]
            continue
        m, v = (state or {}).get(name, (np.zeros_like(p64), np.zeros_like(p64)))
        new_p[name], mm, vv = _g.adamw(p64, grads[name], m, v, t, lr, beta1, beta2, eps, wd)
        new_s[name] = (mm, vv)
    return loss, grads, new_p, new_s


def shapes(n_layer: int, vocab: int, d: int, inner: int) -> Dict[str, Tuple[int, ...]]:
    """Dense shape of every parameter, in param_names order."""
    out = {"wte": (vocab, d)}
    for l in range(n_layer):
        p = f"h{l}."
        out.update({p + "attn_norm_g": (d,), p + "w_qkv": (d, 3 * d), p + "w_o": (d, d),
                    p + "mlp_norm_g": (d,), p + "w_gate": (d, inner), p + "w_up": (d, inner),
                    p + "w_down": (inner, d)})
    out.update({"norm_f_g": (d,), "w_head": (vocab, d)})
    return out
