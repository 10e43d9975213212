"""Untiled float64 GPT2 forward, backward and AdamW (the oracle).

TEST INFRASTRUCTURE: only tests/, the smoke check and the benchmark's
CPU-baseline leg may use this module.

What it follows. The pith.science review of NNTile ("What carries the
argument") lists the layers every training step is made of: embedding,
linear, layer norm, softmax, attention, cross-entropy and the Adam/SGD
update, each with a forward and a backward. The NNTile README ("Minimal
working GPT example") fixes the training example: a GPT2 model, fused AdamW
with eps 1e-8 and weight decay 0.1, lr 3e-4, and the loss reported as the
mean over all tokens of the batch. The pages define none of the layers
themselves; they cite the defining papers by title on the arXiv index page
("Builds on": Attention Is All You Need; Layer Normalization; On Layer
Normalization in the Transformer Architecture; Decoupled Weight Decay
Regularization). Readings taken where the pages are silent:

  R1 GPT2 block = pre-LN: h += Attn(LN1(h)); h += MLP(LN2(h)); final LN.
  R2 MLP activation: GELU, tanh approximation; inner width from the config.
  R3 LayerNorm: biased variance over the embedding axis, eps 1e-5 inside
     the square root.
  R4 no dropout.
  R5 biases on every linear layer, none on the LM head; head tied to wte.
  R6 attention: scale 1/sqrt(head_dim), causal mask, no padding mask.
  R7 loss: mean over the B*T next-token targets.
  R8 AdamW: beta1 0.9, beta2 0.999, decoupled decay p *= (1 - lr*wd)
     applied before the moment step, bias correction on, eps outside the
     square root, one parameter group (decay on every parameter).
  R9 SGD (the review's Adam/SGD update; the README's --optimizer flag
     picks the optimizer): the plain step p - lr*g, no momentum and no
     weight decay (the README ties weight decay to AdamW); the same lr
     schedule.

The arithmetic below is the plain definition of each layer; the only
library primitive used is numpy's matmul (and exp/log/tanh/sqrt).

Parity unpinned: lr_at between its ends. The README fixes the learning
rate of iteration 1 (start_lr) and of iteration full_lr_iter onwards (the
full lr); the linear ramp in between is a reading that no passage or
closed form fixes, so its interior values are checked only against that
reading. The ends and the constant schedule are pinned.
"""
from __future__ import annotations

import math
from typing import Dict, Tuple

import numpy as np

GELU_C = math.sqrt(2.0 / math.pi)
GELU_A = 0.044715


# --------------------------------------------------------------------- layers

def layernorm_fwd(x: np.ndarray, g: np.ndarray, b: np.ndarray, eps: float = 1e-5):
    """y = (x - mean) / sqrt(var + eps) * g + b over the last axis (R3).

    Returns y and (mean, rstd) per row, the statistics the backward needs."""
    mean = x.mean(axis=-1, keepdims=True)
    var = ((x - mean) ** 2).mean(axis=-1, keepdims=True)
    rstd = 1.0 / np.sqrt(var + eps)
    xhat = (x - mean) * rstd
    return xhat * g + b, (mean[..., 0], rstd[..., 0])


def layernorm_bwd(dy: np.ndarray, x: np.ndarray, g: np.ndarray, mean: np.ndarray,
                  rstd: np.ndarray):
    """Gradient of layernorm_fwd: returns dx, dg, db.

    With xhat = (x - mean) * rstd and dxhat = dy * g:
      dx = rstd * (dxhat - mean(dxhat) - xhat * mean(dxhat * xhat))
      dg = sum over rows of dy * xhat, db = sum over rows of dy."""
    xhat = (x - mean[..., None]) * rstd[..., None]
    dxhat = dy * g
    m1 = dxhat.mean(axis=-1, keepdims=True)
    m2 = (dxhat * xhat).mean(axis=-1, keepdims=True)
    dx = rstd[..., None] * (dxhat - m1 - xhat * m2)
    axes = tuple(range(dy.ndim - 1))
    return dx, (dy * xhat).sum(axis=axes), dy.sum(axis=axes)


def gelu(u: np.ndarray) -> np.ndarray:
    """GELU, tanh approximation (R2)."""
    return 0.5 * u * (1.0 + np.tanh(GELU_C * (u + GELU_A * u ** 3)))


def gelu_grad(u: np.ndarray) -> np.ndarray:
    """d gelu / du, differentiated by hand from ``gelu``."""
    a = GELU_C * (u + GELU_A * u ** 3)
    t = np.tanh(a)
    return 0.5 * (1.0 + t) + 0.5 * u * (1.0 - t * t) * GELU_C * (1.0 + 3.0 * GELU_A * u * u)


def softmax(s: np.ndarray, axis: int = -1) -> np.ndarray:
    """Row softmax; rows that are entirely -inf are not expected."""
    m = s.max(axis=axis, keepdims=True)
    e = np.exp(s - m)
    return e / e.sum(axis=axis, keepdims=True)


def logsumexp(s: np.ndarray, axis: int = -1) -> np.ndarray:
    m = s.max(axis=axis, keepdims=True)
    return (m + np.log(np.exp(s - m).sum(axis=axis, keepdims=True)))[..., 0]


def causal_attention_fwd(q: np.ndarray, k: np.ndarray, v: np.ndarray):
    """Scaled dot-product attention with a causal mask (R6).

    q, k, v: [..., T, hd]. Returns O [..., T, hd] and P [..., T, T]."""
    t, hd = q.shape[-2], q.shape[-1]
    s = (q @ np.swapaxes(k, -1, -2)) / math.sqrt(hd)
    mask = np.triu(np.ones((t, t), dtype=bool), k=1)
    s = np.where(mask, -np.inf, s)
    p = softmax(s, axis=-1)
    return p @ v, p


def causal_attention_bwd(dO: np.ndarray, q: np.ndarray, k: np.ndarray, v: np.ndarray,
                         p: np.ndarray):
    """Gradient of causal_attention_fwd through the softmax Jacobian.

    dV = P^T dO; dP = dO V^T; dS = P * (dP - sum_j P dP); dQ = dS K / sqrt(hd);
    dK = dS^T Q / sqrt(hd). Masked entries have P = 0, so dS = 0 there."""
    hd = q.shape[-1]
    dv = np.swapaxes(p, -1, -2) @ dO
    dp = dO @ np.swapaxes(v, -1, -2)
    ds = p * (dp - (p * dp).sum(axis=-1, keepdims=True))
    scale = 1.0 / math.sqrt(hd)
    dq = (ds @ k) * scale
    dk = (np.swapaxes(ds, -1, -2) @ q) * scale
    return dq, dk, dv


def cross_entropy(z: np.ndarray, y: np.ndarray):
    """Mean next-token cross-entropy over all rows (R7).

    z: [N, V] logits, y: [N] labels. Returns (loss, dz, lse)."""
    n = z.shape[0]
    lse = logsumexp(z, axis=-1)
    loss = float(np.mean(lse - z[np.arange(n), y]))
    dz = np.exp(z - lse[:, None])
    dz[np.arange(n), y] -= 1.0
    return loss, dz / n, lse


def adamw(p, g, m, v, t: int, lr: float, beta1: float, beta2: float, eps: float, wd: float):
    """One decoupled-weight-decay Adam step (R8). Returns new (p, m, v)."""
    p = p * (1.0 - lr * wd)
    m = beta1 * m + (1.0 - beta1) * g
    v = beta2 * v + (1.0 - beta2) * g * g
    mhat = m / (1.0 - beta1 ** t)
    vhat = v / (1.0 - beta2 ** t)
    return p - lr * mhat / (np.sqrt(vhat) + eps), m, v


def sgd(p, g, lr: float):
    """One plain stochastic-gradient step (R9)."""
    return p - lr * g


# ---------------------------------------------------------------------- model

def _heads(x: np.ndarray, n_head: int) -> np.ndarray:
    b, t, d = x.shape
    return x.reshape(b, t, n_head, d // n_head).transpose(0, 2, 1, 3)


def _merge_heads(x: np.ndarray) -> np.ndarray:
    b, h, t, hd = x.shape
    return x.transpose(0, 2, 1, 3).reshape(b, t, h * hd)


def forward(params: Dict[str, np.ndarray], x: np.ndarray, y: np.ndarray, n_layer: int,
            n_head: int, ln_eps: float = 1e-5):
    """GPT2 forward + loss. params are promoted to float64.

    Returns (loss, cache) where cache holds every activation the backward
    needs, plus the logits and the per-row logsumexp."""
    P = {k: np.asarray(v, np.float64) for k, v in params.items()}
    B, T = x.shape
    d = P["wte"].shape[1]
    cache = {"x": x, "y": y, "P": P, "blocks": []}
    h = P["wte"][x] + P["wpe"][np.arange(T)][None]
    cache["h0"] = h
    for l in range(n_layer):
        p = f"h{l}."
        c = {"h_in": h}
        n1, (mu1, r1) = layernorm_fwd(h, P[p + "ln1_g"], P[p + "ln1_b"], ln_eps)
        qkv = n1 @ P[p + "w_qkv"] + P[p + "b_qkv"]
        q, k, v = (_heads(qkv[..., i * d:(i + 1) * d], n_head) for i in range(3))
        o, pr = causal_attention_fwd(q, k, v)
        om = _merge_heads(o)
        h_mid = h + om @ P[p + "w_o"] + P[p + "b_o"]
        n2, (mu2, r2) = layernorm_fwd(h_mid, P[p + "ln2_g"], P[p + "ln2_b"], ln_eps)
        u = n2 @ P[p + "w_fc"] + P[p + "b_fc"]
        gu = gelu(u)
        h = h_mid + gu @ P[p + "w_p"] + P[p + "b_p"]
        c.update(n1=n1, ln1=(mu1, r1), q=q, k=k, v=v, o=o, p=pr, om=om, h_mid=h_mid,
                 n2=n2, ln2=(mu2, r2), u=u, g=gu)
        cache["blocks"].append(c)
    cache["h_last"] = h
    nf, (muf, rf) = layernorm_fwd(h, P["lnf_g"], P["lnf_b"], ln_eps)
    z = nf.reshape(B * T, d) @ P["wte"].T
    loss, dz, lse = cross_entropy(z, y.reshape(-1))
    cache.update(nf=nf, lnf=(muf, rf), z=z, dz=dz, lse=lse, loss=loss)
    return loss, cache


def row_losses(params: Dict[str, np.ndarray], x: np.ndarray, y: np.ndarray, n_layer: int, n_head: int,
               ln_eps: float = 1e-5) -> np.ndarray:
    """Per-token next-token losses [B, T]: logsumexp of the row's logits
    minus its label's logit, i.e. the terms whose mean is the loss (R7)."""
    _, cache = forward(params, x, y, n_layer, n_head, ln_eps)
    z, lse = cache["z"], cache["lse"]
    return (lse - z[np.arange(z.shape[0]), y.reshape(-1)]).reshape(x.shape)


def backward(cache, n_layer: int, n_head: int) -> Dict[str, np.ndarray]:
    """Analytic gradients of the mean loss w.r.t. every parameter (float64)."""
    P, x = cache["P"], cache["x"]
    B, T = x.shape
    d = P["wte"].shape[1]
    G: Dict[str, np.ndarray] = {}
    dz = cache["dz"]
    nf = cache["nf"].reshape(B * T, d)
    G["wte"] = dz.T @ nf                                  # tied head part
    dnf = (dz @ P["wte"]).reshape(B, T, d)
    dh, G["lnf_g"], G["lnf_b"] = layernorm_bwd(dnf, cache["h_last"], P["lnf_g"], *cache["lnf"])
    for l in reversed(range(n_layer)):
        p = f"h{l}."
        c = cache["blocks"][l]
        # MLP branch: h = h_mid + gelu(u) W_p + b_p
        G[p + "w_p"] = c["g"].reshape(-1, c["g"].shape[-1]).T @ dh.reshape(-1, d)
        G[p + "b_p"] = dh.sum(axis=(0, 1))
        dg = dh @ P[p + "w_p"].T
        du = dg * gelu_grad(c["u"])
        G[p + "w_fc"] = c["n2"].reshape(-1, d).T @ du.reshape(-1, du.shape[-1])
        G[p + "b_fc"] = du.sum(axis=(0, 1))
        dn2 = du @ P[p + "w_fc"].T
        dx2, G[p + "ln2_g"], G[p + "ln2_b"] = layernorm_bwd(dn2, c["h_mid"], P[p + "ln2_g"], *c["ln2"])
        dh = dh + dx2
        # attention branch: h_mid = h_in + merge(O) W_o + b_o
        G[p + "w_o"] = c["om"].reshape(-1, d).T @ dh.reshape(-1, d)
        G[p + "b_o"] = dh.sum(axis=(0, 1))
        do = _heads(dh @ P[p + "w_o"].T, n_head)
        dq, dk, dv = causal_attention_bwd(do, c["q"], c["k"], c["v"], c["p"])
        dqkv = np.concatenate([_merge_heads(dq), _merge_heads(dk), _merge_heads(dv)], axis=-1)
        G[p + "w_qkv"] = c["n1"].reshape(-1, d).T @ dqkv.reshape(-1, 3 * d)
        G[p + "b_qkv"] = dqkv.sum(axis=(0, 1))
        dn1 = dqkv @ P[p + "w_qkv"].T
        dx1, G[p + "ln1_g"], G[p + "ln1_b"] = layernorm_bwd(dn1, c["h_in"], P[p + "ln1_g"], *c["ln1"])
        dh = dh + dx1
    # embedding: h0 = wte[x] + wpe[t]
    dwte_emb = np.zeros_like(P["wte"])
    np.add.at(dwte_emb, x.reshape(-1), dh.reshape(-1, d))
    G["wte"] = G["wte"] + dwte_emb
    G["wpe"] = np.zeros_like(P["wpe"])
    G["wpe"][:T] = dh.sum(axis=0)
    return G


def lr_at(t: int, lr: float, start_lr: float, full_lr_iter: int) -> float:
    """Learning rate of AdamW iteration t (counted from 1). The NNTile README
    ("Minimal working GPT example") fixes the ends: the first iteration uses
    start_lr, iteration full_lr_iter and every later one the full lr, and
    full_lr_iter = 1 means the full lr throughout. Reading: linear in t
    between the ends."""
    if full_lr_iter <= 1 or t >= full_lr_iter:
        return lr
    return start_lr + (lr - start_lr) * (t - 1) / (full_lr_iter - 1)


def step(params: Dict[str, np.ndarray], tokens: np.ndarray, n_layer: int, n_head: int,
         lr: float = 3e-4, beta1: float = 0.9, beta2: float = 0.999, eps: float = 1e-8,
         wd: float = 0.1, t: int = 1, ln_eps: float = 1e-5, state=None, optimizer: str = "adamw"):
    """One training step: forward, loss, backward, then AdamW (or SGD, R9)
    on every parameter.

    tokens: int [B, T+1] window; inputs are tokens[:, :-1], labels tokens[:, 1:].
    state: optional dict name -> (m, v); zeros when absent (first step); SGD
    leaves it as given.
    Returns (loss, grads, new_params, new_state)."""
    if optimizer not in ("adamw", "sgd"):
        raise ValueError(f"unknown optimizer {optimizer!r}")
    tok = np.asarray(tokens, np.int64)
    x, y = tok[:, :-1], tok[:, 1:]
    loss, cache = forward(params, x, y, n_layer, n_head, ln_eps)
    grads = backward(cache, n_layer, n_head)
    new_p, new_s = {}, {}
    for name, p in params.items():
        p64 = np.asarray(p, np.float64)
        if optimizer == "sgd":
            new_p[name] = sgd(p64, grads[name], lr)
            if state and name in state:
                new_s[name] = state[name]
            continue
        m, v = (state or {}).get(name, (np.zeros_like(p64), np.zeros_like(p64)))
        new_p[name], mm, vv = adamw(p64, grads[name], m, v, t, lr, beta1, beta2, eps, wd)
        new_s[name] = (mm, vv)
    return loss, grads, new_p, new_s

