"""Pins of the fp64 oracle to things other than itself.

Each test fixes a property that the mathematics (or an independent
library routine) decides, chosen so that a plausible slip in the oracle --
a dropped term, a wrong sign or index, a transposed operand -- fails at
least one of them:

  * central finite differences of the whole loss in every parameter
    (catches any wrong backward term);
  * softmax rows sum to one and are causal; LayerNorm output statistics;
  * cross-entropy of all-equal logits is ln(V), with dz = (1/V - onehot)/N;
  * attention with zero query/key projections averages the causal prefix;
  * a model whose blocks are all zero reduces to LN_f(wte[x] + wpe) wte^T;
  * the first AdamW step has the closed form p(1 - lr wd) - lr g/(|g| + eps).
"""
import math

import numpy as np
import pytest

import synth
from oracle import gpt2 as og

TINY = synth.GPT2Shape(n_layer=2, vocab=11, n_embd=8, n_head=2, n_inner=16, seq=5, batch=2)


def _rich_params(shape, seed=3):
    """Parameters with non-trivial biases and LayerNorm gains so that every
    gradient term is exercised (std 0.3 instead of 0.02)."""
    rng = np.random.default_rng(seed)
    out = {}
    for name, shp, kind in synth.param_specs(shape):
        base = 1.0 if kind == "ones" else 0.0
        out[name] = base + rng.standard_normal(shp) * 0.3
    return out


def _tokens(shape, seed=4):
    rng = np.random.default_rng(seed)
    return rng.integers(0, shape.vocab, size=(shape.batch, shape.seq + 1))


def _loss(params, tok, shape):
    return og.forward(params, tok[:, :-1], tok[:, 1:], shape.n_layer, shape.n_head)[0]


def test_finite_difference_every_parameter():
    params = _rich_params(TINY)
    tok = _tokens(TINY)
    loss, cache = og.forward(params, tok[:, :-1], tok[:, 1:], TINY.n_layer, TINY.n_head)
    grads = og.backward(cache, TINY.n_layer, TINY.n_head)
    assert set(grads) == set(params)
    rng = np.random.default_rng(5)
    h = 1e-6
    for name, p in params.items():
        assert grads[name].shape == p.shape, name
        u = rng.standard_normal(p.shape)
        u /= np.linalg.norm(u)
        pp = dict(params); pp[name] = p + h * u
        pm = dict(params); pm[name] = p - h * u
        fd = (_loss(pp, tok, TINY) - _loss(pm, tok, TINY)) / (2 * h)
        an = float((grads[name] * u).sum())
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)) + 1e-9, (name, fd, an)
    # twenty single entries
    names = list(params)
    for _ in range(20):
        name = names[rng.integers(len(names))]
        idx = tuple(rng.integers(s) for s in params[name].shape)
        e = np.zeros_like(params[name]); e[idx] = 1.0
        pp = dict(params); pp[name] = params[name] + h * e
        pm = dict(params); pm[name] = params[name] - h * e
        fd = (_loss(pp, tok, TINY) - _loss(pm, tok, TINY)) / (2 * h)
        an = float(grads[name][idx])
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)) + 1e-9, (name, idx, fd, an)


def test_softmax_rows_and_causality():
    rng = np.random.default_rng(0)
    q, k, v = (rng.standard_normal((3, 7, 4)) for _ in range(3))
    o, p = og.causal_attention_fwd(q, k, v)
    assert np.abs(p.sum(axis=-1) - 1.0).max() <= 1e-14
    assert np.all(p[:, np.triu_indices(7, 1)[0], np.triu_indices(7, 1)[1]] == 0.0)
    assert np.allclose(p[:, 0, :], np.eye(7)[0], atol=1e-14)
    # first output row is exactly v_0
    assert np.abs(o[:, 0, :] - v[:, 0, :]).max() <= 1e-14
    s = rng.standard_normal((5, 9)) * 10
    assert np.abs(og.softmax(s).sum(-1) - 1).max() <= 1e-14
    assert np.abs(og.logsumexp(s) - np.log(np.exp(s).sum(-1))).max() <= 1e-12


def test_row_losses_depend_on_the_prefix_only():
    """Causal attention: the loss at position t is fixed by tokens 0..t, so a
    window cut after t reproduces it, and changing a later token does not
    move it; the per-token losses average to the loss."""
    params = _rich_params(TINY)
    rng = np.random.default_rng(5)
    tok = rng.integers(0, TINY.vocab, size=(TINY.batch, TINY.seq + 1))
    x, y = tok[:, :-1], tok[:, 1:]
    full = og.row_losses(params, x, y, TINY.n_layer, TINY.n_head)
    loss, _ = og.forward(params, x, y, TINY.n_layer, TINY.n_head)
    assert abs(full.mean() - loss) <= 1e-13
    for p in range(1, TINY.seq):
        pre = og.row_losses(params, x[:, :p], y[:, :p], TINY.n_layer, TINY.n_head)
        assert np.abs(pre - full[:, :p]).max() <= 1e-13
    x2 = x.copy()
    x2[:, -1] = (x2[:, -1] + 1) % TINY.vocab
    moved = og.row_losses(params, x2, y, TINY.n_layer, TINY.n_head)
    assert np.abs(moved[:, :-1] - full[:, :-1]).max() <= 1e-13
    assert np.abs(moved[:, -1] - full[:, -1]).max() > 1e-6


def test_lr_schedule_ends_and_constant_case():
    """The README's warm-up flags: iteration 1 uses start_lr, iteration
    full_lr_iter and later the full lr; full_lr_iter = 1 keeps it constant."""
    assert og.lr_at(1, 3e-4, 0.0, 10) == 0.0
    assert og.lr_at(10, 3e-4, 0.0, 10) == 3e-4
    assert og.lr_at(57, 3e-4, 0.0, 10) == 3e-4
    assert all(og.lr_at(t, 3e-4, 1e-5, 1) == 3e-4 for t in range(1, 5))
    ramp = [og.lr_at(t, 1.0, 0.1, 4) for t in range(1, 5)]
    assert np.allclose(np.diff(ramp), 0.3) and ramp[0] == 0.1 and ramp[-1] == 1.0


def test_accumulated_minibatch_gradients_equal_the_batch_gradient():
    """Mean loss over a batch = average of the minibatch mean losses (equal
    sizes), so the batch gradient is the average of minibatch gradients --
    what accumulating over minibatches must reproduce."""
    params = _rich_params(TINY)
    rng = np.random.default_rng(11)
    tok = rng.integers(0, TINY.vocab, size=(4, TINY.seq + 1))
    x, y = tok[:, :-1], tok[:, 1:]
    loss, cache = og.forward(params, x, y, TINY.n_layer, TINY.n_head)
    grads = og.backward(cache, TINY.n_layer, TINY.n_head)
    parts = []
    for i in range(2):
        li, ci = og.forward(params, x[2 * i:2 * i + 2], y[2 * i:2 * i + 2], TINY.n_layer, TINY.n_head)
        parts.append((li, og.backward(ci, TINY.n_layer, TINY.n_head)))
    assert abs(loss - (parts[0][0] + parts[1][0]) / 2) <= 1e-13
    for name, g in grads.items():
        assert np.abs(g - (parts[0][1][name] + parts[1][1][name]) / 2).max() <= 1e-13 * max(1.0, np.abs(g).max())


def test_layernorm_statistics():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((6, 33)) * 3 + 2
    y, (mean, rstd) = og.layernorm_fwd(x, np.ones(33), np.zeros(33), 1e-5)
    var = x.var(axis=-1)
    assert np.abs(y.mean(-1)).max() <= 1e-12
    assert np.abs(y.var(-1) - var / (var + 1e-5)).max() <= 1e-12
    assert np.abs(mean - x.mean(-1)).max() <= 1e-12
    assert np.abs(rstd - 1 / np.sqrt(var + 1e-5)).max() <= 1e-12
    # affine part: y = xhat * g + b
    g, b = rng.standard_normal(33), rng.standard_normal(33)
    y2, _ = og.layernorm_fwd(x, g, b, 1e-5)
    assert np.abs(y2 - (y * g + b)).max() <= 1e-12


@pytest.mark.parametrize("vocab", [256, 11])
def test_cross_entropy_uniform_logits(vocab):
    n = 7
    y = np.arange(n) % vocab
    loss, dz, lse = og.cross_entropy(np.full((n, vocab), 0.37), y)
    assert abs(loss - math.log(vocab)) <= 1e-14
    onehot = np.eye(vocab)[y]
    assert np.abs(dz - (1.0 / vocab - onehot) / n).max() <= 1e-15


def test_cross_entropy_through_model_with_zero_wte():
    shape = synth.GPT2Shape(2, 256, 16, 2, 32, 6, 2)
    params = _rich_params(shape)
    params["wte"] = np.zeros_like(params["wte"])
    tok = _tokens(shape)
    loss, cache = og.forward(params, tok[:, :-1], tok[:, 1:], shape.n_layer, shape.n_head)
    assert abs(loss - math.log(256)) <= 1e-14
    assert abs(math.log(256) - 5.545177444479562) <= 1e-15
    assert abs(math.log(50257) - 10.82490511970208) <= 1e-14


def test_attention_uniform_when_qk_projections_zero():
    shape = synth.GPT2Shape(1, 13, 8, 2, 16, 6, 2)
    params = _rich_params(shape)
    d = shape.n_embd
    params["h0.w_qkv"][:, :2 * d] = 0.0
    params["h0.b_qkv"][:2 * d] = 0.0
    tok = _tokens(shape)
    _, cache = og.forward(params, tok[:, :-1], tok[:, 1:], 1, shape.n_head)
    c = cache["blocks"][0]
    v = c["v"]
    cummean = np.cumsum(v, axis=2) / np.arange(1, shape.seq + 1)[None, None, :, None]
    assert np.abs(c["o"] - cummean).max() <= 1e-13


def test_zero_blocks_reduce_to_embedding_head():
    import torch
    shape = synth.GPT2Shape(3, 17, 8, 2, 16, 5, 2)
    params = _rich_params(shape)
    for name in params:
        if name.startswith("h") and (".w_" in name or ".b_" in name):
            params[name] = np.zeros_like(params[name])
    tok = _tokens(shape)
    x = tok[:, :-1]
    loss, cache = og.forward(params, x, tok[:, 1:], shape.n_layer, shape.n_head)
    h0 = torch.tensor(params["wte"][x] + params["wpe"][None, :shape.seq])
    nf = torch.nn.functional.layer_norm(h0, (shape.n_embd,), torch.tensor(params["lnf_g"]),
                                        torch.tensor(params["lnf_b"]), 1e-5)
    z = (nf.reshape(-1, shape.n_embd) @ torch.tensor(params["wte"]).T).numpy()
    assert np.abs(cache["z"] - z).max() <= 1e-13


def test_adamw_first_step_closed_form():
    rng = np.random.default_rng(2)
    p = rng.standard_normal(1000)
    g = rng.standard_normal(1000) * np.logspace(-6, 1, 1000)
    lr, wd, eps = 3e-4, 0.1, 1e-8
    p1, m1, v1 = og.adamw(p, g, np.zeros_like(p), np.zeros_like(p), 1, lr, 0.9, 0.999, eps, wd)
    expect = p * (1 - lr * wd) - lr * g / (np.abs(g) + eps)
    assert np.abs(p1 - expect).max() <= 1e-15
    assert np.abs(m1 - 0.1 * g).max() <= 1e-15
    assert np.abs(v1 - 0.001 * g * g).max() <= 1e-15 * np.abs(g * g).max()


def test_step_updates_every_parameter():
    params = _rich_params(TINY)
    tok = _tokens(TINY)
    loss, grads, newp, state = og.step(params, tok, TINY.n_layer, TINY.n_head)
    for name in params:
        assert newp[name].shape == params[name].shape
        m, v = state[name]
        assert np.abs(m - 0.1 * grads[name]).max() <= 1e-15
