"""Pins of the LLaMA-style fp64 oracle (oracle/llama.py) to things other
than itself:

  * RMSNorm against torch.nn.functional.rms_norm and its autograd (fp64);
  * SwiGLU against torch's silu and autograd;
  * the rotary embedding against closed forms: the identity at position 0,
    a plain 2-D rotation by t when hd = 2, preserved norms, scores that
    depend on the positions' difference only, and a backward that is the
    forward's adjoint;
  * central finite differences of the whole loss in every parameter (any
    wrong backward term fails);
  * Hugging Face's LlamaForCausalLM in float64 (block form, RMSNorm, the
    rotary pairing and direction, SwiGLU, untied head): logits, loss and
    every parameter gradient.

Library routines are witnesses here only; the oracle uses none of them."""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import synth
from oracle import llama as ol

TINY = synth.GPT2Shape(n_layer=2, vocab=11, n_embd=8, n_head=2, n_inner=12, seq=5, batch=2)


def _rich_params(shape, seed=3, std=0.3):
    """Non-trivial gains and weights (std 0.3) so every gradient term matters."""
    rng = np.random.default_rng(seed)
    out = {}
    for name, shp, kind in synth.llama_param_specs(shape):
        base = 1.0 if kind == "ones" else 0.0
        out[name] = base + rng.standard_normal(shp) * std
    return out


def _tokens(shape, seed=4):
    rng = np.random.default_rng(seed)
    return rng.integers(0, shape.vocab, size=(shape.batch, shape.seq + 1))


def test_param_names_match_specs():
    names = [n for n, _, _ in synth.llama_param_specs(TINY)]
    assert names == ol.param_names(TINY.n_layer)
    shp = ol.shapes(TINY.n_layer, TINY.vocab, TINY.n_embd, TINY.n_inner)
    assert {n: s for n, s, _ in synth.llama_param_specs(TINY)} == shp


def test_rmsnorm_matches_torch():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((3, 7, 40)) * 2
    g = rng.standard_normal(40)
    y, rstd = ol.rmsnorm_fwd(x, g, 1e-5)
    xt = torch.tensor(x, requires_grad=True)
    gt = torch.tensor(g, requires_grad=True)
    yt = F.rms_norm(xt, (40,), gt, 1e-5)
    assert np.abs(y - yt.detach().numpy()).max() <= 1e-12
    dy = rng.standard_normal(y.shape)
    yt.backward(torch.tensor(dy))
    dx, dg = ol.rmsnorm_bwd(dy, x, g, rstd)
    assert np.abs(dx - xt.grad.numpy()).max() <= 1e-11
    assert np.abs(dg - gt.grad.numpy()).max() <= 1e-11
    # output rows have mean square g^2-weighted one: with g = 1, mean(y^2) = ms / (ms + eps)
    y1, _ = ol.rmsnorm_fwd(x, np.ones(40), 1e-5)
    ms = (x * x).mean(-1)
    assert np.abs((y1 * y1).mean(-1) - ms / (ms + 1e-5)).max() <= 1e-12


def test_swiglu_matches_torch():
    rng = np.random.default_rng(1)
    a = rng.standard_normal(500) * 5
    b = rng.standard_normal(500)
    at = torch.tensor(a, requires_grad=True)
    bt = torch.tensor(b, requires_grad=True)
    ht = F.silu(at) * bt
    assert np.abs(ol.swiglu_fwd(a, b) - ht.detach().numpy()).max() <= 1e-13
    dh = rng.standard_normal(500)
    ht.backward(torch.tensor(dh))
    da, db = ol.swiglu_bwd(dh, a, b)
    assert np.abs(da - at.grad.numpy()).max() <= 1e-12
    assert np.abs(db - bt.grad.numpy()).max() <= 1e-12


def test_rope_closed_forms():
    rng = np.random.default_rng(2)
    hd, T = 16, 9
    ang = ol.rope_angles(T, hd)
    # position 0 is the identity; the first pair turns by t radians (theta_0 = 1),
    # the last by t * base^(-(hd-2)/hd)
    assert np.all(ang[0] == 0) and np.allclose(ang[:, 0], np.arange(T))
    assert math.isclose(ang[1, hd // 2 - 1], 10000.0 ** (-(hd - 2) / hd), rel_tol=1e-15)
    x = rng.standard_normal((3, T, hd))
    y = ol.rope_fwd(x, ang)
    assert np.array_equal(y[:, 0], x[:, 0])
    # hd = 2: a plain rotation of (x0, x1) by t
    x2 = rng.standard_normal((T, 2))
    y2 = ol.rope_fwd(x2, ol.rope_angles(T, 2))
    t = np.arange(T)
    assert np.allclose(y2[:, 0], x2[:, 0] * np.cos(t) - x2[:, 1] * np.sin(t), atol=1e-15)
    assert np.allclose(y2[:, 1], x2[:, 1] * np.cos(t) + x2[:, 0] * np.sin(t), atol=1e-15)
    # rotations keep norms
    assert np.allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-14)
    # a score depends on the positions' difference only
    q, k = rng.standard_normal(hd), rng.standard_normal(hd)
    qs = ol.rope_fwd(np.tile(q, (T, 1)), ang)
    ks = ol.rope_fwd(np.tile(k, (T, 1)), ang)
    for m, n, s in [(5, 2, 2), (8, 8, 6), (4, 1, 1), (3, 7, 3)]:
        assert math.isclose(qs[m] @ ks[n], qs[m - s] @ ks[n - s], rel_tol=1e-12, abs_tol=1e-12)
    assert not math.isclose(qs[5] @ ks[2], qs[5] @ ks[3], rel_tol=1e-6)
    # the backward is the adjoint of the forward
    dy = rng.standard_normal(y.shape)
    assert math.isclose(float((y * dy).sum()), float((x * ol.rope_bwd(dy, ang)).sum()), rel_tol=1e-13)


def _loss(params, tok, shape):
    return ol.forward(params, tok[:, :-1], tok[:, 1:], shape.n_layer, shape.n_head)[0]


def test_finite_difference_every_parameter():
    params = _rich_params(TINY)
    tok = _tokens(TINY)
    loss, cache = ol.forward(params, tok[:, :-1], tok[:, 1:], TINY.n_layer, TINY.n_head)
    grads = ol.backward(cache, TINY.n_layer, TINY.n_head)
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


def test_llama_matches_transformers_fp64():
    """Hugging Face's LLaMA in float64. Its RMSNorm normalises in float32 and
    its rotary tables are float32, so agreement is at float32's level
    (relative 2e-5 of each tensor's largest entry), far below what a wrong
    sign, pairing or missing term would give."""
    tr = pytest.importorskip("transformers")
    shape = synth.GPT2Shape(2, 37, 32, 4, 48, 9, 3)
    params = _rich_params(shape, seed=7, std=0.2)
    rng = np.random.default_rng(8)
    tok = rng.integers(0, shape.vocab, size=(shape.batch, shape.seq + 1))
    x, y = tok[:, :-1], tok[:, 1:]
    loss, cache = ol.forward(params, x, y, shape.n_layer, shape.n_head)
    grads = ol.backward(cache, shape.n_layer, shape.n_head)

    d = shape.n_embd
    cfg = tr.LlamaConfig(vocab_size=shape.vocab, hidden_size=d, intermediate_size=shape.n_inner,
                         num_hidden_layers=shape.n_layer, num_attention_heads=shape.n_head,
                         num_key_value_heads=shape.n_head, max_position_embeddings=shape.seq,
                         rms_norm_eps=1e-5, rope_theta=10000.0, attention_bias=False, mlp_bias=False,
                         tie_word_embeddings=False, hidden_act="silu", attn_implementation="eager")
    torch.manual_seed(0)
    model = tr.LlamaForCausalLM(cfg).double().eval()
    T = lambda a: torch.tensor(np.ascontiguousarray(a), dtype=torch.float64)  # noqa: E731
    names = {"model.embed_tokens.weight": ("wte", False), "model.norm.weight": ("norm_f_g", False),
             "lm_head.weight": ("w_head", False)}
    for l in range(shape.n_layer):
        p, hp = f"h{l}.", f"model.layers.{l}."
        names[hp + "input_layernorm.weight"] = (p + "attn_norm_g", False)
        names[hp + "post_attention_layernorm.weight"] = (p + "mlp_norm_g", False)
        names[hp + "self_attn.o_proj.weight"] = (p + "w_o", True)
        names[hp + "mlp.gate_proj.weight"] = (p + "w_gate", True)
        names[hp + "mlp.up_proj.weight"] = (p + "w_up", True)
        names[hp + "mlp.down_proj.weight"] = (p + "w_down", True)
    with torch.no_grad():
        sd = dict(model.named_parameters())
        assert set(sd) == set(names) | {f"model.layers.{l}.self_attn.{w}_proj.weight"
                                        for l in range(shape.n_layer) for w in "qkv"}
        for hf, (ours, tr_) in names.items():
            sd[hf].copy_(T(params[ours].T if tr_ else params[ours]))
        for l in range(shape.n_layer):
            w = params[f"h{l}.w_qkv"]
            for i, nm in enumerate("qkv"):
                sd[f"model.layers.{l}.self_attn.{nm}_proj.weight"].copy_(T(w[:, i * d:(i + 1) * d].T))
    logits = model(input_ids=torch.tensor(x)).logits
    z = logits.detach().numpy().reshape(-1, shape.vocab)
    assert np.abs(z - cache["z"]).max() <= 2e-5 * np.abs(cache["z"]).max()
    lt = F.cross_entropy(logits.reshape(-1, shape.vocab), torch.tensor(y).reshape(-1))
    assert abs(lt.item() - loss) <= 2e-5 * abs(loss)
    lt.backward()
    sd = dict(model.named_parameters())
    for hf, (ours, tr_) in names.items():
        ref = sd[hf].grad.numpy()
        ref = ref.T if tr_ else ref
        assert np.abs(grads[ours] - ref).max() <= 2e-5 * np.abs(ref).max(), hf
    for l in range(shape.n_layer):
        ref = np.concatenate([sd[f"model.layers.{l}.self_attn.{nm}_proj.weight"].grad.numpy().T for nm in "qkv"], 1)
        assert np.abs(grads[f"h{l}.w_qkv"] - ref).max() <= 2e-5 * np.abs(ref).max(), l


def test_step_updates_every_parameter_and_lowers_the_loss():
    params = _rich_params(TINY, std=0.1)
    tok = _tokens(TINY)
    loss, grads, new_p, state = ol.step(params, tok, TINY.n_layer, TINY.n_head, lr=1e-2, wd=0.0)
    for name in params:
        assert not np.array_equal(new_p[name], params[name]), name
        assert name in state
    assert _loss(new_p, tok, TINY) < loss
    _, _, sgd_p, _ = ol.step(params, tok, TINY.n_layer, TINY.n_head, lr=1e-2, optimizer="sgd")
    for name in params:
        assert np.allclose(sgd_p[name], params[name] - 1e-2 * grads[name], rtol=0, atol=1e-15)
