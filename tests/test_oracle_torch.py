"""Cross-check of the oracle's conventions against independent fp64 library
routines on the CPU: torch.nn.functional ops, autograd, torch.optim.AdamW,
and Hugging Face's GPT2LMHeadModel (GPT2 block form, tied head, GELU tanh,
LayerNorm eps, attention scale). Library calls are used only here, as
witnesses; the oracle itself uses none of them."""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import synth
from oracle import gpt2 as og


def test_ops_match_torch():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((4, 5, 24))
    g, b = rng.standard_normal(24), rng.standard_normal(24)
    y, (mu, rs) = og.layernorm_fwd(x, g, b, 1e-5)
    xt = torch.tensor(x, requires_grad=True)
    gt = torch.tensor(g, requires_grad=True)
    bt = torch.tensor(b, requires_grad=True)
    yt = F.layer_norm(xt, (24,), gt, bt, 1e-5)
    assert np.abs(y - yt.detach().numpy()).max() <= 1e-12
    dy = rng.standard_normal(y.shape)
    yt.backward(torch.tensor(dy))
    dx, dg, db = og.layernorm_bwd(dy, x, g, mu, rs)
    assert np.abs(dx - xt.grad.numpy()).max() <= 1e-11
    assert np.abs(dg - gt.grad.numpy()).max() <= 1e-11
    assert np.abs(db - bt.grad.numpy()).max() <= 1e-11

    u = rng.standard_normal(1000) * 4
    ut = torch.tensor(u, requires_grad=True)
    gl = F.gelu(ut, approximate="tanh")
    gl.sum().backward()
    assert np.abs(og.gelu(u) - gl.detach().numpy()).max() <= 1e-13
    assert np.abs(og.gelu_grad(u) - ut.grad.numpy()).max() <= 1e-12

    q, k, v = (rng.standard_normal((2, 3, 9, 8)) for _ in range(3))
    o, p = og.causal_attention_fwd(q, k, v)
    qt, kt, vt = (torch.tensor(a, requires_grad=True) for a in (q, k, v))
    ot = F.scaled_dot_product_attention(qt, kt, vt, is_causal=True)
    assert np.abs(o - ot.detach().numpy()).max() <= 1e-12
    do = rng.standard_normal(o.shape)
    ot.backward(torch.tensor(do))
    dq, dk, dv = og.causal_attention_bwd(do, q, k, v, p)
    assert np.abs(dq - qt.grad.numpy()).max() <= 1e-11
    assert np.abs(dk - kt.grad.numpy()).max() <= 1e-11
    assert np.abs(dv - vt.grad.numpy()).max() <= 1e-11

    z = rng.standard_normal((13, 50)) * 3
    yl = rng.integers(0, 50, 13)
    loss, dz, lse = og.cross_entropy(z, yl)
    zt = torch.tensor(z, requires_grad=True)
    lt = F.cross_entropy(zt, torch.tensor(yl), reduction="mean")
    lt.backward()
    assert abs(loss - lt.item()) <= 1e-13
    assert np.abs(dz - zt.grad.numpy()).max() <= 1e-14


def test_adamw_matches_torch_optim_three_steps():
    rng = np.random.default_rng(1)
    p0 = rng.standard_normal(64)
    gs = [rng.standard_normal(64) * 10 ** rng.uniform(-5, 0) for _ in range(3)]
    pt = torch.tensor(p0, requires_grad=True)
    opt = torch.optim.AdamW([pt], lr=3e-4, betas=(0.9, 0.999), eps=1e-8, weight_decay=0.1,
                            foreach=False, fused=False)
    p, m, v = p0.copy(), np.zeros(64), np.zeros(64)
    for t, g in enumerate(gs, start=1):
        pt.grad = torch.tensor(g)
        opt.step()
        p, m, v = og.adamw(p, g, m, v, t, 3e-4, 0.9, 0.999, 1e-8, 0.1)
        assert np.abs(p - pt.detach().numpy()).max() <= 1e-15


def test_sgd_matches_torch_optim_three_steps():
    rng = np.random.default_rng(2)
    p0 = rng.standard_normal(64)
    gs = [rng.standard_normal(64) * 10 ** rng.uniform(-5, 0) for _ in range(3)]
    pt = torch.tensor(p0, requires_grad=True)
    opt = torch.optim.SGD([pt], lr=3e-4, momentum=0.0, weight_decay=0.0, foreach=False)
    p = p0.copy()
    for g in gs:
        pt.grad = torch.tensor(g)
        opt.step()
        p = og.sgd(p, g, 3e-4)
        assert np.abs(p - pt.detach().numpy()).max() <= 1e-15


def test_sgd_step_descends_the_loss():
    # a small enough plain gradient step lowers the loss (first-order
    # decrease lr*|g|^2 dominates the O(lr^2) term)
    shape = synth.WORKLOADS["tiny"].shape
    params = synth.init_params(shape, seed=0)
    tokens = synth.token_stream(shape, seed=1)
    loss0, grads, p1, _ = og.step(params, tokens, shape.n_layer, shape.n_head, lr=1e-2, optimizer="sgd")
    loss1, _ = og.forward(p1, np.asarray(tokens)[:, :-1], np.asarray(tokens)[:, 1:], shape.n_layer, shape.n_head)
    gnorm2 = sum(float(np.sum(g * g)) for g in grads.values())
    assert loss1 < loss0
    assert abs((loss0 - loss1) - 1e-2 * gnorm2) <= 0.05 * 1e-2 * gnorm2


def _hf_model(shape, params):
    from transformers import GPT2Config, GPT2LMHeadModel
    cfg = GPT2Config(vocab_size=shape.vocab, n_positions=shape.seq, n_embd=shape.n_embd,
                     n_layer=shape.n_layer, n_head=shape.n_head, n_inner=shape.n_inner,
                     activation_function="gelu_new", resid_pdrop=0.0, embd_pdrop=0.0,
                     attn_pdrop=0.0, layer_norm_epsilon=1e-5, tie_word_embeddings=True)
    model = GPT2LMHeadModel(cfg).double().eval()
    if hasattr(model.config, "_attn_implementation"):
        model.config._attn_implementation = "eager"
    tr = model.transformer
    sd = {"wte.weight": params["wte"], "wpe.weight": params["wpe"],
          "ln_f.weight": params["lnf_g"], "ln_f.bias": params["lnf_b"]}
    for l in range(shape.n_layer):
        p = f"h{l}."
        sd.update({
            f"h.{l}.ln_1.weight": params[p + "ln1_g"], f"h.{l}.ln_1.bias": params[p + "ln1_b"],
            f"h.{l}.attn.c_attn.weight": params[p + "w_qkv"], f"h.{l}.attn.c_attn.bias": params[p + "b_qkv"],
            f"h.{l}.attn.c_proj.weight": params[p + "w_o"], f"h.{l}.attn.c_proj.bias": params[p + "b_o"],
            f"h.{l}.ln_2.weight": params[p + "ln2_g"], f"h.{l}.ln_2.bias": params[p + "ln2_b"],
            f"h.{l}.mlp.c_fc.weight": params[p + "w_fc"], f"h.{l}.mlp.c_fc.bias": params[p + "b_fc"],
            f"h.{l}.mlp.c_proj.weight": params[p + "w_p"], f"h.{l}.mlp.c_proj.bias": params[p + "b_p"],
        })
    with torch.no_grad():
        own = dict(tr.named_parameters())
        for k, val in sd.items():
            own[k].copy_(torch.tensor(np.asarray(val, np.float64)))
    return model, sd


def test_gpt2_matches_transformers_fp64():
    pytest.importorskip("transformers")
    shape = synth.GPT2Shape(2, 37, 16, 4, 40, 9, 3)
    rng = np.random.default_rng(7)
    params = {}
    for name, shp, kind in synth.param_specs(shape):
        base = 1.0 if kind == "ones" else 0.0
        params[name] = base + rng.standard_normal(shp) * 0.2
    tok = rng.integers(0, shape.vocab, size=(shape.batch, shape.seq + 1))
    x, y = tok[:, :-1], tok[:, 1:]
    loss, cache = og.forward(params, x, y, shape.n_layer, shape.n_head)
    grads = og.backward(cache, shape.n_layer, shape.n_head)

    model, sd = _hf_model(shape, params)
    logits = model(input_ids=torch.tensor(x)).logits
    assert np.abs(logits.detach().numpy().reshape(-1, shape.vocab) - cache["z"]).max() <= 1e-11
    lt = F.cross_entropy(logits.reshape(-1, shape.vocab), torch.tensor(y).reshape(-1))
    assert abs(lt.item() - loss) <= 1e-12
    per_tok = F.cross_entropy(logits.reshape(-1, shape.vocab), torch.tensor(y).reshape(-1), reduction="none")
    rl = og.row_losses(params, x, y, shape.n_layer, shape.n_head)
    assert np.abs(rl - per_tok.detach().numpy().reshape(x.shape)).max() <= 1e-11
    lt.backward()
    own = dict(model.transformer.named_parameters())
    names = {"wte.weight": "wte", "wpe.weight": "wpe", "ln_f.weight": "lnf_g", "ln_f.bias": "lnf_b"}
    for l in range(shape.n_layer):
        for hf, ours in [("ln_1.weight", "ln1_g"), ("ln_1.bias", "ln1_b"),
                         ("attn.c_attn.weight", "w_qkv"), ("attn.c_attn.bias", "b_qkv"),
                         ("attn.c_proj.weight", "w_o"), ("attn.c_proj.bias", "b_o"),
                         ("ln_2.weight", "ln2_g"), ("ln_2.bias", "ln2_b"),
                         ("mlp.c_fc.weight", "w_fc"), ("mlp.c_fc.bias", "b_fc"),
                         ("mlp.c_proj.weight", "w_p"), ("mlp.c_proj.bias", "b_p")]:
            names[f"h.{l}.{hf}"] = f"h{l}.{ours}"
    for hf, ours in names.items():
        ref = own[hf].grad.numpy()
        assert np.abs(grads[ours] - ref).max() <= 1e-10 * max(1.0, np.abs(ref).max()), hf
