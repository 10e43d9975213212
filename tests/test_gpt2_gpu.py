"""End-to-end parity of the tiled GPT2 step (HIP) with the untiled fp64 oracle.

Bar (fp32 path vs fp64 oracle, same seeded inputs):
  * loss: relative error <= 1e-4;
  * every gradient tensor: normwise relative error <= 1e-3 and
    max |g - g_ref| <= 1e-3 * max |g_ref|;
  * AdamW itself: the GPU's updated parameters equal the oracle's AdamW fed
    with the GPU's own fp32 gradients, elementwise within 1e-3 relative with
    an absolute floor of 1e-3 * lr;
  * every updated parameter vs the full oracle step: normwise relative error
    <= 1e-3 over the elements whose update direction the arithmetic decides,
    and |p - p_ref| <= 2 lr (1 + 1e-3) everywhere.
The first decoupled-Adam step moves each weight by about lr * sign(g). Where
the fp64 gradient is below the gradient tolerance (1e-3 * max|g_ref| of its
tensor) its sign is not fixed by fp32 arithmetic -- e.g. the key bias,
whose exact gradient is zero because a per-query constant added to every
score leaves the softmax unchanged -- so both results are valid there and
only the step-size bound applies.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import synth  # noqa: E402
from oracle import gpt2 as og  # noqa: E402
from tile_task_transformer_amd.runtime import Context, GPT2  # noqa: E402
from tests.gpu_util import normwise  # noqa: E402

pytestmark = pytest.mark.gpu


def run_gpu(shape, tiles, params, tokens, n_streams=4, steps=1):
    specs = synth.param_specs(shape)
    with Context(0, n_streams=n_streams) as ctx:
        model = GPT2(ctx, shape, tiles)
        model.set_params(params, specs)
        tok = torch.from_numpy(tokens.astype(np.int32)).cuda()
        losses = []
        for _ in range(steps):
            model.step(tok)
            losses.append(model.loss())
        out = dict(loss=losses, grads=model.get(specs, 1), params=model.get(specs, 0),
                   m=model.get(specs, 2), v=model.get(specs, 3), tasks=model.task_count())
        model.close()
    return out


def check_against_oracle(shape, gpu, params, tokens, w):
    loss, grads, newp, _ = og.step(params, tokens, shape.n_layer, shape.n_head, lr=w.lr, beta1=w.beta1,
                                   beta2=w.beta2, eps=w.eps, wd=w.weight_decay)
    assert abs(gpu["loss"][0] - loss) <= 1e-4 * abs(loss), (gpu["loss"][0], loss)
    for name, ref in grads.items():
        got = gpu["grads"][name].astype(np.float64)
        assert normwise(got, ref) <= 1e-3, (name, normwise(got, ref))
        assert np.abs(got - ref).max() <= 1e-3 * np.abs(ref).max() + 1e-30, name
    for name, ref in newp.items():
        got = gpu["params"][name].astype(np.float64)
        # AdamW fed with the GPU's own gradients
        p1, _, _ = og.adamw(np.asarray(params[name], np.float64), gpu["grads"][name].astype(np.float64), 0, 0, 1,
                            w.lr, w.beta1, w.beta2, w.eps, w.weight_decay)
        err = np.abs(got - p1)
        assert (err <= 1e-3 * np.abs(p1) + 1e-3 * w.lr).all(), (name, err.max())
        # against the full oracle step
        assert np.abs(got - ref).max() <= 2 * w.lr * (1 + 1e-3) + 1e-6 * np.abs(ref).max(), name
        g_ref = grads[name]
        decided = np.abs(g_ref) > 1e-3 * np.abs(g_ref).max()
        if decided.any():
            assert normwise(got[decided], ref[decided]) <= 1e-3, (name, normwise(got[decided], ref[decided]))
    return loss


TINY = synth.WORKLOADS["tiny"]


@pytest.mark.parametrize("tiles", [
    TINY.tiles,                                  # 32 on every axis, clamped
    synth.Tiles(2, 32, 64, 256, 4, 256),         # untiled
    synth.Tiles(1, 16, 16, 48, 2, 40),           # split batch/seq/head, ragged inner and vocab
    synth.Tiles(2, 8, 24, 40, 1, 100),           # ragged embd, one head per tile, seq tile 8
])
def test_tiny_step_matches_oracle(tiles):
    shape = TINY.shape
    params = synth.init_params(shape, seed=0)
    tokens = synth.token_stream(shape, seed=1)
    gpu = run_gpu(shape, tiles, params, tokens)
    check_against_oracle(shape, gpu, params, tokens, TINY)


def test_tiny_step_with_rich_params_two_layers():
    """Larger weights, random LayerNorm gains/biases and two blocks, so every
    gradient term is far from zero."""
    shape = synth.GPT2Shape(2, 256, 64, 4, 256, 32, 2)
    rng = np.random.default_rng(9)
    params = {}
    for name, shp, kind in synth.param_specs(shape):
        base = 1.0 if kind == "ones" else 0.0
        params[name] = (base + rng.standard_normal(shp) * 0.1).astype(np.float32)
    tokens = synth.token_stream(shape, seed=2)
    gpu = run_gpu(shape, synth.Tiles(1, 16, 32, 96, 2, 64), params, tokens)
    check_against_oracle(shape, gpu, params, tokens, TINY)


def test_uniform_logits_loss_is_ln_vocab():
    shape = TINY.shape
    params = synth.init_params(shape, seed=0)
    params["wte"] = np.zeros_like(params["wte"])
    gpu = run_gpu(shape, TINY.tiles, params, synth.token_stream(shape, seed=1))
    assert abs(gpu["loss"][0] - np.log(256)) <= 1e-6 * np.log(256)


def test_tile_shapes_agree_and_steps_are_deterministic():
    shape = TINY.shape
    params = synth.init_params(shape, seed=0)
    tokens = synth.token_stream(shape, seed=1)
    a = run_gpu(shape, TINY.tiles, params, tokens, steps=2)
    b = run_gpu(shape, synth.Tiles(1, 8, 16, 64, 1, 48), params, tokens, steps=2)
    c = run_gpu(shape, TINY.tiles, params, tokens, steps=2, n_streams=1)
    assert abs(a["loss"][1] - b["loss"][1]) <= 1e-5 * abs(a["loss"][1])
    for name in a["grads"]:
        assert normwise(a["grads"][name], b["grads"][name]) <= 1e-4, name
    # same tiles, different stream counts: bitwise equal (no atomics anywhere)
    assert a["loss"] == c["loss"]
    for name in a["params"]:
        assert np.array_equal(a["params"][name], c["params"][name]), name
        assert np.array_equal(a["grads"][name], c["grads"][name]), name


def test_priority_launch_order_gives_the_same_bits():
    """Critical-path priorities reorder launches across 4 streams; every
    result is bitwise the submission-order run's."""
    shape = synth.GPT2Shape(2, 256, 64, 4, 256, 32, 2)
    params = synth.init_params(shape, seed=5)
    tokens = synth.token_stream(shape, seed=6)
    tiles = synth.Tiles(1, 8, 16, 64, 1, 48)
    specs = synth.param_specs(shape)
    outs = []
    for prio in (False, True):
        with Context(0, n_streams=4) as ctx:
            ctx.priorities(prio)
            model = GPT2(ctx, shape, tiles)
            model.set_params(params, specs)
            tok = torch.from_numpy(tokens.astype(np.int32)).cuda()
            losses = []
            for _ in range(2):
                model.step(tok)
                losses.append(model.loss())
            outs.append((losses, model.get(specs, 0), model.get(specs, 1)))
            model.close()
    assert outs[0][0] == outs[1][0]
    for name in outs[0][1]:
        assert np.array_equal(outs[0][1][name], outs[1][1][name]), name
        assert np.array_equal(outs[0][2][name], outs[1][2][name]), name


def test_context_on_caller_streams_gives_the_same_bits():
    """A context whose tasks run on two torch streams (tt_ctx_create_on_streams)
    gives bitwise the results of one with its own two streams, leaves the
    streams usable after it is destroyed, and rejects a repeated or null
    stream."""
    from tile_task_transformer_amd import _lib as L
    shape = synth.GPT2Shape(2, 256, 64, 4, 256, 32, 2)
    params = synth.init_params(shape, seed=5)
    tokens = synth.token_stream(shape, seed=6)
    tiles = synth.Tiles(1, 8, 16, 64, 1, 48)
    specs = synth.param_specs(shape)
    mine = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = []
    for streams in (None, mine):
        with Context(0, n_streams=2, streams=streams) as ctx:
            model = GPT2(ctx, shape, tiles)
            model.set_params(params, specs)
            tok = torch.from_numpy(tokens.astype(np.int32)).cuda()
            losses = []
            for _ in range(2):
                model.step(tok)
                losses.append(model.loss())
            outs.append((losses, model.get(specs, 0), model.get(specs, 1)))
            model.close()
    assert outs[0][0] == outs[1][0]
    for name in outs[0][1]:
        assert np.array_equal(outs[0][1][name], outs[1][1][name]), name
        assert np.array_equal(outs[0][2][name], outs[1][2][name]), name
    # the borrowed streams outlive the context
    with torch.cuda.stream(mine[1]):
        x = torch.arange(1024, device="cuda", dtype=torch.float32) * 2
    mine[1].synchronize()
    assert float(x.sum()) == 1023 * 1024
    with pytest.raises(L.TTError) as e:
        Context(0, streams=[mine[0], mine[0]])
    assert e.value.code == L.TT_ERR_ARG
    with pytest.raises(L.TTError) as e:
        Context(0, streams=[mine[0], 0])
    assert e.value.code == L.TT_ERR_ARG


def test_gpt2_small_full_size_step_matches_oracle():
    """The GPT2-small workload at its full size and README tiles, checked
    against the full fp64 oracle step."""
    w = synth.WORKLOADS["gpt2_small"]
    params = synth.init_params(w.shape, seed=0)
    tokens = synth.token_stream(w.shape, seed=1)
    gpu = run_gpu(w.shape, w.tiles, params, tokens)
    check_against_oracle(w.shape, gpu, params, tokens, w)


def test_two_minibatches_make_the_batch_step():
    """The README's batch/minibatch flags: a batch of 4 windows processed as
    2 minibatches of 2 with gradients accumulated, then one update, is the
    step on the whole batch (mean loss over all its tokens)."""
    shape = TINY.shape
    big = synth.GPT2Shape(shape.n_layer, shape.vocab, shape.n_embd, shape.n_head, shape.n_inner, shape.seq,
                          2 * shape.batch)
    params = synth.init_params(shape, seed=0)
    tokens = synth.token_stream(big, seed=1)
    specs = synth.param_specs(shape)
    with Context(0, n_streams=4) as ctx:
        model = GPT2(ctx, shape, synth.Tiles(1, 16, 32, 64, 2, 48))
        model.set_params(params, specs)
        model.step(torch.from_numpy(tokens.astype(np.int32)).cuda(), n_micro=2)
        gpu = dict(loss=[model.loss()], grads=model.get(specs, 1), params=model.get(specs, 0))
        model.close()
    check_against_oracle(big, gpu, params, tokens, TINY)


def test_lr_warmup_schedule():
    """start_lr at the first update, lr from update full_lr_iter on, linear in
    between: with start_lr = 0 the first update leaves every parameter
    exactly as it was, so the second forward repeats the first bitwise; three
    steps follow the oracle's schedule."""
    shape = TINY.shape
    params = synth.init_params(shape, seed=0)
    tokens = synth.token_stream(shape, seed=1)
    specs = synth.param_specs(shape)
    lr, full = 1e-3, 3
    with Context(0, n_streams=4) as ctx:
        model = GPT2(ctx, shape, TINY.tiles)
        model.set_params(params, specs)
        tok = torch.from_numpy(tokens.astype(np.int32)).cuda()
        losses = []
        for _ in range(3):
            model.step(tok, lr=lr, start_lr=0.0, full_lr_iter=full)
            losses.append(model.loss())
        got = model.get(specs, 0)
        model.close()
    assert losses[1] == losses[0]
    p, state, ref_losses, lrs, decided = params, None, [], [], {}
    for t in range(1, 4):
        lr_t = og.lr_at(t, lr, 0.0, full)
        lrs.append(lr_t)
        loss, grads, p, state = og.step(p, tokens, shape.n_layer, shape.n_head, lr=lr_t, beta1=TINY.beta1,
                                        beta2=TINY.beta2, eps=TINY.eps, wd=TINY.weight_decay, t=t, state=state)
        ref_losses.append(loss)
        for name, g in grads.items():  # elements whose update direction every step's gradient decides
            d = np.abs(g) > 1e-3 * np.abs(g).max()
            decided[name] = d if t == 1 else decided[name] & d
    assert lrs == [0.0, lr / 2, lr]
    for a, b in zip(losses, ref_losses):
        assert abs(a - b) <= 1e-4 * abs(b), (a, b)
    for name, ref in p.items():
        g = got[name].astype(np.float64)
        assert np.abs(g - ref).max() <= 2 * sum(lrs) * (1 + 1e-3) + 1e-6 * np.abs(ref).max(), name
        if decided[name].any():
            assert normwise(g[decided[name]], ref[decided[name]]) <= 1e-3, name


def test_sgd_steps_match_oracle():
    """The README's --optimizer choice: plain SGD. The kernel applies exactly
    p - lr*g to the GPU's own gradients, the moments stay untouched, and two
    steps follow the oracle's chain (second loss within the loss bar, the
    parameters within lr times the gradient bar)."""
    shape = TINY.shape
    params = synth.init_params(shape, seed=0)
    tokens = synth.token_stream(shape, seed=1)
    specs = synth.param_specs(shape)
    lr = 0.1
    with Context(0, n_streams=2) as ctx:
        model = GPT2(ctx, shape, TINY.tiles)
        model.set_params(params, specs)
        tok = torch.from_numpy(tokens.astype(np.int32)).cuda()
        model.step(tok, lr=lr, optimizer="sgd")
        loss1, g1, p1 = model.loss(), model.get(specs, 1), model.get(specs, 0)
        m, v = model.get(specs, 2), model.get(specs, 3)
        model.step(tok, lr=lr, optimizer="sgd")
        loss2 = model.loss()
        model.close()
    rl1, rg1, rp1, _ = og.step(params, tokens, shape.n_layer, shape.n_head, lr=lr, optimizer="sgd")
    rl2, _, _, _ = og.step(rp1, tokens, shape.n_layer, shape.n_head, lr=lr, optimizer="sgd")
    assert abs(loss1 - rl1) <= 1e-4 * abs(rl1)
    assert abs(loss2 - rl2) <= 1e-4 * abs(rl2), (loss2, rl2)
    assert loss2 < loss1
    for name, p0 in params.items():
        p0 = np.asarray(p0, np.float32).astype(np.float64)
        got = p1[name].astype(np.float64)
        own = og.sgd(p0, g1[name].astype(np.float64), lr)
        assert np.abs(got - own).max() <= 2.0 ** -22 * (np.abs(p0).max() + lr * np.abs(g1[name]).max()), name
        gmax = np.abs(rg1[name]).max()
        assert np.abs(got - rp1[name]).max() <= lr * 1e-3 * gmax + 2.0 ** -22 * np.abs(p0).max() + 1e-30, name
        assert not m[name].any() and not v[name].any(), name


def test_task_timing_and_busy_union():
    """Per-task timing over a whole step: every task of the step is timed
    once, the union of their GPU intervals is positive and no longer than
    the span from the first start to the last end, and the per-label totals
    are at least the union (overlapping tasks on several streams count once
    in the union, once each in the totals)."""
    shape, tiles = TINY.shape, TINY.tiles
    params = synth.init_params(shape, seed=0)
    tokens = synth.token_stream(shape, seed=1)
    with Context(0, n_streams=4) as ctx:
        model = GPT2(ctx, shape, tiles)
        model.set_params(params, synth.param_specs(shape))
        tok = torch.from_numpy(tokens.astype(np.int32)).cuda()
        model.step(tok)
        ctx.profile("*")
        model.step(tok)
        busy = ctx.profile_busy()
        per_label = ctx.profile_take()
        ctx.profile(None)
        n = model.task_count()
        model.close()
    assert busy["tasks"] == n == sum(v["count"] for v in per_label.values())
    assert 0 < busy["busy_ms"] <= busy["span_ms"] * (1 + 1e-6)
    assert sum(v["total_ms"] for v in per_label.values()) >= busy["busy_ms"] * (1 - 1e-6)
