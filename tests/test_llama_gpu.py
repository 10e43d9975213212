"""Parity of the LLaMA-style path (HIP) with the fp64 oracle (oracle/llama.py).

Kernels: RMSNorm forward/backward over 1..4 feature tiles, the rotary table
and rotation (forward and transposed) with position offsets and several
sequences per tile, SwiGLU forward/backward (vector and scalar paths, in
place). Tolerances follow the fp32 arithmetic of memory-bound ops: a few
units of 2^-24 of the inputs' scale.

Model: the tiled LLaMA step against the untiled fp64 oracle step, with the
bar of the GPT2 step (tests/test_gpt2_gpu.py): loss within 1e-4 relative,
every gradient normwise within 1e-3 and max error within 1e-3 of its
tensor's largest entry, AdamW against the oracle's AdamW fed with the GPU's
own gradients, updated parameters against the full oracle step where the
fp64 gradient decides the direction. Same-tile runs on 1 and 4 streams,
and pinned-host parameters, are bitwise equal to the all-in-HBM 4-stream run.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import synth  # noqa: E402
import tile_task_transformer_amd as tt  # noqa: E402
from oracle import gpt2 as og  # noqa: E402
from oracle import llama as ol  # noqa: E402
from tile_task_transformer_amd import _lib as L  # noqa: E402
from tile_task_transformer_amd.runtime import Context, GPT2  # noqa: E402
from tests.gpu_util import EPS32, assert_rel, dev, empty, host, normwise  # noqa: E402

pytestmark = pytest.mark.gpu


# ------------------------------------------------------------------ kernels

@pytest.mark.parametrize("rows,cols", [(37, [64]), (5, [32, 32, 16]), (130, [512, 512, 256]), (64, [2048, 768]),
                                       (1, [4]), (0, [64])])
@pytest.mark.parametrize("dx_acc", [0, 1])
def test_rmsnorm_fwd_bwd(rows, cols, dx_acc):
    seed = rows + sum(cols) + dx_acc
    total = sum(cols)
    x = synth.rand_normal((rows, total), seed, std=2.0)
    g = synth.rand_normal((total,), seed + 1) + 1.0
    dy = synth.rand_normal((rows, total), seed + 2)
    dx0 = synth.rand_normal((rows, total), seed + 3)
    dg0 = synth.rand_normal((total,), seed + 4)
    y_ref, r_ref = ol.rmsnorm_fwd(x.astype(np.float64), g.astype(np.float64), 1e-5)
    dx_ref, dg_ref = ol.rmsnorm_bwd(dy.astype(np.float64), x.astype(np.float64), g.astype(np.float64), r_ref)
    if dx_acc:
        dx_ref = dx_ref + dx0
    dg_ref = dg_ref + dg0
    bounds = np.cumsum([0] + cols)
    sl = [slice(bounds[i], bounds[i + 1]) for i in range(len(cols))]
    xs = [dev(x[:, s]) for s in sl]
    gs = [dev(g[s]) for s in sl]
    ys = [empty((rows, c)) for c in cols]
    rstd = empty((max(rows, 1),))
    tt.tile_rmsnorm_fwd(None, rows, cols, xs, gs, rstd, ys, 1e-5)
    dys = [dev(dy[:, s]) for s in sl]
    dxs = [dev(dx0[:, s]) for s in sl]
    dgs = [dev(dg0[s]) for s in sl]
    need = tt.tile_rmsnorm_bwd_workspace(rows, total)
    ws = torch.empty(max(need, 16) // 4, device="cuda")
    tt.tile_rmsnorm_bwd(None, rows, cols, dys, xs, gs, rstd, dxs, dx_acc, dgs, ws, need)
    if rows == 0:
        for s, t in zip(sl, dgs):
            assert np.array_equal(host(t), dg0[s])
        return
    y = np.concatenate([host(t) for t in ys], 1)
    dx = np.concatenate([host(t) for t in dxs], 1)
    dg = np.concatenate([host(t) for t in dgs])
    assert_rel(host(rstd)[:rows], r_ref, 8 * EPS32, what="rstd")
    assert_rel(y, y_ref, 16 * EPS32, 16 * EPS32 * np.abs(y_ref).max(), "y")
    scale = np.abs(dy).max() * np.abs(g).max() * r_ref.max()
    assert_rel(dx, dx_ref, 0, 64 * EPS32 * (scale + np.abs(dx_ref).max()), "dx")
    n_ref = x.astype(np.float64) * r_ref[:, None]
    bound = 8 * EPS32 * (rows + 4) * (np.abs(dy) * np.abs(n_ref)).sum(0) + 8 * EPS32 * np.abs(dg0)
    assert (np.abs(dg - dg_ref) <= bound + 1e-30).all(), "dgamma"


def test_rmsnorm_rejects_bad_widths():
    with pytest.raises(L.TTError) as e:
        tt.tile_rmsnorm_fwd(None, 4, [30], [empty((4, 30))], [empty((30,))], empty((4,)), [empty((4, 30))])
    assert e.value.code == L.TT_ERR_SHAPE
    with pytest.raises(L.TTError) as e:
        tt.tile_rmsnorm_fwd(None, 4, [16, 32], [empty((4, 16)), empty((4, 32))], [empty((16,)), empty((32,))],
                            empty((4,)), [empty((4, 16)), empty((4, 32))])
    assert e.value.code == L.TT_ERR_SHAPE


@pytest.mark.parametrize("hd", [16, 32, 64, 128])
def test_rope_table(hd):
    seq = 1024
    tab = empty((seq, hd))
    tt.tile_rope_table(None, seq, hd, 10000.0, tab)
    ang = ol.rope_angles(seq, hd)
    ref = np.concatenate([np.cos(ang), np.sin(ang)], 1)
    got = host(tab)
    # each entry is its fp64 value rounded once to fp32
    assert np.abs(got - ref).max() <= 2 ** -24 * 1.0001


@pytest.mark.parametrize("batch,length,heads,hd,pos_off", [(3, 8, 2, 64, 16), (1, 1024, 4, 128, 0), (2, 5, 3, 16, 27),
                                                            (4, 32, 12, 64, 992), (1, 7, 1, 32, 0)])
def test_rope_forward_and_transpose(batch, length, heads, hd, pos_off):
    seq = 1024
    tab = empty((seq, hd))
    tt.tile_rope_table(None, seq, hd, 10000.0, tab)
    rows = batch * length
    x = synth.rand_normal((batch, length, heads, hd), rows + hd + pos_off)
    ang = ol.rope_angles(seq, hd)[pos_off:pos_off + length]
    xh = x.astype(np.float64).transpose(0, 2, 1, 3)
    for inverse in (0, 1):
        ref = (ol.rope_bwd if inverse else ol.rope_fwd)(xh, ang).transpose(0, 2, 1, 3)
        t = dev(x)
        tt.tile_rope(None, t, rows, heads, hd, length, pos_off, tab, seq, inverse)
        # the table's entries are rounded to fp32 (2^-24 relative), the two
        # products and the sum add three roundings
        assert_rel(host(t), ref, 0, 8 * EPS32 * np.abs(x).max(), f"rope inverse={inverse}")
    # forward then transpose gives back the input
    t = dev(x)
    tt.tile_rope(None, t, rows, heads, hd, length, pos_off, tab, seq, 0)
    tt.tile_rope(None, t, rows, heads, hd, length, pos_off, tab, seq, 1)
    assert_rel(host(t), x.astype(np.float64), 0, 16 * EPS32 * np.abs(x).max(), "round trip")
    with pytest.raises(L.TTError):
        tt.tile_rope(None, dev(x), rows, heads, hd, length, seq - length + 1, tab, seq, 0)
    # several tiles in one launch: each gets the single-tile result, bit for bit
    xs = [synth.rand_normal((batch, length, heads, hd), rows + hd + pos_off + j) for j in range(3)]
    ts = [dev(v) for v in xs]
    tt.tile_rope_multi(None, ts, rows, heads, hd, length, pos_off, tab, seq, 0)
    for v, t in zip(xs, ts):
        one = dev(v)
        tt.tile_rope(None, one, rows, heads, hd, length, pos_off, tab, seq, 0)
        assert np.array_equal(host(t), host(one))


@pytest.mark.parametrize("n", [4096 + 64, 1001, 3, 0])
def test_swiglu_fwd_bwd(n):
    a = synth.rand_normal((max(n, 1),), n + 1, std=4.0)[:n]
    b = synth.rand_normal((max(n, 1),), n + 2)[:n]
    dh = synth.rand_normal((max(n, 1),), n + 3)[:n]
    a64, b64, d64 = a.astype(np.float64), b.astype(np.float64), dh.astype(np.float64)
    h = empty((max(n, 1),))
    tt.tile_swiglu_fwd(None, n, dev(a), dev(b), h)
    if n:
        assert_rel(host(h)[:n], ol.swiglu_fwd(a64, b64), 32 * EPS32, 1e-30, "h")
    da_ref, db_ref = ol.swiglu_bwd(d64, a64, b64)
    da, db = empty((max(n, 1),)), empty((max(n, 1),))
    A, B = dev(a), dev(b)
    tt.tile_swiglu_bwd(None, n, dev(dh), A, B, da, db)
    if n:
        scale = np.abs(d64 * b64).max()
        assert_rel(host(da)[:n], da_ref, 32 * EPS32, 32 * EPS32 * scale, "da")
        assert_rel(host(db)[:n], db_ref, 32 * EPS32, 1e-30, "db")
        # in place (a <- da, b <- db) gives the same bits
        da_sep, db_sep = host(da)[:n], host(db)[:n]
        tt.tile_swiglu_bwd(None, n, dev(dh), A, B, A, B)
        assert np.array_equal(host(A)[:n], da_sep) and np.array_equal(host(B)[:n], db_sep)


# -------------------------------------------------------------------- model

def run_llama(shape, tiles, params, tokens, n_streams=4, steps=1, home=L.TT_HOME_DEVICE, budget=0):
    specs = synth.llama_param_specs(shape)
    with Context(0, n_streams=n_streams, device_budget=budget) as ctx:
        model = GPT2(ctx, shape, tiles, family="llama", param_home=home)
        model.set_params(params, specs)
        tok = torch.from_numpy(tokens.astype(np.int32)).cuda()
        losses = []
        for _ in range(steps):
            model.step(tok)
            losses.append(model.loss())
        out = dict(loss=losses, grads=model.get(specs, 1), params=model.get(specs, 0), m=model.get(specs, 2),
                   v=model.get(specs, 3))
        model.close()
    return out


def check_llama_against_oracle(shape, gpu, params, tokens, w):
    loss, grads, newp, _ = ol.step(params, tokens, shape.n_layer, shape.n_head, lr=w.lr, beta1=w.beta1,
                                   beta2=w.beta2, eps=w.eps, wd=w.weight_decay)
    assert abs(gpu["loss"][0] - loss) <= 1e-4 * abs(loss), (gpu["loss"][0], loss)
    for name, ref in grads.items():
        got = gpu["grads"][name].astype(np.float64)
        assert normwise(got, ref) <= 1e-3, (name, normwise(got, ref))
        assert np.abs(got - ref).max() <= 1e-3 * np.abs(ref).max() + 1e-30, name
    for name, ref in newp.items():
        got = gpu["params"][name].astype(np.float64)
        p1, _, _ = og.adamw(np.asarray(params[name], np.float64), gpu["grads"][name].astype(np.float64), 0, 0, 1,
                            w.lr, w.beta1, w.beta2, w.eps, w.weight_decay)
        err = np.abs(got - p1)
        assert (err <= 1e-3 * np.abs(p1) + 1e-3 * w.lr).all(), (name, err.max())
        assert np.abs(got - ref).max() <= 2 * w.lr * (1 + 1e-3) + 1e-6 * np.abs(ref).max(), name
        g_ref = grads[name]
        decided = np.abs(g_ref) > 1e-3 * np.abs(g_ref).max()
        if decided.any():
            assert normwise(got[decided], ref[decided]) <= 1e-3, (name, normwise(got[decided], ref[decided]))
    return loss


LT = synth.LLAMA_WORKLOADS["llama_tiny"]


@pytest.mark.parametrize("tiles", [
    LT.tiles,                                    # two embd tiles, ragged inner (176 = 5 x 32 + 16)
    synth.Tiles(2, 32, 64, 256, 4, 256),         # untiled
    synth.Tiles(1, 16, 16, 48, 2, 40),           # split batch/seq/head, ragged inner and vocab
    synth.Tiles(2, 8, 32, 40, 1, 100),           # one head per tile, seq tile 8 (rotary offsets)
])
def test_llama_tiny_step_matches_oracle(tiles):
    shape = LT.shape
    params = synth.init_params(shape, seed=0, specs=synth.llama_param_specs(shape))
    tokens = synth.token_stream(shape, seed=1)
    gpu = run_llama(shape, tiles, params, tokens)
    check_llama_against_oracle(shape, gpu, params, tokens, LT)


def test_llama_rich_params_two_layers():
    """Larger weights and random RMSNorm gains over two blocks, so every
    gradient term is far from zero."""
    shape = synth.GPT2Shape(2, 256, 64, 4, 176, 32, 2)
    rng = np.random.default_rng(9)
    params = {}
    for name, shp, kind in synth.llama_param_specs(shape):
        base = 1.0 if kind == "ones" else 0.0
        params[name] = (base + rng.standard_normal(shp) * 0.1).astype(np.float32)
    tokens = synth.token_stream(shape, seed=2)
    gpu = run_llama(shape, synth.Tiles(1, 16, 32, 96, 2, 64), params, tokens)
    check_llama_against_oracle(shape, gpu, params, tokens, LT)


def test_llama_streams_and_pinned_homes_are_bitwise_equal():
    shape = synth.GPT2Shape(2, 256, 64, 4, 176, 32, 2)
    specs = synth.llama_param_specs(shape)
    params = synth.init_params(shape, seed=3, specs=specs)
    tokens = synth.token_stream(shape, seed=4)
    tiles = synth.Tiles(1, 16, 32, 64, 2, 64)
    a = run_llama(shape, tiles, params, tokens, steps=2)
    b = run_llama(shape, tiles, params, tokens, steps=2, n_streams=1)
    c = run_llama(shape, tiles, params, tokens, steps=2, home=L.TT_HOME_PINNED_HOST, budget=300 * 1024)
    for other in (b, c):
        assert other["loss"] == a["loss"]
        for key in ("params", "grads", "m", "v"):
            for name in a[key]:
                assert np.array_equal(other[key][name], a[key][name]), (key, name)


def test_llama_two_minibatches_make_the_batch_step():
    """Gradient accumulation for the LLaMA-style step: 2 minibatches of 2
    windows, then one update, against the oracle's step on all 4 windows."""
    shape = LT.shape
    big = synth.GPT2Shape(shape.n_layer, shape.vocab, shape.n_embd, shape.n_head, shape.n_inner, shape.seq,
                          2 * shape.batch)
    specs = synth.llama_param_specs(shape)
    params = synth.init_params(shape, seed=0, specs=specs)
    tokens = synth.token_stream(big, seed=1)
    with Context(0, n_streams=4) as ctx:
        model = GPT2(ctx, shape, synth.Tiles(1, 16, 32, 64, 2, 48), family="llama")
        model.set_params(params, specs)
        model.step(torch.from_numpy(tokens.astype(np.int32)).cuda(), n_micro=2)
        gpu = dict(loss=[model.loss()], grads=model.get(specs, 1), params=model.get(specs, 0))
        model.close()
    check_llama_against_oracle(big, gpu, params, tokens, LT)


def test_llama_small_full_size_step_matches_oracle():
    """The LLaMA-style model at GPT2-small's width and depth (12 blocks, d
    768, SwiGLU width 2048, vocab 32000, 4 x 1024 tokens, its benchmark
    tiles), against the full fp64 oracle step."""
    w = synth.LLAMA_WORKLOADS["llama_small"]
    params = synth.init_params(w.shape, seed=0, threads=8, specs=synth.llama_param_specs(w.shape))
    tokens = synth.token_stream(w.shape, seed=1)
    gpu = run_llama(w.shape, w.tiles, params, tokens)
    check_llama_against_oracle(w.shape, gpu, params, tokens, w)
