"""The wide GPT2 (4 blocks, d 8192, 64 heads of 128, inner 32768, vocab
50257, seq 1024, batch 4; 3.64 B parameters) at its full size, with the
large tiles (seq 1024, embd 2048, inner 8192, 16 heads, vocab 2048) and the
small ones (256, 512, 2048, 8, 512) that give ~16x more tile-grid cells --
the pages' deep-and-narrow regime ("Performance" on the NNTile review).

The fp64 oracle cannot run this step in seconds, so the full-size runs are
checked by what holds at any size:
  * per-token losses at sampled positions against the oracle run on a
    prefix of each window (causal attention: position t depends on tokens
    0..t only);
  * the two tilings agree (tiling does not change the mathematics: the
    review's "Core claim");
  * out-of-core residency (pinned-host homes, a 32 GiB device arena) is
    bitwise equal to the all-in-HBM run;
and a one-block, one-sequence slice with the same per-tile widths is
checked element by element against the full oracle step.
"""
import contextlib
import os
import time

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import synth  # noqa: E402
from tests.gpu_util import normwise  # noqa: E402
from oracle import gpt2 as og  # noqa: E402
from tile_task_transformer_amd import _lib as L  # noqa: E402
from tile_task_transformer_amd.runtime import Context, GPT2  # noqa: E402

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(900)]

WIDE = synth.WORKLOADS["wide4"]
SMALL_TILES = synth.WORKLOADS["wide4_small_tiles"].tiles
THREADS = min(16, os.cpu_count() or 1)


def log(msg):
    print(f"[wide] {msg}", flush=True)


@contextlib.contextmanager
def stepped(shape, tiles, params, tokens, home=L.TT_HOME_DEVICE, budget=0, n_streams=4):
    """A model after one training step; yields (model, specs, ctx)."""
    specs = synth.param_specs(shape)
    t0 = time.perf_counter()
    with Context(0, n_streams=n_streams, window=4096, device_budget=budget) as ctx:
        model = GPT2(ctx, shape, tiles, param_home=home)
        try:
            model.set_params(params, specs)
            tok = torch.from_numpy(tokens.astype(np.int32)).cuda()
            model.step(tok)
            log(f"step done: loss {model.loss():.6f}, {model.task_count()} tasks, "
                f"{time.perf_counter() - t0:.1f} s with upload")
            yield model, specs, ctx
        finally:
            model.close()


def collect(model, specs, which):
    return {name: model._wrap(i, which, shp).copy_out() for i, (name, shp, _) in enumerate(specs)}


@pytest.fixture(scope="module")
def inputs():
    t0 = time.perf_counter()
    params = synth.init_params(WIDE.shape, seed=0, threads=THREADS)
    tokens = synth.token_stream(WIDE.shape, seed=1)
    log(f"parameters drawn in {time.perf_counter() - t0:.1f} s")
    return params, tokens


@pytest.fixture(scope="module")
def reference(inputs):
    """Large tiles, all in HBM: loss, per-token losses, gradients, new params."""
    params, tokens = inputs
    with stepped(WIDE.shape, WIDE.tiles, params, tokens) as (model, specs, _):
        return dict(loss=model.loss(), rows=model.row_losses(), grads=collect(model, specs, 1),
                    params=collect(model, specs, 0))


def test_sampled_token_losses_match_oracle_on_prefixes(inputs, reference):
    params, tokens = inputs
    x, y = synth.split_tokens(tokens)
    prefix = 16
    t0 = time.perf_counter()
    ref = og.row_losses(params, x[:, :prefix], y[:, :prefix], WIDE.shape.n_layer, WIDE.shape.n_head)
    log(f"oracle on {x.shape[0]}x{prefix} prefixes: {time.perf_counter() - t0:.1f} s")
    got = reference["rows"][:, :prefix].astype(np.float64)
    assert np.all(np.abs(got - ref) <= 1e-4 * np.abs(ref)), np.abs(got - ref).max()
    # the mean of the per-token losses is the reported loss
    assert abs(reference["rows"].astype(np.float64).mean() - reference["loss"]) <= 1e-5 * reference["loss"]
    # at init each logit is a sum of d products of a unit-variance LayerNorm
    # output and an N(0, 0.02^2) embedding weight: Gaussian with variance
    # s2 = d * 0.02^2, so E[logsumexp] = ln V + s2 / 2 for large V
    s2 = WIDE.shape.n_embd * 0.02 ** 2
    expect = np.log(WIDE.shape.vocab) + s2 / 2
    assert abs(reference["loss"] - expect) < 0.02 * expect, (reference["loss"], expect)


def _assert_updates_agree(got, ref, g_ref, lr):
    """AdamW turns gradient noise into a sign flip of a step of size lr where
    the gradient is near zero; elsewhere the updated values must agree."""
    assert np.abs(got - ref).max() <= 2 * lr * (1 + 1e-3) + 1e-6 * np.abs(ref).max()
    decided = np.abs(g_ref) > 1e-3 * np.abs(g_ref).max()
    if decided.any():
        assert normwise(got[decided].astype(np.float64), ref[decided].astype(np.float64)) <= 1e-3


def test_small_tiles_agree_with_large_tiles(inputs, reference):
    params, tokens = inputs
    with stepped(WIDE.shape, SMALL_TILES, params, tokens) as (model, specs, _):
        loss = model.loss()
        assert abs(loss - reference["loss"]) <= 1e-5 * reference["loss"]
        rows = model.row_losses().astype(np.float64)
        assert np.all(np.abs(rows - reference["rows"]) <= 1e-4 * np.abs(reference["rows"]))
        for i, (name, shp, _) in enumerate(specs):
            g = model._wrap(i, 1, shp).copy_out()
            gr = reference["grads"][name]
            assert normwise(g.astype(np.float64), gr.astype(np.float64)) <= 1e-3, name
            assert np.abs(g - gr).max() <= 1e-3 * np.abs(gr).max() + 1e-30, name
            p = model._wrap(i, 0, shp).copy_out()
            _assert_updates_agree(p, reference["params"][name], gr, WIDE.lr)


def test_out_of_core_is_bitwise_equal_to_hbm(inputs, reference):
    params, tokens = inputs
    budget = 32 << 30
    with stepped(WIDE.shape, WIDE.tiles, params, tokens, home=L.TT_HOME_PINNED_HOST, budget=budget) as (
            model, specs, ctx):
        st = ctx.stats()
        log(f"residency: h2d {st['h2d_bytes'] / 1e9:.1f} GB, d2h {st['d2h_bytes'] / 1e9:.1f} GB, "
            f"{st['evictions']} evictions, {st['prefetches']} prefetches")
        assert st["evictions"] > 0 and st["d2h_bytes"] > 0
        assert model.loss() == reference["loss"]
        assert np.array_equal(model.row_losses(), reference["rows"])
        for i, (name, shp, _) in enumerate(specs):
            assert np.array_equal(model._wrap(i, 1, shp).copy_out(), reference["grads"][name]), name
            assert np.array_equal(model._wrap(i, 0, shp).copy_out(), reference["params"][name]), name


SLICE = synth.GPT2Shape(1, WIDE.shape.vocab, WIDE.shape.n_embd, WIDE.shape.n_head, WIDE.shape.n_inner,
                        WIDE.shape.seq, 1)


@pytest.fixture(scope="module")
def slice_oracle():
    params = synth.init_params(SLICE, seed=0, threads=THREADS)
    tokens = synth.token_stream(SLICE, seed=1)
    t0 = time.perf_counter()
    loss, grads, newp, _ = og.step(params, tokens, SLICE.n_layer, SLICE.n_head, lr=WIDE.lr, beta1=WIDE.beta1,
                                   beta2=WIDE.beta2, eps=WIDE.eps, wd=WIDE.weight_decay)
    log(f"oracle step on the one-block slice: {time.perf_counter() - t0:.1f} s")
    return params, tokens, loss, grads, newp


@pytest.mark.parametrize("tiles", [WIDE.tiles, SMALL_TILES], ids=["large_tiles", "small_tiles"])
def test_one_block_slice_matches_oracle(slice_oracle, tiles):
    params, tokens, loss, grads, newp = slice_oracle
    tiles = synth.Tiles(1, tiles.seq, tiles.embd, tiles.inner, tiles.head, tiles.vocab)
    with stepped(SLICE, tiles, params, tokens) as (model, specs, _):
        assert abs(model.loss() - loss) <= 1e-4 * abs(loss)
        for i, (name, shp, _) in enumerate(specs):
            got = model._wrap(i, 1, shp).copy_out().astype(np.float64)
            ref = grads[name]
            assert normwise(got, ref) <= 1e-3, (name, normwise(got, ref))
            assert np.abs(got - ref).max() <= 1e-3 * np.abs(ref).max() + 1e-30, name
            p = model._wrap(i, 0, shp).copy_out()
            _assert_updates_agree(p, newp[name], ref, WIDE.lr)
