"""The LLaMA-style wide model (4 blocks, d 8192, 64 heads of 128, SwiGLU
width 22016 -- two full 8192-wide inner tiles and a ragged 5632-wide one --,
vocab 32000, seq 1024, batch 4; 3.76 B parameters) at its full size, with
the tiles and the single executor stream its benchmark line uses.

The fp64 oracle cannot run this step in seconds, so the full-size run is
checked by what holds at any size:
  * per-token losses at sampled positions against the oracle run on a
    prefix of each window (causal attention and rotary positions counted
    from the window's start: position t depends on tokens 0..t only);
  * the mean of the per-token losses is the reported loss;
  * at initialisation the loss is close to its closed form;
and a one-block, one-sequence slice with the same widths and tiles is
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
from oracle import llama as ol  # noqa: E402
from tile_task_transformer_amd.runtime import Context, GPT2  # noqa: E402

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(900)]

WIDE = synth.LLAMA_WORKLOADS["llama_wide4"]
THREADS = min(16, os.cpu_count() or 1)


def log(msg):
    print(f"[llama wide] {msg}", flush=True)


@contextlib.contextmanager
def stepped(shape, tiles, params, tokens, n_streams=1):
    """A LLaMA-style model after one training step; yields (model, specs)."""
    specs = synth.llama_param_specs(shape)
    t0 = time.perf_counter()
    with Context(0, n_streams=n_streams, window=4096) as ctx:
        model = GPT2(ctx, shape, tiles, family="llama")
        try:
            model.set_params(params, specs)
            tok = torch.from_numpy(tokens.astype(np.int32)).cuda()
            model.step(tok)
            log(f"step done: loss {model.loss():.6f}, {model.task_count()} tasks, "
                f"{time.perf_counter() - t0:.1f} s with upload")
            yield model, specs
        finally:
            model.close()


def test_full_size_token_losses_match_oracle_on_prefixes():
    t0 = time.perf_counter()
    params = synth.init_params(WIDE.shape, seed=0, threads=THREADS, specs=synth.llama_param_specs(WIDE.shape))
    tokens = synth.token_stream(WIDE.shape, seed=1)
    log(f"parameters drawn in {time.perf_counter() - t0:.1f} s")
    with stepped(WIDE.shape, WIDE.tiles, params, tokens) as (model, _):
        loss = model.loss()
        rows = model.row_losses().astype(np.float64)
    x, y = synth.split_tokens(tokens)
    prefix = 16
    t0 = time.perf_counter()
    ref = ol.row_losses(params, x[:, :prefix], y[:, :prefix], WIDE.shape.n_layer, WIDE.shape.n_head)
    log(f"oracle on {x.shape[0]}x{prefix} prefixes: {time.perf_counter() - t0:.1f} s")
    got = rows[:, :prefix]
    assert np.all(np.abs(got - ref) <= 1e-4 * np.abs(ref)), np.abs(got - ref).max()
    assert abs(rows.mean() - loss) <= 1e-5 * loss
    # at init each logit is a sum of d products of an RMSNorm output (unit
    # mean square per token, gain 1) and an N(0, 0.02^2) head weight:
    # Gaussian with variance s2 = d * 0.02^2, so E[logsumexp] = ln V + s2 / 2
    # for large V
    s2 = WIDE.shape.n_embd * 0.02 ** 2
    expect = np.log(WIDE.shape.vocab) + s2 / 2
    assert abs(loss - expect) < 0.02 * expect, (loss, expect)


SLICE = synth.GPT2Shape(1, WIDE.shape.vocab, WIDE.shape.n_embd, WIDE.shape.n_head, WIDE.shape.n_inner,
                        WIDE.shape.seq, 1)


def test_one_block_slice_matches_oracle():
    specs = synth.llama_param_specs(SLICE)
    params = synth.init_params(SLICE, seed=0, threads=THREADS, specs=specs)
    tokens = synth.token_stream(SLICE, seed=1)
    t0 = time.perf_counter()
    loss, grads, newp, _ = ol.step(params, tokens, SLICE.n_layer, SLICE.n_head, lr=WIDE.lr, beta1=WIDE.beta1,
                                   beta2=WIDE.beta2, eps=WIDE.eps, wd=WIDE.weight_decay)
    log(f"oracle step on the one-block slice: {time.perf_counter() - t0:.1f} s")
    t = WIDE.tiles
    tiles = synth.Tiles(1, t.seq, t.embd, t.inner, t.head, t.vocab)
    with stepped(SLICE, tiles, params, tokens) as (model, specs):
        assert abs(model.loss() - loss) <= 1e-4 * abs(loss)
        for i, (name, shp, _) in enumerate(specs):
            got = model._wrap(i, 1, shp).copy_out().astype(np.float64)
            ref = grads[name]
            assert normwise(got, ref) <= 1e-3, (name, normwise(got, ref))
            assert np.abs(got - ref).max() <= 1e-3 * np.abs(ref).max() + 1e-30, name
            p = model._wrap(i, 0, shp).copy_out().astype(np.float64)
            # AdamW against the oracle's AdamW fed with the GPU's own gradients
            p1, _, _ = og.adamw(np.asarray(params[name], np.float64), got, 0, 0, 1, WIDE.lr, WIDE.beta1,
                                WIDE.beta2, WIDE.eps, WIDE.weight_decay)
            assert (np.abs(p - p1) <= 1e-3 * np.abs(p1) + 1e-3 * WIDE.lr).all(), name
            # against the full oracle step: a sign flip of one lr step where
            # the gradient is near zero, agreement where it decides
            assert np.abs(p - newp[name]).max() <= 2 * WIDE.lr * (1 + 1e-3) + 1e-6 * np.abs(newp[name]).max(), name
            decided = np.abs(ref) > 1e-3 * np.abs(ref).max()
            if decided.any():
                assert normwise(p[decided], newp[name][decided]) <= 1e-3, name
