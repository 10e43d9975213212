"""Out-of-core residency: parameters, gradients and AdamW moments whose home
is pinned host RAM are staged through a small device arena (LRU eviction,
write-back of dirty tiles, look-ahead prefetch). Placement must not change
any result: the step is bitwise equal to the all-in-HBM run (tile placement
is the runtime's business, not the math's -- the pages' "Core claim")."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import synth  # noqa: E402
from tile_task_transformer_amd import _lib as L  # noqa: E402
from tile_task_transformer_amd.runtime import Context, GPT2  # noqa: E402

pytestmark = pytest.mark.gpu


def _run(shape, tiles, params, tokens, home, budget, steps=2):
    specs = synth.param_specs(shape)
    with Context(0, n_streams=4, device_budget=budget) as ctx:
        model = GPT2(ctx, shape, tiles, param_home=home)
        model.set_params(params, specs)
        tok = torch.from_numpy(tokens.astype(np.int32)).cuda()
        losses = []
        for _ in range(steps):
            model.step(tok)
            losses.append(model.loss())
        out = dict(loss=losses, params=model.get(specs, 0), grads=model.get(specs, 1), m=model.get(specs, 2),
                   v=model.get(specs, 3), stats=ctx.stats())
        model.close()
    return out


@pytest.mark.parametrize("budget_kib", [128, 400])
def test_pinned_host_step_is_bitwise_equal_to_hbm(budget_kib):
    w = synth.WORKLOADS["tiny"]
    shape, tiles = w.shape, w.tiles
    params = synth.init_params(shape, seed=0)
    tokens = synth.token_stream(shape, seed=1)
    ref = _run(shape, tiles, params, tokens, L.TT_HOME_DEVICE, 0)
    got = _run(shape, tiles, params, tokens, L.TT_HOME_PINNED_HOST, budget_kib * 1024)
    assert got["loss"] == ref["loss"]
    for key in ("params", "grads", "m", "v"):
        for name in ref[key]:
            assert np.array_equal(got[key][name], ref[key][name]), (key, name)
    st = got["stats"]
    assert st["h2d_bytes"] > 0 and st["evictions"] > 0 and st["d2h_bytes"] > 0, st


def test_budget_smaller_than_a_tile_is_reported():
    w = synth.WORKLOADS["tiny"]
    shape, tiles = w.shape, w.tiles
    params = synth.init_params(shape, seed=0)
    tokens = synth.token_stream(shape, seed=1)
    with pytest.raises(L.TTError) as e:
        _run(shape, tiles, params, tokens, L.TT_HOME_PINNED_HOST, 1024, steps=1)
    assert e.value.code == L.TT_ERR_OOM
