"""A GPT2 step written by a user through tt_submit (tests/submit_gpt2.py:
every layer as tasks over a few tiles, ungrouped) runs on the GPU and
matches the fp64 oracle's step: loss, every gradient, every updated weight
(same bar as the library's own step, tests/test_gpt2_gpu.py)."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import synth  # noqa: E402
from tile_task_transformer_amd.runtime import Context  # noqa: E402
from tests.submit_gpt2 import SubmitGPT2  # noqa: E402
from tests.test_gpt2_gpu import check_against_oracle  # noqa: E402

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("shape,tiles,fused", [
    (synth.GPT2Shape(2, 100, 64, 4, 96, 32, 2), synth.Tiles(1, 16, 32, 48, 2, 40), False),   # every axis split, ragged
    (synth.GPT2Shape(2, 100, 64, 4, 96, 32, 2), synth.Tiles(1, 16, 32, 48, 2, 40), True),    # head statistics fused
    (synth.WORKLOADS["tiny"].shape, synth.WORKLOADS["tiny"].tiles, False),
])
def test_user_built_step_matches_oracle(shape, tiles, fused):
    w = synth.WORKLOADS["tiny"]
    params = synth.init_params(shape, seed=0)
    tokens = synth.token_stream(shape, seed=1)
    with Context(0, n_streams=4, window=4096) as ctx:
        m = SubmitGPT2(ctx, shape, tiles, fused_head=fused)
        m.set_params(params)
        tok = torch.from_numpy(tokens.astype(np.int32)).cuda()
        ctx.wait_stream(torch.cuda.current_stream())
        m.submit_step(tok.data_ptr(), lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps, wd=w.weight_decay)
        ctx.wait()
        gpu = dict(loss=[m.loss_value()], grads=m.get(m.G), params=m.get(m.P))
        del tok
    check_against_oracle(shape, gpu, params, tokens, w)


def test_launch_error_is_latched():
    """A task whose launch fails (a rotary embedding of head dim 8, which no
    kernel covers: the submit-time checks pass, the launch refuses it) stops
    the window: wait reports that error, later submits and copies report the
    latched state, and destroying the context reports it once more and frees
    it."""
    from tile_task_transformer_amd import _lib as L
    ctx = Context(0, n_streams=2, window=64)
    a = ctx.tensor([4, 8], [4, 8])
    b = ctx.tensor([4, 8], [4, 8])
    x = ctx.tensor([1, 3, 2, 8], [1, 3, 2, 8])
    table = ctx.tensor([3, 8], [3, 8])
    for t in (a, b, x, table):
        t.copy_in(np.zeros(t.shape, np.float32))
    ctx.submit_fill(a, (0, 0), 1.0)
    ctx.submit(L.TT_OP_ROPE, [(x, (0, 0, 0, 0)), (table, (0, 0))], L.tt_op_rope(0, 0, 10000.0))
    ctx.submit_fill(b, (0, 0), 2.0)
    with pytest.raises(L.TTError) as e:
        ctx.wait()
    assert e.value.code == L.TT_ERR_ARG and "tile_rope" in str(e.value)
    with pytest.raises(L.TTError) as e:
        ctx.submit_fill(b, (0, 0), 3.0)
    assert e.value.code == L.TT_ERR_STATE
    with pytest.raises(L.TTError):
        a.copy_out()
    with pytest.raises(L.TTError) as e:
        ctx.close()
    assert e.value.code == L.TT_ERR_ARG and ctx.h is None
