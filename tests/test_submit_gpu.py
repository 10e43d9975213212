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
