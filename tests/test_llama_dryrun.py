"""CPU (dry-run) tests of the LLaMA-style step built from tile tasks: the
whole step's task graph is race free for several tilings, uses the LLaMA
ops (RMSNorm, rotary embedding forward and backward, SwiGLU forward and
backward, the token-only embedding) and none of GPT2's position or bias
tasks, and has the task counts the tiling implies."""
import pytest

import synth

tt = pytest.importorskip("tile_task_transformer_amd")
from tile_task_transformer_amd import _lib as L  # noqa: E402
from tile_task_transformer_amd.runtime import Context, GPT2  # noqa: E402
from tests.test_abi_dryrun import _check_races  # noqa: E402

SHAPE = synth.GPT2Shape(2, 100, 64, 4, 96, 32, 2)


def _dag(shape, tiles, tmp_path, n_micro=1, home=L.TT_HOME_DEVICE, budget=0):
    with Context(L.TT_DEVICE_DRYRUN, n_streams=4, window=100000, device_budget=budget) as ctx:
        model = GPT2(ctx, shape, tiles, family="llama", param_home=home)
        n_params = model.n_params
        model.step(None, n_micro=n_micro)
        n = model.task_count()
        dag = ctx.dump_dag(str(tmp_path / "dag.jsonl"))
        model.close()
    return n, n_params, dag


@pytest.mark.parametrize("tiles", [
    synth.Tiles(2, 32, 32, 32, 4, 32),     # one token tile, two embd tiles, ragged inner
    synth.Tiles(1, 8, 16, 40, 1, 40),      # split seq/head/batch, ragged inner and vocab
    synth.Tiles(2, 16, 64, 256, 2, 256),   # untiled embd/inner/vocab
])
def test_llama_step_dag_is_race_free(tiles, tmp_path):
    n, n_params, dag = _dag(SHAPE, tiles, tmp_path)
    assert n_params == 1 + 7 * SHAPE.n_layer + 2
    # the rotary table is filled once, at creation, before the step's tasks
    assert dag[0]["label"] == "rope_table" and n == len(dag) - 1
    _check_races(dag)
    by = {}
    for r in dag:
        by[r["label"]] = by.get(r["label"], 0) + 1
    for need in ("emb_fwd", "rms_fwd", "qkv", "rope", "attn_fwd", "attn_proj", "fc", "swiglu", "mlp_proj", "head",
                 "ce_merge", "ce_grad", "head_dw", "head_dx", "mlp_proj_dw", "mlp_proj_dx", "swiglu_bwd", "fc_dw",
                 "fc_dx", "rms_bwd", "attn_bwd", "rope_bwd", "qkv_dw", "qkv_dx", "adamw", "emb_dw"):
        assert need in by, need
    for absent in ("emb_dpos", "ln_fwd", "ln_bwd", "colsum"):
        assert absent not in by, absent
    nb, ns = SHAPE.batch // tiles.batch, SHAPE.seq // tiles.seq
    # the head's statistics: fused into its batched launch with one embd
    # tile, a separate pass after the per-vocab-tile long-K tasks with several
    ne = -(-SHAPE.n_embd // tiles.embd)
    assert ("ce_stats" in by) == (ne > 1)
    nh = SHAPE.n_head // tiles.head
    ntok = nb * ns
    assert by["rope"] == by["rope_bwd"] == SHAPE.n_layer * ntok * nh
    assert by["rms_fwd"] == by["rms_bwd"] == (2 * SHAPE.n_layer + 1) * ntok
    # every rotary task reads the table the creation task wrote
    table_id = dag[0]["id"]
    assert any(table_id in r["deps"] for r in dag if r["label"] == "rope")


def test_llama_accumulating_and_pinned_step_dags(tmp_path):
    """Two minibatches into one update, and pinned-host parameters under a
    small arena: both race free; the second minibatch doubles the forward and
    backward tasks but not the updates or the gradient zeroing."""
    tiles = synth.Tiles(1, 16, 32, 48, 2, 40)
    counts = []
    for n_micro in (1, 2):
        _, _, dag = _dag(SHAPE, tiles, tmp_path, n_micro=n_micro)
        _check_races(dag)
        counts.append({lab: sum(r["label"] == lab for r in dag) for lab in ("adamw", "fill", "rope", "head_dw")})
    one, two = counts
    assert two["adamw"] == one["adamw"] and two["fill"] == one["fill"]
    assert two["rope"] == 2 * one["rope"] and two["head_dw"] == 2 * one["head_dw"]
    _, _, dag = _dag(SHAPE, tiles, tmp_path, home=L.TT_HOME_PINNED_HOST, budget=1 << 20)
    _check_races(dag)


def test_llama_rejects_bad_shapes():
    with Context(L.TT_DEVICE_DRYRUN) as ctx:
        for shape, tiles in [(synth.GPT2Shape(1, 100, 66, 3, 96, 32, 2), synth.Tiles(2, 32, 66, 32, 3, 32)),
                             (synth.GPT2Shape(1, 100, 64, 4, 96, 32, 2), synth.Tiles(2, 32, 30, 32, 4, 32)),
                             (synth.GPT2Shape(1, 100, 64, 4, 96, 32, 2), synth.Tiles(2, 12, 32, 32, 4, 32))]:
            with pytest.raises(L.TTError) as e:
                GPT2(ctx, shape, tiles, family="llama")
            assert e.value.code in (L.TT_ERR_SHAPE, L.TT_ERR_UNSUPPORTED)


def test_llama_ops_through_tt_submit(tmp_path):
    """The LLaMA ops are reachable through the generic tt_submit with the
    access modes their documentation states."""
    import ctypes as C
    from tile_task_transformer_amd.runtime import Tensor
    with Context(L.TT_DEVICE_DRYRUN, n_streams=2) as ctx:
        x = Tensor(ctx, (2, 8, 2, 16), (2, 8, 2, 16))
        k = Tensor(ctx, (2, 8, 2, 16), (2, 8, 2, 16))
        tab = Tensor(ctx, (8, 16), (8, 16))
        a, b, h = (Tensor(ctx, (16, 24), (16, 24)) for _ in range(3))
        tiles = lambda *ts: (L.tt_tile * len(ts))(*[L.tt_tile(t.h, (C.c_int64 * L.TT_MAX_DIMS)()) for t in ts])  # noqa
        rope = L.tt_op_rope(0, 0, 10000.0)
        L.check(L.lib.tt_submit(ctx.h, L.TT_OP_ROPE_TABLE, tiles(tab), 1, C.byref(rope), C.sizeof(rope)))
        L.check(L.lib.tt_submit(ctx.h, L.TT_OP_ROPE, tiles(x, k, tab), 3, C.byref(rope), C.sizeof(rope)))
        L.check(L.lib.tt_submit(ctx.h, L.TT_OP_SWIGLU_FWD, tiles(a, b, h), 3, None, 0))
        L.check(L.lib.tt_submit(ctx.h, L.TT_OP_SWIGLU_BWD, tiles(h, a, b), 3, None, 0))
        bad = L.tt_op_rope(1, 0, 10000.0)  # positions 1..8 exceed the 8-row table
        assert L.lib.tt_submit(ctx.h, L.TT_OP_ROPE, tiles(x, tab), 2, C.byref(bad), C.sizeof(bad)) == L.TT_ERR_SHAPE
        dag = ctx.dump_dag(str(tmp_path / "ops.jsonl"))
    lab = [r["label"] for r in dag]
    assert lab == ["rope_table", "rope", "swiglu", "swiglu_bwd"]
    assert dag[1]["deps"] == [dag[0]["id"]]          # rope reads the table
    assert dag[3]["deps"] == [dag[2]["id"]]          # swiglu_bwd reads h, updates a and b after swiglu read them
