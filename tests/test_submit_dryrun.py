"""CPU tests of the generic task interface (tt_submit): a whole GPT2 step
written through it from Python (tests/submit_gpt2.py) in a dry-run context.
Checked: every op's access modes as the header states them, the edges the
executor derives against an independent reading of the sequential-task-flow
rule (a reader waits for the tile's last writer, a writer for the last
writer and every reader since), the absence of races over the whole step,
and the argument and shape errors of the interface."""
import ctypes as C

import pytest

import synth

pytest.importorskip("tile_task_transformer_amd")
from tile_task_transformer_amd import _lib as L  # noqa: E402
from tile_task_transformer_amd.runtime import Context  # noqa: E402
from tests.submit_gpt2 import SubmitGPT2  # noqa: E402
from tests.test_abi_dryrun import _check_races  # noqa: E402

R, W, RW = L.TT_R, L.TT_W, L.TT_RW
SHAPE = synth.GPT2Shape(2, 100, 64, 4, 96, 32, 2)
TILES = synth.Tiles(1, 16, 32, 48, 2, 40)   # 2 x 2 token tiles, 2 embd, 2 inner, 2 head, 3 vocab (ragged)


def stf_edges(dag):
    """The dependency rule applied to the dumped accesses, written out
    independently of the executor."""
    last_writer, readers, out = {}, {}, {}
    for r in dag:
        deps = set()
        for tid, lin, mode in r["acc"]:
            key = (tid, lin)
            if key in last_writer:
                deps.add(last_writer[key])
            if mode & W:
                deps.update(readers.get(key, ()))
                readers[key] = []
                last_writer[key] = r["id"]
            else:
                readers.setdefault(key, []).append(r["id"])
        out[r["id"]] = sorted(deps)
    return out


@pytest.fixture(scope="module")
def step_dag(tmp_path_factory):
    path = str(tmp_path_factory.mktemp("dag") / "submit.jsonl")
    with Context(L.TT_DEVICE_DRYRUN, n_streams=4, window=100000) as ctx:
        m = SubmitGPT2(ctx, SHAPE, TILES)
        m.submit_step(None)
        dag = ctx.dump_dag(path)
        ids = {id(t): i for i, t in enumerate(ctx._tensors)}  # tensor ids follow creation order
    return m, dag, ids


def test_step_edges_follow_the_stf_rule_and_are_race_free(step_dag):
    m, dag, _ = step_dag
    assert len(dag) == m.tasks > 0
    assert {r["id"]: sorted(r["deps"]) for r in dag} == stf_edges(dag)
    _check_races(dag)


def test_fused_head_step_edges_and_access_modes(tmp_path):
    """The same step with the head's last embd tile as one batched task
    carrying the cross-entropy statistics (TT_EPI_XSTATS): STF edges,
    race-free, and the task's access modes (logits written or updated,
    labels read, one partials tile per vocab tile written); the merge reads
    exactly those partials."""
    path = str(tmp_path / "fused.jsonl")
    with Context(L.TT_DEVICE_DRYRUN, n_streams=4, window=100000) as ctx:
        m = SubmitGPT2(ctx, SHAPE, TILES, fused_head=True)
        m.submit_step(None)
        dag = ctx.dump_dag(path)
        ids = {id(t): i for i, t in enumerate(ctx._tensors)}
    assert {r["id"]: sorted(r["deps"]) for r in dag} == stf_edges(dag)
    _check_races(dag)
    assert not [r for r in dag if r["label"] == "ce_stats"]
    heads = [r for r in dag if r["label"] == "gemm_batch_xstats"]
    assert len(heads) == m.nb * m.ns
    pid, zid, lid = ids[id(m.ce_parts)], ids[id(m.z)], ids[id(m.labels)]
    for r in heads:
        modes = {}
        for t, lin, md in r["acc"]:
            modes.setdefault(t, set()).add(md)
        assert modes[pid] == {W} and modes[lid] == {R} and modes[zid] == {RW}  # two embd tiles: beta = 1
        assert sum(t == pid for t, _, _ in r["acc"]) == m.NV
    merges = [r for r in dag if r["label"] == "ce_merge"]
    for r in merges:
        assert {(t, lin) for t, lin, md in r["acc"] if t == pid} <= {(t, lin) for h in heads for t, lin, _ in h["acc"]
                                                                      if t == pid}


def test_fused_head_argument_errors():
    with Context(L.TT_DEVICE_DRYRUN, n_streams=1) as ctx:
        A = ctx.tensor((64, 32), (64, 32))
        Bt = ctx.tensor((96, 32), (48, 32))
        Z = ctx.tensor((64, 96), (64, 48))
        lab = ctx.tensor((64,), (64,), L.TT_I32)
        parts = ctx.tensor((2, 64 * 3), (1, 64 * 3))
        sc = L.tt_op_gemm(0, 1, L.TT_EPI_XSTATS, 1.0, 0.0, 0)
        tl = [(A, (0, 0)), (Bt, (0, 0)), (Z, (0, 0)), (A, (0, 0)), (Bt, (1, 0)), (Z, (0, 1)), (lab, (0,)),
              (parts, (0, 0)), (parts, (1, 0))]
        ctx.submit(L.TT_OP_GEMM_BATCH, tl, sc)                                    # fine
        bad = [
            (tl[:3] + tl[6:8], L.tt_op_gemm(1, 1, L.TT_EPI_XSTATS, 1.0, 0.0, 0), L.TT_ERR_ARG),   # transA
            (tl[:3] + tl[6:8] + [tl[8]], sc, L.TT_ERR_ARG),                                        # tile count
            (tl[3:6] + tl[:3] + tl[6:], sc, L.TT_ERR_ARG),                                         # vocab order
            (tl[:3] + [(A, (0, 0)), (Bt, (1, 0)), (Z, (0, 1))] + [(A, (0, 0))] + tl[7:], sc, L.TT_ERR_ARG),  # labels f32
        ]
        for tiles, s, code in bad:
            with pytest.raises(L.TTError) as e:
                ctx.submit(L.TT_OP_GEMM_BATCH, tiles, s)
            assert e.value.code == code, e.value
        small = ctx.tensor((2, 3), (1, 3))
        with pytest.raises(L.TTError) as e:
            ctx.submit(L.TT_OP_GEMM_BATCH, tl[:7] + [(small, (0, 0)), (small, (1, 0))], sc)
        assert e.value.code == L.TT_ERR_SHAPE
        lse = ctx.tensor((64,), (64,))
        with pytest.raises(L.TTError) as e:   # 3 vocab tiles of 48 for vocab 96 would be 2
            ctx.submit(L.TT_OP_XENTROPY_MERGE, [(lse, (0,)), (lse, (0,)), (parts, (0, 0))],
                       L.tt_op_xe_groups(96, 48, 64))
        assert e.value.code == L.TT_ERR_ARG


def _modes(task, ids, tensors_and_tiles):
    """mode of each given (tensor, tile lin) in a task's dumped accesses."""
    acc = {(t, l): md for t, l, md in task["acc"]}
    return [acc.get((ids[id(t)], lin)) for t, lin in tensors_and_tiles]


def _lin(t, idx):
    grid = [-(-n // min(k, n)) for n, k in zip(t.shape, t.tile)]
    lin, mul = 0, 1
    for g, i in zip(grid, idx):
        lin += i * mul
        mul *= g
    return lin


def test_access_modes_of_each_op(step_dag):
    m, dag, ids = step_dag
    by = {}
    for r in dag:
        by.setdefault(r["label"], []).append(r)
    b0 = m.blk[0]
    # LayerNorm forward over the 2 embd tiles of token tile (0, 0): x, gamma, beta read; stats, y written
    ln = by["ln_fwd"][0]
    assert _modes(ln, ids, [(b0["h_in"], _lin(b0["h_in"], (0, 0, e))) for e in range(2)]) == [R, R]
    assert _modes(ln, ids, [(m.P["h0.ln1_g"], e) for e in range(2)]) == [R, R]
    assert _modes(ln, ids, [(b0["ln1"], 0)] + [(b0["n1"], _lin(b0["n1"], (0, 0, e))) for e in range(2)]) == [W] * 3
    # GEMM: beta 0 writes C, beta 1 updates it; GELU writes its pre-activation when beta == 0
    gem = by["gemm"]
    q0 = [r for r in gem if (ids[id(b0["q"])], _lin(b0["q"], (0, 0, 0, 0))) in {(a, b) for a, b, _ in r["acc"]}]
    assert [_modes(r, ids, [(b0["q"], _lin(b0["q"], (0, 0, 0, 0)))])[0] for r in q0] == [W, RW]
    fc_last = [r for r in gem if any(a == ids[id(b0["g"])] for a, _, _ in r["acc"])][0]
    assert _modes(fc_last, ids, [(b0["g"], 0), (b0["u"], 0)]) == [W, RW]  # beta 1 on the last embd tile: aux read too
    # attention forward: first key tile writes O and the running state, the last writes lse
    af = by["attn_fwd"]
    first_last = [r for r in af if len(r["acc"]) == 5]   # single (0, 0) tile pair: no running state
    assert first_last and all(_modes(r, ids, [(b0["lse"], r["acc"][-1][1])])[0] in (W, None) for r in first_last)
    # attention backward: dQ written for the first key tile, updated after
    ab = by["attn_bwd"]
    assert {md for r in ab for t, _, md in r["acc"] if t == ids[id(m.dq)]} == {W, RW}
    # cross-entropy: stats write partials, grad updates the logits in place
    assert {md for t, _, md in by["ce_stats"][0]["acc"] if t == ids[id(m.ce_parts)]} == {W}
    assert {md for t, _, md in by["ce_grad"][0]["acc"] if t == ids[id(m.z)]} == {RW}
    # AdamW: p, m, v updated, g and the bias corrections read
    ad = by["adamw"][0]
    name = "lnf_g"
    assert _modes(ad, ids, [(m.P[name], 0), (m.G[name], 0), (m.M[name], 0), (m.Vm[name], 0), (m.bc, 0)]) == \
        [RW, R, RW, RW, R]
    # LayerNorm backward: dgamma and dbeta accumulate, dx written (final LN) or updated (blocks)
    lb = by["ln_bwd"]
    assert {md for t, _, md in lb[0]["acc"] if t == ids[id(m.G["lnf_g"])]} == {RW}
    assert {md for r in lb for t, _, md in r["acc"] if t == ids[id(m.dh)]} == {W, RW}
    # embedding: forward reads every vocab tile of its column, backward updates them
    assert sum(t == ids[id(m.P["wte"])] for t, _, _ in by["emb_fwd"][0]["acc"]) == m.NV
    assert {md for t, _, md in by["emb_dw"][0]["acc"] if t == ids[id(m.G["wte"])]} == {RW}


def test_argument_and_shape_errors():
    with Context(L.TT_DEVICE_DRYRUN, n_streams=1) as ctx:
        A = ctx.tensor((64, 32), (32, 32))
        B = ctx.tensor((32, 48), (32, 16))
        Cc = ctx.tensor((64, 48), (32, 16))
        I32 = ctx.tensor((8,), (8,), L.TT_I32)
        g = L.tt_op_gemm(0, 0, 0, 1.0, 0.0, 0)
        ctx.submit(L.TT_OP_GEMM, [(A, (0, 0)), (B, (0, 0)), (Cc, (0, 0))], g)       # fine
        cases = [
            (L.TT_OP_GEMM, [(A, (0, 0)), (B, (0, 0))], g, L.TT_ERR_ARG),             # too few tiles
            (L.TT_OP_GEMM, [(A, (0, 0)), (A, (0, 0)), (Cc, (0, 0))], g, L.TT_ERR_SHAPE),
            (L.TT_OP_GEMM, [(A, (0, 0)), (B, (0, 0)), (Cc, (0, 0))], L.tt_op_fill(0.0), L.TT_ERR_ARG),  # scalars
            (L.TT_OP_GEMM, [(A, (2, 0)), (B, (0, 0)), (Cc, (0, 0))], g, L.TT_ERR_ARG),   # index out of range
            (L.TT_OP_FILL, [(I32, (0,))], L.tt_op_fill(0.0), L.TT_ERR_ARG),              # i32 tile
            (99, [(A, (0, 0))], None, L.TT_ERR_ARG),                                     # unknown op
            (L.TT_OP_GEMM, [(A, (0, 0)), (B, (0, 0)), (Cc, (0, 0))],
             L.tt_op_gemm(0, 0, L.TT_EPI_BIAS, 1.0, 0.0, 0), L.TT_ERR_ARG),              # bias tile missing
            (L.TT_OP_LAYERNORM_FWD, [(A, (0, 0))] * 4, L.tt_op_layernorm(1e-5, 0), L.TT_ERR_ARG),
        ]
        for op, tiles, sc, code in cases:
            with pytest.raises(L.TTError) as e:
                ctx.submit(op, tiles, sc)
            assert e.value.code == code, (op, e.value)
        # a null scalar pointer with a struct size, through the raw ABI
        arr = (L.tt_tile * 1)()
        arr[0].tensor = Cc.h
        assert L.lib.tt_submit(ctx.h, L.TT_OP_FILL, arr, 1, None, C.sizeof(L.tt_op_fill)) == L.TT_ERR_ARG
        assert ctx.stats()["tasks"] == 1


def test_gemm_chain_edges_through_submit(tmp_path):
    """K-split chain on one C tile, then an overwrite of an A tile the second
    product read: the same edges as with tt_submit_gemm."""
    with Context(L.TT_DEVICE_DRYRUN, n_streams=2) as ctx:
        A = ctx.tensor((64, 96), (64, 32))
        B = ctx.tensor((96, 64), (32, 64))
        Cc = ctx.tensor((64, 64), (64, 64))
        for kt in range(3):
            ctx.submit(L.TT_OP_GEMM, [(A, (0, kt)), (B, (kt, 0)), (Cc, (0, 0))],
                       L.tt_op_gemm(0, 0, 0, 1.0, 0.0 if kt == 0 else 1.0, 0))
        ctx.submit(L.TT_OP_FILL, [(A, (0, 1))], L.tt_op_fill(0.0))
        dag = ctx.dump_dag(str(tmp_path / "dag.jsonl"))
    assert {r["id"]: sorted(r["deps"]) for r in dag} == {0: [], 1: [0], 2: [1], 3: [1]}
