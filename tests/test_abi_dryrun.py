"""CPU tests of the C ABI: the library loads and exports every symbol the
header declares, argument errors are reported, and the sequential-task-flow
executor infers exactly the read-after-write, write-after-read and
write-after-write edges (dry-run contexts launch nothing and need no GPU)."""
import ctypes as C
import os
import re

import pytest

import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tiletask.h")

tt = pytest.importorskip("tile_task_transformer_amd")
from tile_task_transformer_amd import _lib as L  # noqa: E402
from tile_task_transformer_amd.runtime import Context, GPT2  # noqa: E402


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**\s*((?:tt|tile)_\w+)\s*\(", src, flags=re.M)))


def test_every_declared_symbol_is_exported_and_bound():
    names = declared_functions()
    assert len(names) >= 40, names
    for n in names:
        assert hasattr(L.lib, n), n
        assert n in L.SIGNATURES, f"{n} has no ctypes signature"
    assert L.lib.tt_version().decode().startswith("tiletask")


def test_argument_errors_without_gpu():
    # validation happens on the host before any launch
    with pytest.raises(L.TTError) as e:
        tt.tile_gemm(None, 0, 0, -1, 4, 4, 1.0, 0, 4, 0, 4, 0.0, 0, 4)
    assert e.value.code == L.TT_ERR_ARG
    with pytest.raises(L.TTError) as e:
        tt.tile_attention_fwd(None, 1, 1, 8, 8, 48, 0, 0, 16, 16, 16, 16, 16, 16, 1, 1, 1.0)
    assert e.value.code == L.TT_ERR_UNSUPPORTED
    with pytest.raises(L.TTError) as e:
        tt.tile_layernorm_fwd(None, L.TT_LN_FUSED, 4, 4096, 16, 4096, 16, 16, None, 0, 0, 16, 16, 4096, 1e-5)
    assert e.value.code == L.TT_ERR_SHAPE
    # zero-size problems are no-ops
    tt.tile_gemm(None, 0, 0, 0, 4, 4, 1.0, None, 4, None, 4, 0.0, None, 4)
    tt.tile_fill(None, 0, None, 0.0)


def _edges(dag):
    return {r["id"]: sorted(r["deps"]) for r in dag}


def test_stf_hazard_edges(tmp_path):
    with Context(L.TT_DEVICE_DRYRUN, n_streams=2) as ctx:
        a = ctx.tensor((4, 4), (2, 2))
        b = ctx.tensor((4, 4), (2, 2))
        R, W, RW = L.TT_R, L.TT_W, L.TT_RW
        ctx.submit_nop("w0", [(a, (0, 0), W)])                      # 0
        ctx.submit_nop("r1", [(a, (0, 0), R)])                      # 1: RAW on 0
        ctx.submit_nop("r2", [(a, (0, 0), R), (b, (1, 0), W)])      # 2: RAW on 0
        ctx.submit_nop("w3", [(a, (0, 0), W)])                      # 3: WAW 0, WAR 1, 2
        ctx.submit_nop("r4", [(a, (1, 1), R)])                      # 4: independent tile
        ctx.submit_nop("rw5", [(a, (0, 0), RW), (a, (1, 1), R)])    # 5: RAW/WAW on 3; R-R with 4 is free
        ctx.submit_nop("w6", [(a, (1, 1), W)])                      # 6: WAR on 4 and 5
        ctx.submit_nop("r7", [(b, (1, 0), R), (b, (1, 0), W)])      # 7: duplicate access merges to RW: on 2
        ctx.submit_nop("none", [])                                  # 8: no accesses
        dag = ctx.dump_dag(str(tmp_path / "dag.jsonl"))
    e = _edges(dag)
    assert e == {0: [], 1: [0], 2: [0], 3: [0, 1, 2], 4: [], 5: [3], 6: [4, 5], 7: [2], 8: []}
    labels = [r["label"] for r in dag]
    assert labels[:3] == ["w0", "r1", "r2"]


def test_stream_assignment_keeps_chains_and_spreads_independent_work(tmp_path):
    with Context(L.TT_DEVICE_DRYRUN, n_streams=4) as ctx:
        a = ctx.tensor((8,), (1,))
        W, RW, R = L.TT_W, L.TT_RW, L.TT_R
        for i in range(4):                     # 4 independent writers
            ctx.submit_nop("w", [(a, (i,), W)])
        for i in range(4):                     # each continues its own chain
            ctx.submit_nop("rw", [(a, (i,), RW)])
        ctx.submit_nop("join", [(a, (i,), R) for i in range(4)] + [(a, (7,), W)])
        dag = ctx.dump_dag(str(tmp_path / "dag.jsonl"))
        st = ctx.stats()
    s = [r["stream"] for r in dag]
    assert sorted(s[:4]) == [0, 1, 2, 3]
    assert s[4:8] == s[:4]                     # chain continuation stays on its stream
    assert st["cross_stream_waits"] == 3       # the join waits on the three other streams
    assert st["tasks"] == 9 and st["edges"] == 4 + 4


def test_streams_active_narrows_the_assignment(tmp_path):
    with Context(L.TT_DEVICE_DRYRUN, n_streams=4) as ctx:
        a = ctx.tensor((8,), (1,))
        for i in range(4):
            ctx.submit_nop("w", [(a, (i,), L.TT_W)])
        ctx.streams_active(1)
        for i in range(4):                     # chains from streams 1..3 cannot continue there
            ctx.submit_nop("rw", [(a, (i,), L.TT_RW)])
        ctx.streams_active(2)
        for i in range(4, 8):
            ctx.submit_nop("w2", [(a, (i,), L.TT_W)])
        with pytest.raises(L.TTError):
            ctx.streams_active(5)
        with pytest.raises(L.TTError):
            ctx.streams_active(0)
        dag = ctx.dump_dag(str(tmp_path / "dag.jsonl"))
    s = [r["stream"] for r in dag]
    assert sorted(s[:4]) == [0, 1, 2, 3]
    assert s[4:8] == [0, 0, 0, 0]
    assert sorted(s[8:]) == [0, 0, 1, 1]


def test_heavy_lane_puts_large_tasks_in_order_on_stream_zero(tmp_path):
    with Context(L.TT_DEVICE_DRYRUN, n_streams=4) as ctx:
        ctx.heavy_lane(1e6)
        A = ctx.tensor((256, 256), (128, 128))
        a = ctx.tensor((8,), (1,))
        C = ctx.tensor((256, 256), (128, 128))
        for i in range(2):                     # 2*128^3 flops each: heavy
            for j in range(2):
                ctx.submit_gemm(0, 0, 1.0, A, (i, 0), A, (0, j), 0.0, C, (i, j))
        for i in range(6):                     # light, independent
            ctx.submit_nop("w", [(a, (i,), L.TT_W)])
        ctx.submit_nop("rd", [(C, (0, 0), L.TT_R)])  # light reader of a heavy result
        with pytest.raises(L.TTError):
            ctx.heavy_lane(-1.0)
        dag = ctx.dump_dag(str(tmp_path / "dag.jsonl"))
    s = [r["stream"] for r in dag]
    assert s[:4] == [0, 0, 0, 0]
    assert all(x in (1, 2, 3) for x in s[4:])
    assert sorted(s[4:10]) == [1, 1, 2, 2, 3, 3]


def test_ksplit_gemm_chain_edges(tmp_path):
    with Context(L.TT_DEVICE_DRYRUN, n_streams=2) as ctx:
        A = ctx.tensor((64, 96), (64, 32))    # 3 K tiles
        B = ctx.tensor((96, 64), (32, 64))
        Cc = ctx.tensor((64, 64), (64, 64))
        for kt in range(3):
            ctx.submit_gemm(0, 0, 1.0, A, (0, kt), B, (kt, 0), 0.0 if kt == 0 else 1.0, Cc, (0, 0))
        ctx.submit_fill(A, (0, 1), 0.0)       # overwrites a tile the second GEMM read
        with pytest.raises(L.TTError) as e:   # shape mismatch is rejected at submit time
            ctx.submit_gemm(0, 0, 1.0, A, (0, 0), A, (0, 1), 0.0, Cc, (0, 0))
        assert e.value.code == L.TT_ERR_SHAPE
        dag = ctx.dump_dag(str(tmp_path / "dag.jsonl"))
    assert _edges(dag) == {0: [], 1: [0], 2: [1], 3: [1]}


def _check_races(dag):
    """Every pair of accesses to one tile where at least one writes must be
    ordered by a path of dependency edges (STF as the race model)."""
    n = len(dag)
    ids = [r["id"] for r in dag]
    pos = {t: i for i, t in enumerate(ids)}
    reach = [0] * n   # bitset of ancestors
    for i, r in enumerate(dag):
        m = 0
        for d in r["deps"]:
            assert d < r["id"], "edge must point to an earlier task"
            j = pos[d]
            m |= reach[j] | (1 << j)
        reach[i] = m
    last = {}
    for i, r in enumerate(dag):
        for tid, lin, mode in r["acc"]:
            key = (tid, lin)
            for j, m2 in last.get(key, []):
                if (mode & 2) or (m2 & 2):
                    assert (reach[i] >> j) & 1, f"race on tile {key} between {dag[j]['label']} and {r['label']}"
            last.setdefault(key, []).append((i, mode))


@pytest.mark.parametrize("tiles", [
    synth.Tiles(2, 32, 32, 32, 4, 32),     # the tiny workload's tiles
    synth.Tiles(1, 8, 16, 24, 1, 40),      # ragged embd/inner/vocab, split seq/head/batch
    synth.Tiles(2, 16, 64, 256, 2, 256),   # untiled embd/inner/vocab
])
def test_gpt2_step_dag_is_race_free(tiles, tmp_path):
    shape = synth.GPT2Shape(2, 100, 64, 4, 96, 32, 2)
    with Context(L.TT_DEVICE_DRYRUN, n_streams=4, window=100000) as ctx:
        model = GPT2(ctx, shape, tiles)
        model.step(None)
        n = model.task_count()
        dag = ctx.dump_dag(str(tmp_path / "dag.jsonl"))
        model.close()
    assert n == len(dag) > 0
    _check_races(dag)
    labels = {r["label"] for r in dag}
    for need in ("emb_fwd", "qkv", "attn_fwd", "attn_proj", "fc", "mlp_proj", "head", "ce_merge",
                 "ce_loss", "ce_grad", "head_dw", "head_dx", "attn_bwd", "adamw", "emb_dw", "emb_dpos"):
        assert need in labels, need
    label_of = {r["id"]: r["label"] for r in dag}
    merges = [r for r in dag if r["label"] == "ce_merge"]
    ne = -(-shape.n_embd // tiles.embd)
    nv = -(-shape.vocab // tiles.vocab)
    ntok = (shape.batch // tiles.batch) * (shape.seq // tiles.seq)
    heads = sum(1 for r in dag if r["label"] == "head")
    if ne == 1:
        # one embd tile: the cross-entropy statistics come from the head's
        # batched launch (its epilogue), not from a separate pass over the
        # logits: every merge reads partials that a head task wrote
        assert "ce_stats" not in labels
        assert merges and all(any(label_of[d] == "head" for d in r["deps"]) for r in merges)
    else:
        # several embd tiles: one long-K head task per (token tile, vocab
        # tile), then the statistics pass, which the merge reads
        assert heads == ntok * nv
        assert merges and all(any(label_of[d] == "ce_stats" for d in r["deps"]) for r in merges)


def test_gpt2_accumulating_step_dag_is_race_free(tmp_path):
    """Two minibatches into one update: race free, twice the forward and
    backward tasks, AdamW tasks once, and no gradient is zeroed twice."""
    shape = synth.GPT2Shape(2, 100, 64, 4, 96, 32, 2)
    tiles = synth.Tiles(1, 16, 32, 48, 2, 40)
    counts = []
    for n_micro in (1, 2):
        with Context(L.TT_DEVICE_DRYRUN, n_streams=4, window=100000) as ctx:
            model = GPT2(ctx, shape, tiles)
            model.step(None, n_micro=n_micro)
            dag = ctx.dump_dag(str(tmp_path / f"dag{n_micro}.jsonl"))
            model.close()
        _check_races(dag)
        counts.append({lab: sum(r["label"] == lab for r in dag) for lab in ("adamw", "adam_step", "fill", "qkv",
                                                                            "head_dw", "ce_loss")})
    one, two = counts
    assert two["adamw"] == one["adamw"] and two["adam_step"] == one["adam_step"] == 1
    assert two["fill"] == one["fill"]
    for lab in ("qkv", "head_dw", "ce_loss"):
        assert two[lab] == 2 * one[lab], lab
    with Context(L.TT_DEVICE_DRYRUN, n_streams=2) as ctx:
        model = GPT2(ctx, shape, tiles)
        with pytest.raises(L.TTError):
            model.step(None, n_micro=0)
        model.close()


def test_gpt2_sgd_step_dag(tmp_path):
    """The SGD update: race free, one sgd task per AdamW task of the AdamW
    step, no moment or step-counter task; an unknown optimizer is refused."""
    shape = synth.GPT2Shape(2, 100, 64, 4, 96, 32, 2)
    tiles = synth.Tiles(1, 16, 32, 48, 2, 40)
    counts = {}
    for opt in ("adamw", "sgd"):
        with Context(L.TT_DEVICE_DRYRUN, n_streams=4, window=100000) as ctx:
            model = GPT2(ctx, shape, tiles)
            model.step(None, optimizer=opt)
            dag = ctx.dump_dag(str(tmp_path / f"dag_{opt}.jsonl"))
            model.close()
        _check_races(dag)
        counts[opt] = {lab: sum(r["label"] == lab for r in dag) for lab in ("adamw", "adam_step", "sgd")}
    assert counts["sgd"]["sgd"] == counts["adamw"]["adamw"] > 0
    assert counts["sgd"]["adamw"] == counts["sgd"]["adam_step"] == 0
    with Context(L.TT_DEVICE_DRYRUN, n_streams=2) as ctx:
        model = GPT2(ctx, shape, tiles)
        hp = L.tt_adamw_hparams(3e-4, 0.9, 0.999, 1e-8, 0.1, 3e-4, 1, 7)
        import ctypes as C
        assert L.lib.tt_gpt2_step_accum(model.h, None, 1, C.byref(hp), 1) == L.TT_ERR_ARG
        model.close()


def test_gpt2_rejects_bad_tiles():
    shape = synth.GPT2Shape(1, 100, 64, 4, 96, 32, 2)
    with Context(L.TT_DEVICE_DRYRUN) as ctx:
        for bad in (synth.Tiles(2, 12, 32, 32, 4, 32),   # seq tile does not divide seq
                    synth.Tiles(2, 32, 32, 32, 3, 32),   # head tile does not divide heads
                    synth.Tiles(3, 32, 32, 32, 4, 32)):  # batch tile does not divide batch
            with pytest.raises(L.TTError) as e:
                GPT2(ctx, shape, bad)
            assert e.value.code == L.TT_ERR_SHAPE


def test_out_of_core_wide_model_step_dag(tmp_path):
    """The 26.6 B-parameter out-of-core model (8 blocks, d 16384, inner
    65536, vocab 50257, batch 2) with parameters, gradients and moments in
    pinned host RAM, built as a dry run: the whole step's task graph is
    race free, with the task count the tiling implies."""
    w = synth.WORKLOADS["wide8_ooc"]
    with Context(L.TT_DEVICE_DRYRUN, n_streams=1, window=1 << 20) as ctx:
        model = GPT2(ctx, w.shape, w.tiles, param_home=L.TT_HOME_PINNED_HOST)
        model.step(None)
        n = model.task_count()
        dag = ctx.dump_dag(str(tmp_path / "ooc.jsonl"))
        model.close()
    assert n == len(dag)
    _check_races(dag)
    by = {}
    for r in dag:
        by[r["label"]] = by.get(r["label"], 0) + 1
    # 8 embd tiles, 8 inner tiles, 8 head tiles, 25 vocab tiles, one token tile
    assert by["attn_fwd"] == by["attn_bwd"] == 8 * 8
    assert by["ln_fwd"] == 2 * 8 + 1 and by["ln_bwd"] == 2 * 8 + 1
    assert by["head_dx"] == 8 and by["emb_dw"] == 8 * 25  # pinned table: one task per vocab tile



def test_priorities_launch_the_critical_path_first(tmp_path):
    """With critical-path priorities a window is launched as a list
    schedule: a light task that nothing waits for goes after the heavy chain
    that was submitted behind it; the order stays topological."""
    orders = {}
    for on in (False, True):
        with Context(L.TT_DEVICE_DRYRUN, n_streams=2) as ctx:
            ctx.priorities(on)
            x = ctx.tensor((64, 64), (64, 64))
            y = ctx.tensor((256, 256), (256, 256))
            w = ctx.tensor((256, 256), (256, 256))
            z = ctx.tensor((256, 256), (256, 256))
            ctx.submit_fill(x, (0, 0), 1.0)                                    # 0: light, no successor
            ctx.submit_fill(y, (0, 0), 1.0)                                    # 1: light, feeds the GEMM
            ctx.submit_gemm(0, 0, 1.0, y, (0, 0), w, (0, 0), 0.0, z, (0, 0))  # 2: heavy, after 1
            dag = ctx.dump_dag(str(tmp_path / f"p{int(on)}.jsonl"))
        orders[on] = [r["id"] for r in dag]
    assert orders[False] == [0, 1, 2]
    assert orders[True] == [1, 2, 0]


@pytest.mark.parametrize("tiles", [synth.Tiles(1, 8, 16, 24, 1, 40), synth.Tiles(2, 16, 32, 48, 2, 40)])
def test_priority_order_of_a_gpt2_step_is_a_race_free_topological_order(tiles, tmp_path):
    shape = synth.GPT2Shape(2, 100, 64, 4, 96, 32, 2)
    dags = {}
    for on in (False, True):
        with Context(L.TT_DEVICE_DRYRUN, n_streams=4, window=100000) as ctx:
            ctx.priorities(on)
            model = GPT2(ctx, shape, tiles)
            model.step(None)
            dags[on] = ctx.dump_dag(str(tmp_path / f"s{int(on)}.jsonl"))
            model.close()
    base, prio = dags[False], dags[True]
    assert sorted(r["id"] for r in prio) == [r["id"] for r in base]
    assert [r["id"] for r in prio] != [r["id"] for r in base]   # the order did change
    seen = set()
    for r in prio:
        assert all(d in seen for d in r["deps"]), r["label"]
        seen.add(r["id"])
    # same tasks, same edges, same streams
    by_id = {r["id"]: r for r in base}
    for r in prio:
        assert r["deps"] == by_id[r["id"]]["deps"] and r["stream"] == by_id[r["id"]]["stream"]
    _check_races(prio)


def test_caller_streams_need_a_device():
    """tt_ctx_create_on_streams refuses the dry-run device and a null stream
    array before touching any GPU."""
    with pytest.raises(L.TTError) as e:
        Context(L.TT_DEVICE_DRYRUN, streams=[1, 2])
    assert e.value.code == L.TT_ERR_ARG and "needs a device" in str(e.value)
    h = C.c_void_p()
    assert L.lib.tt_ctx_create_on_streams(0, 2, None, 0, 0, C.byref(h)) == L.TT_ERR_ARG
