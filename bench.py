"""Benchmark: one GPT2 training step (forward + backward + AdamW) as tile
tasks on one MI355X, GPT2-small shape (12 blocks, d 768, 12 heads, inner
3072, vocab 50257, seq 1024, batch 4) with the NNTile README's example tiles
(seq 1024, embd 768, inner 3072, head 12, batch 4; vocab tile 768).

Prints ONE JSON line:
  value        tokens/s of the whole step (inputs resident in HBM)
  tflops       model TFLOP/s = 3 x forward matmul flops (causal attention
               counted over T(T+1)/2 pairs) / step time; mfma_frac = / 157.3
  roofline     the dominant tile kernel: algorithmic flops per launch /
               its average launch duration, timed with HIP events on the
               executor stream that launches it, during the timed steps
  cpu_baseline the fp64 oracle step timed on this host's cores on a bounded
               sample (one of the batch's sequences), scaled to tokens/s
Usage: python bench.py [--gpus 1] [--steps 10] [--warmup 3]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "GPT2 train tokens/sec + TFLOP/s (% fp32 MFMA peak) per fwd+bwd+AdamW step, 1 GPU"
MFMA_FP32_PEAK = 157.3  # TFLOP/s, MI355X dense fp32 matrix
HBM_PEAK = 8000.0       # GB/s
GEMM_LABELS = ("qkv", "attn_proj", "fc", "mlp_proj", "head", "head_dw", "head_dx", "mlp_proj_dw", "mlp_proj_dx",
               "fc_dw", "fc_dx", "attn_proj_dw", "attn_proj_dx", "qkv_dw", "qkv_dx")


def model_flops(s) -> float:
    n = s.batch * s.seq
    per_block = 2 * n * s.n_embd * (3 * s.n_embd + s.n_embd + 2 * s.n_inner)
    attn = 2 * 2 * s.batch * s.n_embd * (s.seq * (s.seq + 1) // 2)
    head = 2 * n * s.n_embd * s.vocab
    return 3.0 * (s.n_layer * (per_block + attn) + head)


def gemm_launch_flops(label, s, t) -> float:
    """Algorithmic flops of one launch of a GEMM task class (2*m*n*k)."""
    rows = t.batch * t.seq
    et, it, vt = min(t.embd, s.n_embd), min(t.inner, s.n_inner), min(t.vocab, s.vocab)
    hw = t.head * (s.n_embd // s.n_head)
    table = {
        "qkv": (rows, hw, et), "attn_proj": (rows, et, hw), "fc": (rows, it, et), "mlp_proj": (rows, et, it),
        "head": (rows, vt, et), "head_dx": (rows, et, vt), "head_dw": (vt, et, rows),
        "mlp_proj_dw": (it, et, rows), "mlp_proj_dx": (rows, it, et), "fc_dw": (et, it, rows),
        "fc_dx": (rows, et, it), "attn_proj_dw": (hw, et, rows), "attn_proj_dx": (rows, hw, et),
        "qkv_dw": (et, hw, rows), "qkv_dx": (rows, et, hw),
    }
    m, n, k = table[label]
    return 2.0 * m * n * k


GEMM_SHAPES = {  # label -> (transA, transB, m, n, k, epilogue, beta) in tile terms
    "qkv": lambda r, e, i, h, v: (0, 0, r, h, e, 1, 0.0), "attn_proj": lambda r, e, i, h, v: (0, 0, r, e, h, 3, 0.0),
    "fc": lambda r, e, i, h, v: (0, 0, r, i, e, 5, 0.0), "mlp_proj": lambda r, e, i, h, v: (0, 0, r, e, i, 3, 0.0),
    "head": lambda r, e, i, h, v: (0, 1, r, v, e, 0, 0.0), "head_dw": lambda r, e, i, h, v: (1, 0, v, e, r, 0, 1.0),
    "head_dx": lambda r, e, i, h, v: (0, 0, r, e, v, 0, 1.0),
    "mlp_proj_dw": lambda r, e, i, h, v: (1, 0, i, e, r, 0, 0.0),
    "mlp_proj_dx": lambda r, e, i, h, v: (0, 1, r, i, e, 8, 0.0),
    "fc_dw": lambda r, e, i, h, v: (1, 0, e, i, r, 0, 0.0), "fc_dx": lambda r, e, i, h, v: (0, 1, r, e, i, 0, 0.0),
    "attn_proj_dw": lambda r, e, i, h, v: (1, 0, h, e, r, 0, 0.0),
    "attn_proj_dx": lambda r, e, i, h, v: (0, 1, r, h, e, 0, 0.0),
    "qkv_dw": lambda r, e, i, h, v: (1, 0, e, h, r, 0, 0.0), "qkv_dx": lambda r, e, i, h, v: (0, 1, r, e, h, 0, 1.0),
}


def tile_classes(w, reps=20):
    """Each tile-op class of the workload, launched alone on one stream at its
    task shape; HIP-event time per launch against its roofline."""
    import math

    import torch

    import tile_task_transformer_amd as tt
    s, t = w.shape, w.tiles
    r = t.batch * t.seq
    e, i, v = min(t.embd, s.n_embd), min(t.inner, s.n_inner), min(t.vocab, s.vocab)
    hd = s.n_embd // s.n_head
    h = t.head * hd
    st = torch.cuda.current_stream()
    gen = torch.Generator(device="cuda").manual_seed(0)
    rnd = lambda *shape: torch.randn(*shape, device="cuda", generator=gen)  # noqa: E731

    def timed(fn):
        for _ in range(3):
            fn()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(st)
        for _ in range(reps):
            fn()
        b.record(st)
        b.synchronize()
        return a.elapsed_time(b) / reps

    out = {}
    for label, f in GEMM_SHAPES.items():
        ta, tb, m, n, k, epi, beta = f(r, e, i, h, v)
        A = rnd(k, m) if ta else rnd(m, k)
        B = rnd(n, k) if tb else rnd(k, n)
        C, aux, bias = rnd(m, n), rnd(m, n), rnd(n)
        res = rnd(m, n) if epi & 2 else None
        nws = tt.tile_gemm_workspace(m, n, k)
        ws = torch.empty(max(nws // 4, 1), device="cuda")
        ms = timed(lambda: tt.tile_gemm_ws(st, ta, tb, m, n, k, 1.0, A, A.shape[1], B, B.shape[1], beta, C, n, epi,
                                           bias, res, n if res is not None else 0, aux, n, ws, nws))
        tf = 2.0 * m * n * k / (ms * 1e-3) / 1e12
        out[label] = {"bound": "mfma", "shape": [m, n, k, ta, tb], "us": round(ms * 1e3, 1),
                      "achieved": round(tf, 2), "unit": "TFLOP/s", "frac": round(tf / MFMA_FP32_PEAK, 4)}
    # attention (per (batch tile, head tile) pair of the workload's seq tile)
    Q, K, V = rnd(t.batch, t.seq, t.head, hd), rnd(t.batch, t.seq, t.head, hd), rnd(t.batch, t.seq, t.head, hd)
    O, dO = torch.empty_like(Q), rnd(t.batch, t.seq, t.head, hd)
    lse, Dv = torch.empty(t.batch * t.head * t.seq, device="cuda"), torch.empty(t.batch * t.head * t.seq, device="cuda")
    dQ, dK, dV = torch.empty_like(Q), torch.empty_like(Q), torch.empty_like(Q)
    sc = 1 / math.sqrt(hd)
    fl = 2 * 2 * t.batch * t.head * hd * (t.seq * (t.seq + 1) // 2)
    ms = timed(lambda: tt.tile_attention_fwd(st, t.batch, t.head, t.seq, t.seq, hd, 0, 0, Q, K, V, O, None, lse, 1, 1,
                                             sc))
    out["attn_fwd"] = {"bound": "mfma", "us": round(ms * 1e3, 1), "achieved": round(fl / ms / 1e9, 2),
                       "unit": "TFLOP/s (model)", "frac": round(fl / ms / 1e9 / MFMA_FP32_PEAK, 4)}
    ms = timed(lambda: tt.tile_attention_bwd(st, tt.TT_ATT_GRAD, t.batch, t.head, t.seq, t.seq, hd, 0, 0, Q, K, V,
                                             None, dO, lse, Dv, dQ, dK, dV, 0, 0, sc))
    out["attn_bwd"] = {"bound": "mfma", "us": round(ms * 1e3, 1), "achieved": round(2.5 * fl / ms / 1e9, 2),
                       "unit": "TFLOP/s (model)", "frac": round(2.5 * fl / ms / 1e9 / MFMA_FP32_PEAK, 4)}

    def hbm(label, nbytes, fn):
        ms = timed(fn)
        gbs = nbytes / (ms * 1e-3) / 1e9
        out[label] = {"bound": "hbm", "us": round(ms * 1e3, 1), "bytes": nbytes, "achieved": round(gbs, 1),
                      "unit": "GB/s", "frac": round(gbs / HBM_PEAK, 4)}

    x, y, g_, b_ = rnd(r, e), torch.empty(r, e, device="cuda"), rnd(e), rnd(e)
    stats = torch.empty(r, 2, device="cuda")
    hbm("ln_fwd", 8 * r * e, lambda: tt.tile_layernorm_fwd(st, tt.TT_LN_FUSED, r, e, x, e, g_, b_, None, 0, 0, stats,
                                                           y, e, 1e-5))
    dx, dg, db = rnd(r, e), torch.zeros(e, device="cuda"), torch.zeros(e, device="cuda")
    lws = torch.empty(tt.tile_layernorm_bwd_workspace(r, e) // 4 + 1, device="cuda")
    hbm("ln_bwd", 16 * r * e, lambda: tt.tile_layernorm_bwd(st, tt.TT_LN_FUSED, r, e, e, y, e, x, e, g_, stats, None,
                                                            0, 0, dx, e, 1, dg, db, lws))
    z = rnd(r, v)
    lab = torch.randint(0, v, (r,), device="cuda", dtype=torch.int32)
    parts = torch.empty(r, 3, device="cuda")
    hbm("ce_stats", 4 * r * v, lambda: tt.tile_softmax(st, tt.TT_SM_STATS, r, v, 0, 0, 1.0, 0, z, v, lab, parts, 0, 0,
                                                       None, None, None, 0, 1.0))
    lse_r = torch.zeros(r, device="cuda") + 10.0
    hbm("ce_grad", 8 * r * v, lambda: tt.tile_xentropy(st, tt.TT_XE_GRAD, r, v, 0, lab, z, v, lse_r, None, None, 0,
                                                       1.0 / r))
    n_ad = i * e
    p, gr, m_, v_ = rnd(n_ad), rnd(n_ad), torch.zeros(n_ad, device="cuda"), torch.zeros(n_ad, device="cuda")
    bc = torch.tensor([0.1, 0.001], device="cuda")
    hbm("adamw", 28 * n_ad, lambda: tt.tile_fused_adamw(st, n_ad, p, gr, m_, v_, 3e-4, 0.9, 0.999, 1e-8, 0.1, bc))
    xr = rnd(r, i)
    outc = torch.zeros(i, device="cuda")
    rws = torch.empty(tt.tile_reduce_rows_workspace(r, i) // 4 + 1, device="cuda")
    hbm("colsum", 4 * r * i, lambda: tt.tile_reduce_rows(st, r, i, xr, i, outc, 1, rws))
    return out


def cpu_baseline(w, params, tokens):
    """The fp64 oracle on the host, one sequence of the batch (bounded sample)."""
    import numpy as np
    from oracle import gpt2 as og
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:  # noqa: BLE001
        cores = 1
    sample = np.asarray(tokens[:1], np.int64)
    t0 = time.perf_counter()
    og.step(params, sample, w.shape.n_layer, w.shape.n_head, lr=w.lr, wd=w.weight_decay)
    dt = time.perf_counter() - t0
    return {"value": round(w.shape.seq / dt, 2), "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "sample": f"one {w.shape.seq}-token sequence of the batch (1 of {w.shape.batch}), full model fwd+bwd+AdamW "
                      f"in fp64 numpy, {dt:.1f} s"}


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="gpt2_small")
    ap.add_argument("--streams", type=int, default=4)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--breakdown", default=os.path.join("gpurun_out", "bench_breakdown.json"),
                    help="per-task-class GPU times of one extra profiled step ('' = skip)")
    ap.add_argument("--tile-classes", default="",
                    help="instead of the step: time each tile-op class alone and write this JSON file")
    a = ap.parse_args(argv)
    if a.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (--gpus must be 1)", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import synth
    from tile_task_transformer_amd.runtime import Context, GPT2

    w = synth.WORKLOADS[a.workload]
    if a.tile_classes:
        res = tile_classes(w)
        os.makedirs(os.path.dirname(a.tile_classes) or ".", exist_ok=True)
        with open(a.tile_classes, "w") as f:
            json.dump(res, f, indent=1)
        for k, v in res.items():
            print(f"{k:14s} {v['us']:9.1f} us  {v['achieved']:8.1f} {v['unit']:16s} {100 * v['frac']:5.1f}%",
                  file=sys.stderr)
        return 0
    s, t = w.shape, w.tiles
    specs = synth.param_specs(s)
    params = synth.init_params(s, seed=0)
    tokens = synth.token_stream(s, seed=1)
    ctx = Context(0, n_streams=a.streams, window=4096)
    model = GPT2(ctx, s, t)
    model.set_params(params, specs)
    tok = torch.from_numpy(tokens.astype(np.int32)).cuda()
    hp = dict(lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps, weight_decay=w.weight_decay)

    for _ in range(a.warmup):
        model.step(tok, **hp)
    loss0 = model.loss()
    print(f"[bench] warmup done, loss {loss0:.4f}, {model.task_count()} tasks/step", file=sys.stderr, flush=True)

    breakdown = {}
    if a.breakdown:
        ctx.profile("*")
        model.step(tok, **hp)
        breakdown = ctx.profile_take()
        ctx.profile(None)
        os.makedirs(os.path.dirname(a.breakdown) or ".", exist_ok=True)
        with open(a.breakdown, "w") as f:
            json.dump(breakdown, f, indent=1, sort_keys=True)
    gemm_times = {k: v["total_ms"] for k, v in breakdown.items() if k in GEMM_LABELS}
    dominant = max(gemm_times, key=gemm_times.get) if gemm_times else "fc"

    # timed region: K steps back to back, the dominant GEMM class bracketed by events
    ctx.profile(dominant)
    ctx.reset_stats()
    torch.cuda.synchronize()
    ctx.wait()
    t0 = time.perf_counter()
    for _ in range(a.steps):
        model.step(tok, **hp)
    ctx.wait()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    loss = model.loss()
    prof = ctx.profile_take().get(dominant, {})
    ctx.profile(None)
    st = ctx.stats()

    ms = 1e3 * elapsed / a.steps
    tok_s = s.batch * s.seq / (elapsed / a.steps)
    tflops = model_flops(s) / (elapsed / a.steps) / 1e12
    per_launch = gemm_launch_flops(dominant, s, t)
    avg_ms = prof["total_ms"] / prof["count"] if prof.get("count") else float("nan")
    achieved = per_launch / (avg_ms * 1e-3) / 1e12
    out = {
        "metric": METRIC, "value": round(tok_s, 1), "unit": "tokens/s", "n_gpus": 1, "steps": a.steps,
        "warmup": a.warmup, "ms_per_step": round(ms, 3), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": a.workload, "global_batch": s.batch, "seq_len": s.seq, "n_layer": s.n_layer,
                   "n_embd": s.n_embd, "vocab": s.vocab,
                   "tiles": {"batch": t.batch, "seq": t.seq, "embd": t.embd, "inner": t.inner, "head": t.head,
                             "vocab": t.vocab}, "streams": a.streams},
        "tflops": round(tflops, 2), "mfma_frac": round(tflops / MFMA_FP32_PEAK, 4),
        "tasks_per_step": model.task_count(), "loss": round(loss, 5),
        "host_submit_ms_per_step": round(1e3 * st["submit_seconds"] / a.steps, 3),
        "roofline": {"bound": "mfma", "kernel": f"tile_gemm[{dominant}]", "achieved": round(achieved, 2),
                     "peak": MFMA_FP32_PEAK, "unit": "TFLOP/s", "frac": round(achieved / MFMA_FP32_PEAK, 4),
                     "traffic": None, "flops_per_launch": per_launch, "avg_launch_ms": round(avg_ms, 4),
                     "launches": prof.get("count", 0)},
    }
    print(f"[bench] timed {a.steps} steps: {ms:.2f} ms/step, {tok_s:.0f} tokens/s, {tflops:.1f} TFLOP/s",
          file=sys.stderr, flush=True)
    model.close()
    ctx.close()
    if not a.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, params, tokens)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
