"""Benchmark: one GPT2 training step (forward + backward + AdamW) as tile
tasks on one MI355X. Default workload: the wide 4-block model (d 8192, 64
heads, inner 32768, vocab 50257, seq 1024, batch 4; 3.64 B parameters, all
state in HBM) with large tiles (batch 4, seq 1024, embd 2048, inner 8192,
head 16, vocab 2048) -- the largest configuration that fits one GPU. The
GPT2-small step (12 blocks, d 768, the NNTile README's example tiles) is
timed after it and reported under "gpt2_small", and the LLaMA-style model
at the same width and depth (RMSNorm, rotary embedding, SwiGLU width 2048,
untied head, vocab 32000) under "llama_small".

Prints ONE JSON line:
  value        tokens/s of the whole step (inputs resident in HBM)
  tflops       model TFLOP/s = 3 x forward matmul flops (causal attention
               counted over T(T+1)/2 pairs) / step time; mfma_frac = / 157.3
  roofline     the dominant task class (largest share of a step run on one
               stream, attention included): its algorithmic flops per
               launch / its average launch duration, timed with HIP events
               on the executor stream that launches it, during the timed
               steps (every 5th launch when a step has 5 or more: an event
               pair costs ~4 us of queue time)
  classes      every task class's achieved throughput against its roofline
               (MFMA fp32 or HBM), from one extra step run on one stream
               with each task timed, so no kernel shares the GPU
  probes       on-device ceilings measured in the same run: the fp32
               matrix-core peak (tt_probe_mfma_f32) and a 2 GiB HBM copy
  cpu_baseline the fp64 oracle timed on this host's cores (BLAS threads =
               the CPUs this process may run on) on a bounded sample of the
               workload, scaled to tokens/s of the whole step (see
               cpu_baseline())
Usage: python bench.py [--gpus 1] [--steps 10] [--warmup 3] [--workload NAME]
       [--streams S (default: 1; small tiles 4)] [--pinned [--grads-in-hbm] --budget-gb G]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import synth  # noqa: E402

METRIC = "GPT2 train tokens/sec + TFLOP/s (% fp32 MFMA peak) per fwd+bwd+AdamW step, 1 GPU"
MFMA_FP32_PEAK = 157.3  # TFLOP/s, MI355X dense fp32 matrix
PROFILE_EVERY = 5       # timed-region sampling of the dominant class's launches
HBM_PEAK = 8000.0       # GB/s


# HBM bytes per launch of a task class, from two rocprofv3 --pmc runs of the
# class alone at its task shape (FETCH_SIZE, then WRITE_SIZE, KiB per
# dispatch, summed over the dispatches one task makes), each scaled by what
# the counter reads for a 1 GiB device copy (FETCH_SIZE reads half the bytes
# on gfx950: factor 2.0; WRITE_SIZE: 1.0). Valid only for the kernel source
# the counters were taken on (sha256 prefix of the file); else null.
TRAFFIC = {
    # profiles/gemm_ksum_fc_wide4_traffic.md
    ("wide4", "fc"): {"source": "tile_task_transformer_amd/csrc/gemm.hip", "sha256": "4fe4a33b25390ee5",
                      "fetch_kib": 787707.3, "fetch_factor": 2.0, "write_kib": 262144.0, "write_factor": 1.0},
    # profiles/gemm_batch_head_gpt2_small_traffic.md
    ("gpt2_small", "head"): {"source": "tile_task_transformer_amd/csrc/gemm.hip", "sha256": "4fe4a33b25390ee5",
                             "fetch_kib": 983625.2, "fetch_factor": 2.0, "write_kib": 842538.7, "write_factor": 1.0},
}


def traffic_bytes(workload: str, label: str):
    import hashlib
    t = TRAFFIC.get((workload, label))
    if not t:
        return None
    with open(os.path.join(ROOT, t["source"]), "rb") as f:
        if hashlib.sha256(f.read()).hexdigest()[:16] != t["sha256"]:
            return None
    return 1024.0 * (t["fetch_kib"] * t["fetch_factor"] + t["write_kib"] * t["write_factor"])


ALL_WORKLOADS = {**synth.WORKLOADS, **synth.LLAMA_WORKLOADS}


def family_of(name: str) -> str:
    """Block family of a workload: the LLaMA-style ones use RMSNorm, rotary
    embedding and a SwiGLU MLP (three MLP products instead of two)."""
    return "llama" if name in synth.LLAMA_WORKLOADS else "gpt2"


def specs_of(s, family: str):
    return synth.llama_param_specs(s) if family == "llama" else synth.param_specs(s)


def model_flops(s, family: str = "gpt2") -> float:
    n = s.batch * s.seq
    mlp = 3 if family == "llama" else 2  # gate, up, down against input and output layers
    per_block = 2 * n * s.n_embd * (3 * s.n_embd + s.n_embd + mlp * s.n_inner)
    attn = 2 * 2 * s.batch * s.n_embd * (s.seq * (s.seq + 1) // 2)
    head = 2 * n * s.n_embd * s.vocab
    return 3.0 * (s.n_layer * (per_block + attn) + head)


def class_work(s, family: str = "gpt2") -> dict:
    """Algorithmic work of each task class over one step: label -> (bound,
    amount, unit). GEMM classes count 2*m*n*k over all their tiles (ragged
    tiles included, so dividing by the launch count gives the exact mean per
    launch); attention counts causal pairs T(T+1)/2, the backward as 5
    products against the forward's 2 (its recompute of P included); memory
    classes count the bytes each kernel must move at least. LLaMA-style
    steps: "fc" is the SwiGLU gate and up products together, RMSNorm,
    rotary and SwiGLU passes replace LayerNorm and the bias column sums."""
    n, d, i, v, L = s.batch * s.seq, s.n_embd, s.n_inner, s.vocab, s.n_layer
    llama = family == "llama"
    f = {"qkv": 2.0 * n * d * 3 * d * L, "attn_proj": 2.0 * n * d * d * L,
         "fc": 2.0 * n * d * i * L * (2 if llama else 1), "mlp_proj": 2.0 * n * i * d * L, "head": 2.0 * n * d * v}
    out = {}
    for k, x in f.items():
        for suf in ("", "_dx", "_dw"):
            out[k + suf] = ("mfma", x, "flop")
    att = 2 * 2 * s.batch * d * (s.seq * (s.seq + 1) // 2) * L
    out["attn_fwd"] = ("mfma", float(att), "flop")
    out["attn_bwd"] = ("mfma", 2.5 * att, "flop")
    norm = "rms" if llama else "ln"
    out[norm + "_fwd"] = ("hbm", 8.0 * n * d * (2 * L + 1), "B")
    out[norm + "_bwd"] = ("hbm", 16.0 * n * d * (2 * L + 1), "B")
    out["ce_stats"] = ("hbm", 4.0 * n * v, "B")
    out["ce_grad"] = ("hbm", 8.0 * n * v, "B")
    if llama:
        out["rope"] = ("hbm", 16.0 * n * d * L, "B")         # q and k read and written in place
        out["rope_bwd"] = ("hbm", 16.0 * n * d * L, "B")
        out["swiglu"] = ("hbm", 12.0 * n * i * L, "B")       # gate, up read; product written
        out["swiglu_bwd"] = ("hbm", 20.0 * n * i * L, "B")   # dh, gate, up read; two gradients written
    else:
        out["colsum"] = ("hbm", 4.0 * n * (3 * d + d + i + d) * L, "B")
    n_params = sum(int(np.prod(shp)) for _, shp, _ in specs_of(s, family))
    out["adamw"] = ("hbm", 28.0 * n_params, "B")
    return out


# share of each memory class's algorithmic bytes that are writes: LayerNorm
# forward reads x and writes y; its backward reads dy, x and the dx it adds
# to and writes dx; the statistics and column sums only read; the gradient
# of the logits reads z and writes dz; AdamW reads p, g, m, v and writes p,
# m, v
WRITE_SHARE = {"ln_fwd": 0.5, "ln_bwd": 0.25, "ce_stats": 0.0, "ce_grad": 0.5, "colsum": 0.0, "adamw": 3 / 7,
               "rms_fwd": 0.5, "rms_bwd": 0.25, "rope": 0.5, "rope_bwd": 0.5, "swiglu": 1 / 3, "swiglu_bwd": 0.4}


def hbm_ceiling(probe: dict, write_share: float) -> float:
    """Stream-probe rate for a traffic mix (GB/s): the read probe for pure
    reads, the 1:1 copy probe at half writes, linear in between."""
    r, c = probe["hbm_read_GBps"], probe["hbm_copy_GBps_lib"]
    return r + (c - r) * min(write_share, 0.5) / 0.5


# task labels whose kernels together do one class's work (LayerNorm over
# several embd tiles runs as partial statistics, merge and apply tasks)
CLASS_LABELS = {"ln_fwd": ("ln_fwd", "ln_part", "ln_merge", "ln_apply"), "ln_bwd": ("ln_bwd", "lnb_part", "lnb_apply")}


def class_rooflines(breakdown: dict, s, family: str = "gpt2") -> dict:
    """Per-class achieved throughput from a serialized profiled step."""
    res = {}
    for label, (bound, amount, unit) in class_work(s, family).items():
        parts = [breakdown[x] for x in CLASS_LABELS.get(label, (label,)) if x in breakdown]
        b = {"count": sum(x["count"] for x in parts), "total_ms": sum(x["total_ms"] for x in parts)}
        if not b["count"]:
            continue
        sec = b["total_ms"] * 1e-3
        peak = MFMA_FP32_PEAK if bound == "mfma" else HBM_PEAK
        ach = amount / sec / (1e12 if bound == "mfma" else 1e9)
        res[label] = {"bound": bound, "launches": b["count"], "ms": round(b["total_ms"], 3),
                      "per_launch": amount / b["count"], "unit_per_launch": unit, "achieved": round(ach, 2),
                      "unit": "TFLOP/s" if bound == "mfma" else "GB/s", "frac": round(ach / peak, 4)}
    return res


# entry point of each task class's launches (the rest are tile_gemm)
KERNEL_OF = {"head": "tile_gemm_batch", "head_dw": "tile_gemm_batch", "head_dx": "tile_gemm_ksum",
             "qkv_dw": "tile_gemm_batch", "qkv_dx": "tile_gemm_ksum", "attn_proj_dw": "tile_gemm_batch",
             "fc_dw": "tile_gemm_batch", "mlp_proj_dw": "tile_gemm_batch", "attn_fwd": "tile_attention_fwd",
             "attn_bwd": "tile_attention_bwd_ws"}
# linear layers whose contraction the step sums as one long-K task when it
# spans several tiles (the MLP output layer stays a chain of tile_gemm at
# 512-1023 output blocks with 8192-wide contraction tiles)
KSUM_WHEN_SPLIT = {"qkv": "embd", "attn_proj": "head", "fc": "embd", "mlp_proj": "inner", "mlp_proj_dx": "embd",
                   "fc_dx": "inner", "attn_proj_dx": "embd"}


def kernel_of(label: str, s, t) -> str:
    """The entry point a class's launches go through at this tiling."""
    axis = KSUM_WHEN_SPLIT.get(label)
    if axis:
        full = {"embd": s.n_embd, "inner": s.n_inner, "head": s.n_head}[axis]
        tile = getattr(t, axis)
        if tile < full:
            rows = (t.batch * t.seq) // 128
            cols = {"qkv": t.head * (s.n_embd // s.n_head), "attn_proj": t.embd, "fc": t.inner, "mlp_proj": t.embd,
                    "mlp_proj_dx": t.inner, "fc_dx": t.embd, "attn_proj_dx": t.head * (s.n_embd // s.n_head)}[label]
            k_tile = {"embd": t.embd, "inner": t.inner, "head": t.head * (s.n_embd // s.n_head)}[axis]
            nb = rows * (cols // 128)
            chain = 512 <= nb < 1024 and label in ("qkv", "attn_proj", "fc", "mlp_proj") and k_tile >= 8192
            return "tile_gemm" if chain else "tile_gemm_ksum"
    return KERNEL_OF.get(label, "tile_gemm")

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


def tile_classes(w, reps=20, only=None):
    """Each tile-op class of the workload (or just `only`), launched alone on
    one stream at its task shape; HIP-event time per launch against its
    roofline."""
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
    # the tied head runs over every vocab tile in one task: z_v = nf wte_v^T
    # and dwte_v = dz_v^T nf as one tile_gemm_batch launch, dnf = sum_v dz_v
    # wte_v as one tile_gemm_ksum launch (the last vocab tile ragged)
    lens = [min(v, s.vocab - v0) for v0 in range(0, s.vocab, v)]
    head_flops = 2.0 * r * e * s.vocab
    for label in ("head", "head_dw", "head_dx"):
        if only and label != only:
            continue
        X = rnd(r, e)
        Z = [rnd(r, n) for n in lens]
        W = [rnd(n, e) for n in lens]
        if label == "head":
            fn = lambda: tt.tile_gemm_batch(st, 0, 1, r, lens, e, 1.0, [X] * len(lens), e, W, e, 0.0, Z, lens)  # noqa
        elif label == "head_dw":
            fn = lambda: tt.tile_gemm_batch(st, 1, 0, lens, e, r, 1.0, Z, lens, [X] * len(lens), e, 1.0, W, e)  # noqa
        else:
            fn = lambda: tt.tile_gemm_ksum(st, r, e, lens, 1.0, Z, lens, W, [e] * len(lens), 0.0, X, e)  # noqa
        ms = timed(fn)
        tf = head_flops / (ms * 1e-3) / 1e12
        out[label] = {"bound": "mfma", "shape": [r, e, s.vocab, len(lens)], "us": round(ms * 1e3, 1),
                      "achieved": round(tf, 2), "unit": "TFLOP/s", "frac": round(tf / MFMA_FP32_PEAK, 4)}
        del X, Z, W
    # the attention block's q, k and v weight gradients as one batched
    # (split-K) launch, its input gradient as one long-K launch over the
    # 3 x head-tile pairs (as the step runs them)
    nq = 3 * (s.n_head // t.head)
    for label in ("qkv_dw", "qkv_dx"):
        if only and label != only:
            continue
        X = rnd(r, e)
        D = [rnd(r, h) for _ in range(nq)]
        W = [rnd(e, h) for _ in range(nq)]
        if label == "qkv_dw":
            nws = tt.tile_gemm_batch_workspace([e] * nq, [h] * nq, r)
            ws = torch.empty(max(nws // 4, 1), device="cuda")
            fn = lambda: tt.tile_gemm_batch_ws(st, 1, 0, e, h, r, 1.0, [X] * nq, e, D, h, 0.0, W, h, ws, nws)  # noqa
        else:
            fn = lambda: tt.tile_gemm_ksum(st, r, e, [h] * nq, 1.0, D, [h] * nq, W, [h] * nq, 0.0, X, e,  # noqa
                                           transB=1)
        ms = timed(fn)
        tf = 2.0 * r * e * h * nq / (ms * 1e-3) / 1e12
        out[label] = {"bound": "mfma", "shape": [r, e, h, nq], "us": round(ms * 1e3, 1),
                      "achieved": round(tf, 2), "unit": "TFLOP/s", "frac": round(tf / MFMA_FP32_PEAK, 4)}
        del X, D, W
    for label, f in GEMM_SHAPES.items():
        if only and label != only:  # "attn": the attention classes only
            continue
        if label in ("head", "head_dw", "head_dx", "qkv_dw", "qkv_dx"):
            continue
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
    if only and only != "attn":
        return out
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
    if only:
        return out

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


def copy_probe(mib: int):
    """A plain device-to-device copy of `mib` MiB (torch's copy kernel), three
    times: the known byte count calibrates the profiler's memory counters."""
    import torch
    n = mib * 2 ** 20 // 4
    src = torch.ones(n, device="cuda")
    dst = torch.empty(n, device="cuda")
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()


def link_probe(mib: int = 1024, reps: int = 5) -> dict:
    """Pinned host <-> HBM copy rates (GB/s): H2D alone, D2H alone, and both
    at once on two streams (the link is full duplex)."""
    import torch
    n = mib * 2 ** 20 // 4
    h_src = torch.ones(n, pin_memory=True)
    h_dst = torch.empty(n, pin_memory=True)
    d_src = torch.ones(n, device="cuda")
    d_dst = torch.empty(n, device="cuda")
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()

    def timed(fns):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(reps):
            for st, fn in fns:
                with torch.cuda.stream(st):
                    fn()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) / reps

    nbytes = n * 4
    h2d = nbytes / timed([(s1, lambda: d_dst.copy_(h_src, non_blocking=True))]) / 1e9
    d2h = nbytes / timed([(s1, lambda: h_dst.copy_(d_src, non_blocking=True))]) / 1e9
    both = 2 * nbytes / timed([(s1, lambda: d_dst.copy_(h_src, non_blocking=True)),
                               (s2, lambda: h_dst.copy_(d_src, non_blocking=True))]) / 1e9
    return {"h2d_GBps": round(h2d, 1), "d2h_GBps": round(d2h, 1), "both_GBps": round(both, 1), "mib": mib}


def pmc_summary(paths, copy_mib: int) -> dict:
    """Mean FETCH_SIZE / WRITE_SIZE (KiB per dispatch) per (kernel, grid) from
    rocprofv3 counter_collection.csv files, and the factor that maps each
    counter to bytes: the known size of the copy probe over what the counter
    reads for it."""
    import csv
    from collections import defaultdict
    acc = defaultdict(lambda: [0.0, 0])
    durations = defaultdict(list)
    for p in paths:
        with open(p) as f:
            for row in csv.DictReader(f):
                if "Counter_Name" in row:
                    key = (row["Counter_Name"], row["Kernel_Name"], int(row["Grid_Size"]))
                    acc[key][0] += float(row["Counter_Value"])
                    acc[key][1] += 1
                else:  # a kernel trace: durations per (kernel, grid)
                    grid = 1
                    for ax in ("X", "Y", "Z"):
                        grid *= int(row.get("Grid_Size_" + ax, 1) or 1)
                    durations[(row["Kernel_Name"], grid)].append(
                        (int(row["End_Timestamp"]) - int(row["Start_Timestamp"])) * 1e-3)
    out = {"kernels": [], "copy_bytes": copy_mib * 2 ** 20}
    for (ctr, name, grid), (tot, cnt) in sorted(acc.items()):
        out["kernels"].append({"counter": ctr, "kernel": name[:160], "grid": grid, "dispatches": cnt,
                               "mean_kib": tot / cnt})
    for (name, grid), us in sorted(durations.items(), key=lambda kv: -sum(kv[1])):
        out["kernels"].append({"kernel": name[:160], "grid": grid, "dispatches": len(us),
                               "mean_us": sum(us) / len(us), "total_ms": sum(us) * 1e-3})
    for ctr in ("FETCH_SIZE", "WRITE_SIZE"):
        copies = [k for k in out["kernels"] if k.get("counter") == ctr and "copy" in k["kernel"].lower()
                  and k["mean_kib"] * 1024 > 0.5 * out["copy_bytes"]]
        if copies:
            c = max(copies, key=lambda k: k["mean_kib"])
            out[ctr + "_factor"] = out["copy_bytes"] / (c["mean_kib"] * 1024)
    return out


def blas_setup():
    """BLAS threads = the CPUs this process may run on; returns (cores,
    vendor string) for the report."""
    cores = len(os.sched_getaffinity(0))
    vendor = "unknown"
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        threadpool_limits(limits=cores, user_api="blas")
        info = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        if info:
            vendor = f"{info[0].get('internal_api')} {info[0].get('version')} ({info[0].get('num_threads')} threads)"
    except Exception:  # noqa: BLE001
        pass
    return cores, vendor


def cpu_baseline(w, params, tokens, sample_tokens: int = 0):
    """The fp64 oracle on the host's cores, on a bounded sample of the step.

    Small models (<= 200 M parameters): the oracle's whole step on one
    sequence of the batch, once after a warm-up, scaled to the batch by
    token count. Larger models: block 0 of the model plus the tied head on
    the first `sample_tokens` tokens of sequence 0 (oracle forward and
    backward), and the oracle's AdamW on that block's attention-projection weight; the
    full step's time is extrapolated by model flops (forward + backward)
    and by parameter count (AdamW), and labelled so."""
    import numpy as np
    from oracle import gpt2 as og
    cores, vendor = blas_setup()
    s = w.shape
    n_params = sum(int(np.prod(shp)) for _, shp, _ in synth.param_specs(s))
    if n_params <= 200_000_000:
        sample = np.asarray(tokens[:1], np.int64)
        og.step(params, sample[:, :65], s.n_layer, s.n_head, lr=w.lr, wd=w.weight_decay)  # warm-up
        t0 = time.perf_counter()
        og.step(params, sample, s.n_layer, s.n_head, lr=w.lr, wd=w.weight_decay)
        dt = time.perf_counter() - t0
        return {"value": round(s.seq / dt, 2), "unit": "tokens/s", "cores": cores, "kind": "oracle", "blas": vendor,
                "extrapolated": False, "seconds": round(dt, 2),
                "sample": f"one {s.seq}-token sequence of the batch (1 of {s.batch}): the oracle's whole step "
                          f"(fwd+bwd+AdamW, fp64 numpy) after a warm-up; tokens/s = {s.seq} / time"}
    T = sample_tokens or min(s.seq, 256)
    sub = {k: np.asarray(v, np.float64) for k, v in params.items()
           if not k.startswith("h") or k.startswith("h0.")}
    tok = np.asarray(tokens[:1, :T + 1], np.int64)
    x, y = tok[:, :-1], tok[:, 1:]
    og.forward(sub, x[:, :16], y[:, :16], 1, s.n_head)  # warm-up (BLAS threads, page-in)
    t0 = time.perf_counter()
    _, cache = og.forward(sub, x, y, 1, s.n_head)
    og.backward(cache, 1, s.n_head)
    t_fb = time.perf_counter() - t0
    del cache
    wfc = sub["h0.w_o"]
    g = np.full_like(wfc, 1e-3)
    t0 = time.perf_counter()
    og.adamw(wfc, g, np.zeros_like(wfc), np.zeros_like(wfc), 1, w.lr, w.beta1, w.beta2, w.eps, w.weight_decay)
    t_opt = time.perf_counter() - t0
    samp = synth.GPT2Shape(1, s.vocab, s.n_embd, s.n_head, s.n_inner, T, 1)
    f_ratio = model_flops(s) / model_flops(samp)
    p_ratio = n_params / wfc.size
    step_s = t_fb * f_ratio + t_opt * p_ratio
    return {"value": round(s.batch * s.seq / step_s, 3), "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "blas": vendor, "extrapolated": True, "seconds_per_step": round(step_s, 1),
            "sample_seconds": {"fwd_bwd": round(t_fb, 2), "adamw": round(t_opt, 2)},
            "sample": f"extrapolated: the oracle's forward+backward (fp64 numpy) of block 0 plus embedding, final "
                      f"LayerNorm and tied head on the first {T} tokens of sequence 0 ({t_fb:.1f} s), scaled by "
                      f"model flops x{f_ratio:.1f} to {s.n_layer} blocks x {s.batch}x{s.seq} tokens; the oracle's "
                      f"AdamW on block 0's attention-projection weight ({wfc.size / 1e6:.0f} M parameters, {t_opt:.1f} s), scaled by "
                      f"parameter count x{p_ratio:.1f}"}


def probes() -> dict:
    """On-device ceilings, in the benchmark's own process: the fp32 matrix
    peak (a launch of the library's MFMA probe, best of 4), the rate of a
    2 GiB device-to-device copy (torch's copy kernel, best of 4) and the
    library's HBM stream probes over the same 2 GiB (read, write, copy)."""
    import torch

    import tile_task_transformer_amd as tt
    st = torch.cuda.current_stream()
    blocks, iters = 2048, 8192
    out = torch.empty(blocks * 256, device="cuda")
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    best = float("inf")
    flops = 0.0
    for _ in range(4):
        a.record(st)
        flops = tt.tt_probe_mfma_f32(st, blocks, iters, out)
        b.record(st)
        b.synchronize()
        best = min(best, a.elapsed_time(b))
    mfma = flops / (best * 1e-3) / 1e12
    n = 2 ** 29  # 2 GiB of fp32
    src = torch.ones(n, device="cuda")
    dst = torch.empty(n, device="cuda")
    cbest = float("inf")
    for _ in range(4):
        a.record(st)
        dst.copy_(src)
        b.record(st)
        b.synchronize()
        cbest = min(cbest, a.elapsed_time(b))
    # the library's stream probes: read, write and 1:1 copy, each the best
    # over grid sizes and store kinds
    hbm = {}
    for name, kind in (("read", tt.TT_PROBE_READ), ("write", tt.TT_PROBE_WRITE), ("copy", tt.TT_PROBE_COPY)):
        rate = 0.0
        for nt in (0, tt.TT_PROBE_NONTEMPORAL):
            for blocks in (1024, 2048, 4096, 8192):
                for _ in range(3):
                    a.record(st)
                    moved = tt.tt_probe_hbm(st, kind | nt, src, dst, n, blocks)
                    b.record(st)
                    b.synchronize()
                    rate = max(rate, moved / (a.elapsed_time(b) * 1e-3) / 1e9)
        hbm[f"hbm_{name}_GBps" + ("_lib" if name == "copy" else "")] = round(rate, 1)
    del src, dst, out
    return {"mfma_f32_tflops": round(mfma, 2), "mfma_f32_frac_of_spec": round(mfma / MFMA_FP32_PEAK, 4),
            "hbm_copy_GBps": round(2 * 4 * n / (cbest * 1e-3) / 1e9, 1), **hbm}


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="wide4", choices=sorted(ALL_WORKLOADS))
    ap.add_argument("--also", default="gpt2_small,llama_small",
                    help="comma-separated workloads timed after the first, each reported under its name "
                         "('' = none)")
    ap.add_argument("--streams", type=int, default=0,
                    help="executor streams (0 = measured best per workload: 1; small tiles 4; pinned 1)")
    ap.add_argument("--heavy-gflops", type=float, default=0.0,
                    help="tasks of at least this many GFLOP run in order on stream 0 (0 = off)")
    ap.add_argument("--priorities", action="store_true",
                    help="launch each window by critical-path priority instead of submission order")
    ap.add_argument("--depth-sweep", default="",
                    help="instead of the step: time the workload's widths at these block counts (e.g. 1,2,4,8,12) "
                         "on 1 and 4 streams, 4 with critical-path priorities, and print the results as JSON "
                         "(also written to --out-dir/depth_sweep.json)")
    ap.add_argument("--out-dir", default=os.environ.get("TT_BENCH_OUT", "bench_out"),
                    help="folder for the per-class breakdown and the depth sweep (default: $TT_BENCH_OUT or bench_out)")
    ap.add_argument("--pinned", action="store_true",
                    help="parameters, gradients and moments live in pinned host RAM (out-of-core residency)")
    ap.add_argument("--grads-in-hbm", action="store_true",
                    help="with --pinned: gradients stay in HBM, only parameters and moments are pinned")
    ap.add_argument("--budget-gb", type=float, default=0.0, help="device arena for pinned tiles (0 = half of free)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--breakdown", default=None,
                    help="file for the per-task-class GPU times of one extra step run on one stream "
                         "(default: --out-dir/bench_breakdown.json; '' = skip)")
    ap.add_argument("--tile-classes", default="",
                    help="instead of the step: time each tile-op class alone and write this JSON file")
    ap.add_argument("--only", default=None, help="with --tile-classes: just this GEMM class")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="after the run, copy this many MiB three times (counter calibration)")
    ap.add_argument("--pmc-summary", nargs="+", default=None,
                    help="instead of running: summarise rocprofv3 counter_collection.csv files")
    a = ap.parse_args(argv)
    if a.breakdown is None:
        a.breakdown = os.path.join(a.out_dir, "bench_breakdown.json")
    if a.pmc_summary:
        res = pmc_summary(a.pmc_summary, a.copy_probe_mib)
        print(json.dumps(res, indent=1))
        return 0
    if a.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (--gpus must be 1)", file=sys.stderr)
        return 2
    if a.steps < 1 or a.warmup < 0:
        print("bench.py: --steps must be at least 1 and --warmup at least 0", file=sys.stderr)
        return 2
    if a.grads_in_hbm and not a.pinned:
        print("bench.py: --grads-in-hbm goes with --pinned", file=sys.stderr)
        return 2

    w = ALL_WORKLOADS[a.workload]
    if a.streams <= 0:
        # measured on MI355X: many small tasks need concurrency (small tiles:
        # 911 ms on 4 streams, 1018 on 2); GPT2-small's and the wide model's
        # tasks fill the GPU alone and run faster one at a time (35.0 vs
        # 35.8 ms; 741.5 vs 753.8 ms); staged tiles want one (fewer tiles
        # needed at once)
        a.streams = {"wide4_small_tiles": 4}.get(a.workload, 1) if not a.pinned else 1
    if a.tile_classes:
        res = tile_classes(w, only=a.only)
        if a.copy_probe_mib:
            copy_probe(a.copy_probe_mib)
        os.makedirs(os.path.dirname(a.tile_classes) or ".", exist_ok=True)
        with open(a.tile_classes, "w") as f:
            json.dump(res, f, indent=1)
        for k, v in res.items():
            print(f"{k:14s} {v['us']:9.1f} us  {v['achieved']:8.1f} {v['unit']:16s} {100 * v['frac']:5.1f}%",
                  file=sys.stderr)
        return 0
    if a.depth_sweep:
        res = depth_sweep(w, [int(x) for x in a.depth_sweep.split(",")])
        os.makedirs(a.out_dir, exist_ok=True)
        with open(os.path.join(a.out_dir, "depth_sweep.json"), "w") as f:
            json.dump(res, f, indent=1)
        print(json.dumps(res), flush=True)
        return 0
    probe = probes()
    print(f"[bench] probes: {probe}", file=sys.stderr, flush=True)
    out, keep = run(w, a, a.streams, a.breakdown, probe)
    out["probes"] = probe
    for name in [x for x in a.also.split(",") if x and x != a.workload]:
        w2 = ALL_WORKLOADS[name]
        o2, _ = run(w2, a, {"wide4_small_tiles": 4}.get(name, 1), "", probe, steps=max(a.steps, 10),
                    warmup=max(a.warmup, 3), want_params=False)
        out[name] = {k: o2[k] for k in ("value", "unit", "ms_per_step", "tflops", "mfma_frac", "tasks_per_step",
                                        "loss", "roofline", "largest_class")}
        out[name]["config"] = o2["config"]
        if family_of(name) == "llama":
            out[name]["classes"] = o2["classes"]
    if not a.no_cpu_baseline and family_of(w.name) != "gpt2":
        print("[bench] the CPU baseline samples the GPT2 oracle: skipped for this workload", file=sys.stderr)
    elif not a.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, keep["params"], keep["tokens"])
        cb = out["cpu_baseline"]
        cb["gpu_speedup"] = round(out["value"] / cb["value"], 1)
        print(f"[bench] cpu baseline {cb['value']} tokens/s on {cb['cores']} cores", file=sys.stderr, flush=True)
    print(json.dumps(out), flush=True)
    return 0


def run(w, a, streams, breakdown_path, probe, steps=None, warmup=None, want_params=True):
    """Time `steps` steps of workload w after `warmup` ones; returns the JSON
    fields and (if want_params) the host parameters and tokens the CPU
    baseline samples."""
    import torch

    from tile_task_transformer_amd import _lib as L
    from tile_task_transformer_amd.runtime import Context, GPT2
    steps = steps or a.steps
    warmup = a.warmup if warmup is None else warmup
    s, t = w.shape, w.tiles
    family = family_of(w.name)
    specs = specs_of(s, family)
    t0 = time.perf_counter()
    params = synth.init_params(s, seed=0, threads=min(16, len(os.sched_getaffinity(0))), specs=specs)
    tokens = synth.token_stream(s, seed=1)
    home = (L.TT_HOME_PINNED_STATE if a.grads_in_hbm else L.TT_HOME_PINNED_HOST) if a.pinned else L.TT_HOME_DEVICE
    ctx = Context(0, n_streams=streams, window=4096, device_budget=int(a.budget_gb * 2 ** 30))
    if a.heavy_gflops > 0:
        ctx.heavy_lane(a.heavy_gflops * 1e9)
    if a.priorities:
        ctx.priorities(True)
    model = GPT2(ctx, s, t, param_home=home, family=family)
    model.set_params(params, specs)
    if not want_params or a.no_cpu_baseline:
        params = None  # the oracle sample is not needed: free the host copy
    tok = torch.from_numpy(tokens.astype(np.int32)).cuda()
    hp = dict(lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps, weight_decay=w.weight_decay)
    print(f"[bench] {w.name}: parameters ready in {time.perf_counter() - t0:.1f} s", file=sys.stderr, flush=True)

    for k in range(warmup):
        model.step(tok, **hp)
        print(f"[bench] warmup step {k + 1}/{warmup} loss {model.loss():.4f}", file=sys.stderr, flush=True)
    print(f"[bench] {model.task_count()} tasks/step", file=sys.stderr, flush=True)

    # one step on a single stream with every task timed: each kernel has the
    # GPU to itself, which gives the per-class rooflines
    ctx.streams_active(1)
    ctx.profile("*")
    model.step(tok, **hp)
    breakdown = ctx.profile_take()
    ctx.profile(None)
    ctx.streams_active(streams)
    classes = class_rooflines(breakdown, s, family)
    if probe:
        # matrix classes against the measured matrix peak; memory classes
        # against the stream probe of their traffic mix
        for k, v in classes.items():
            if v["bound"] == "mfma":
                v["frac_of_probe"] = round(v["achieved"] / probe["mfma_f32_tflops"], 4)
            elif k in WRITE_SHARE:
                v["frac_of_probe"] = round(v["achieved"] / hbm_ceiling(probe, WRITE_SHARE[k]), 4)
    if breakdown_path:
        os.makedirs(os.path.dirname(breakdown_path) or ".", exist_ok=True)
        with open(breakdown_path, "w") as f:
            json.dump({"workload": w.name, "tasks": breakdown, "classes": classes}, f, indent=1, sort_keys=True)
    print(f"[bench] {w.name}: serialized step by class (ms, achieved, % of roofline, % of probe):", file=sys.stderr)
    for k, v in sorted(classes.items(), key=lambda kv: -kv[1]["ms"]):
        fp = f"{100 * v['frac_of_probe']:5.1f}%" if "frac_of_probe" in v else ""
        print(f"  {k:14s} {v['ms']:9.2f} ms  {v['achieved']:9.1f} {v['unit']:8s} {100 * v['frac']:5.1f}%  {fp}",
              file=sys.stderr)
    print(f"  serialized total {sum(b['total_ms'] for b in breakdown.values()):.2f} ms", file=sys.stderr,
          flush=True)
    work = class_work(s, family)
    # the dominant class: the largest share of the step's model flops among
    # the matrix-core classes (GEMM and attention alike), ties (the MLP's
    # six products of equal size) broken by name, so that the choice does
    # not flip between runs whose times differ by noise
    mfma = [k for k, v in classes.items() if v["bound"] == "mfma"]
    dominant = min(mfma, key=lambda k: (-work[k][1], k)) if mfma else "fc"

    # timed region: K steps back to back, every PROFILE_EVERY-th task of the
    # dominant class bracketed by events (an event pair costs ~4 us of queue
    # time; 5 is prime to the 66 vocab tiles of GPT2-small, so the sample
    # rotates through every tile, the ragged last one included); a class
    # with fewer launches per step than that is timed at every launch
    every = PROFILE_EVERY if classes.get(dominant, {}).get("launches", PROFILE_EVERY) >= PROFILE_EVERY else 1
    ctx.profile(dominant, every=every)
    ctx.reset_stats()
    torch.cuda.synchronize()
    ctx.wait()
    # per-step boundaries: after each step the torch stream waits for every
    # context stream (the step has flushed already, so this adds one event
    # record and wait per stream) and records an event, so consecutive events
    # bracket one step's completion on the GPU
    cur = torch.cuda.current_stream()
    bounds = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    t0 = time.perf_counter()
    ctx.join_stream(cur)
    bounds[0].record(cur)
    for i in range(steps):
        model.step(tok, **hp)
        ctx.join_stream(cur)
        bounds[i + 1].record(cur)
    ctx.wait()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    step_ms = [bounds[i].elapsed_time(bounds[i + 1]) for i in range(steps)]
    print(f"[bench] {w.name}: GPU time of each timed step (ms): {[round(x, 1) for x in step_ms]}", file=sys.stderr)
    step_ms.sort()
    loss = model.loss()
    st = ctx.stats()
    prof = ctx.profile_take().get(dominant, {})
    ctx.profile(None)

    ms = 1e3 * elapsed / steps
    tok_s = s.batch * s.seq / (elapsed / steps)
    tflops = model_flops(s, family) / (elapsed / steps) / 1e12
    launches = prof.get("count", 0)
    per_step = classes[dominant]["launches"] if dominant in classes else launches * every / steps
    per_launch = work[dominant][1] / per_step if launches else float("nan")
    avg_ms = prof["total_ms"] / launches if launches else float("nan")
    achieved = per_launch / (avg_ms * 1e-3) / 1e12
    largest = max(classes, key=lambda k: classes[k]["ms"]) if classes else None
    out = {
        "metric": METRIC, "value": round(tok_s, 1), "unit": "tokens/s", "n_gpus": 1, "steps": steps,
        "warmup": warmup, "ms_per_step": round(ms, 3),
        "ms_per_step_median": round(step_ms[len(step_ms) // 2] if steps % 2 else
                                    0.5 * (step_ms[steps // 2 - 1] + step_ms[steps // 2]), 3),
        "ms_per_step_min": round(step_ms[0], 3), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": w.name, "family": family, "global_batch": s.batch, "seq_len": s.seq, "n_layer": s.n_layer,
                   "n_embd": s.n_embd, "n_inner": s.n_inner, "n_head": s.n_head, "vocab": s.vocab,
                   "tiles": {"batch": t.batch, "seq": t.seq, "embd": t.embd, "inner": t.inner, "head": t.head,
                             "vocab": t.vocab}, "streams": streams, "heavy_gflops": a.heavy_gflops,
                   "priorities": bool(a.priorities),
                   "param_home": ("pinned_state" if a.grads_in_hbm else "pinned_host") if a.pinned else "device"},
        "tflops": round(tflops, 2), "mfma_frac": round(tflops / MFMA_FP32_PEAK, 4),
        "mfma_frac_of_probe": round(tflops / probe["mfma_f32_tflops"], 4) if probe else None,
        "tasks_per_step": model.task_count(), "loss": round(loss, 5),
        "host_submit_ms_per_step": round(1e3 * st["submit_seconds"] / steps, 3),
        "roofline": {"bound": "mfma", "kernel": f"{kernel_of(dominant, s, t)}[{dominant}]",
                     "achieved": round(achieved, 2),
                     "peak": MFMA_FP32_PEAK, "unit": "TFLOP/s", "frac": round(achieved / MFMA_FP32_PEAK, 4),
                     "frac_of_probe": round(achieved / probe["mfma_f32_tflops"], 4) if probe else None,
                     "traffic": traffic_bytes(w.name, dominant), "flops_per_launch": per_launch,
                     "avg_launch_ms": round(avg_ms, 4),
                     "launches_timed": launches, "launches_per_step": per_step},
        "largest_class": ({"class": largest, "frac": classes[largest]["frac"], "ms": classes[largest]["ms"]}
                          if largest else None),
    }
    if a.pinned:
        out["residency"] = {k: st[k] / steps for k in ("h2d_bytes", "d2h_bytes", "evictions", "prefetches")}
        out["residency"]["link_GBps"] = round((st["h2d_bytes"] + st["d2h_bytes"]) / elapsed / 1e9, 2)
        out["residency"]["budget_gb"] = a.budget_gb
        out["residency"]["probe"] = link_probe()
    out["classes"] = {k: {x: v[x] for x in ("frac", "frac_of_probe", "achieved", "unit", "ms") if x in v}
                      for k, v in classes.items()}
    print(f"[bench] {w.name}: timed {steps} steps: {ms:.2f} ms/step, {tok_s:.0f} tokens/s, {tflops:.1f} TFLOP/s",
          file=sys.stderr, flush=True)
    out["executor"] = executor_figures(w, model, ctx, tok, hp, streams, ms, st, steps)
    print(f"[bench] {w.name}: executor {out['executor']}", file=sys.stderr, flush=True)
    model.close()
    ctx.close()
    del tok
    torch.cuda.empty_cache()
    return out, {"params": params, "tokens": tokens}


def depth_sweep(w, layers, steps=6, warmup=2):
    """Step time against depth: the workload's widths and tiles at each block
    count in `layers`, run with (streams, priorities) = (1, off), (4, off),
    (4, on); ms per step, ms per block (after the step at zero blocks is
    subtracted, i.e. the embedding, head, loss and their updates), the GPU
    idle fraction of one more step and the task graph's longest chain."""
    import dataclasses

    import torch

    from tile_task_transformer_amd import _lib as L
    from tile_task_transformer_amd.runtime import Context, GPT2
    family = family_of(w.name)
    hp = dict(lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps, weight_decay=w.weight_decay)
    rows = []
    for n_layer in sorted(set([0] + layers)):
        s = dataclasses.replace(w.shape, n_layer=n_layer)
        specs = specs_of(s, family)
        params = synth.init_params(s, seed=0, threads=min(16, len(os.sched_getaffinity(0))), specs=specs)
        tok = torch.from_numpy(synth.token_stream(s, seed=1).astype(np.int32)).cuda()
        for streams, prio in ((1, False), (4, False), (4, True)):
            ctx = Context(0, n_streams=streams, window=8192)
            ctx.priorities(prio)
            model = GPT2(ctx, s, w.tiles, family=family)
            model.set_params(params, specs)
            for _ in range(warmup):
                model.step(tok, **hp)
            ctx.wait()
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for _ in range(steps):
                model.step(tok, **hp)
            ctx.wait()
            torch.cuda.synchronize()
            ms = 1e3 * (time.perf_counter() - t0) / steps
            ctx.profile("*", every=1)
            model.step(tok, **hp)
            busy = ctx.profile_busy()
            ctx.profile_take()
            ctx.profile(None)
            rows.append({"n_layer": n_layer, "streams": streams, "priorities": prio, "ms_per_step": round(ms, 3),
                         "tasks": model.task_count(),
                         "gpu_idle_frac": round(1 - busy["busy_ms"] / busy["span_ms"], 4) if busy["span_ms"] else None})
            print(f"[bench] depth {n_layer:2d} streams {streams} priorities {int(prio)}: {ms:8.3f} ms/step, "
                  f"idle {rows[-1]['gpu_idle_frac']}", file=sys.stderr, flush=True)
            model.close()
            ctx.close()
        del tok
        torch.cuda.empty_cache()
    base = {(r["streams"], r["priorities"]): r["ms_per_step"] for r in rows if r["n_layer"] == 0}
    for r in rows:
        if r["n_layer"]:
            r["ms_per_block"] = round((r["ms_per_step"] - base[(r["streams"], r["priorities"])]) / r["n_layer"], 3)
    return {"workload": w.name, "family": family, "steps": steps, "rows": rows}


def executor_figures(w, model, ctx, tok, hp, streams, ms, st, steps, busy_steps=2):
    """Executor overhead beside the timed step: tasks per step and GPU time
    per task; the host's own cost of building a step's task graph (the same
    step submitted to a dry-run context: dependency inference, stream
    assignment and bookkeeping without launches, so the GPU cannot hold it
    back); host time inside submit calls in the timed region (launches
    included, which block once the GPU queues are full); and the GPU's idle
    fraction: every task of busy_steps extra steps bracketed by timing
    events, 1 - (union of their GPU intervals) / (first start to last end)."""
    from tile_task_transformer_amd import _lib as L
    from tile_task_transformer_amd.runtime import Context, GPT2
    import tempfile
    ntask = model.task_count()
    with Context(L.TT_DEVICE_DRYRUN, n_streams=streams, window=4096) as dctx:
        dm = GPT2(dctx, w.shape, w.tiles, family=family_of(w.name))
        dm.step(None, **hp)
        t0 = time.perf_counter()
        for _ in range(2):
            dm.step(None, **hp)
        dry = (time.perf_counter() - t0) / 2
        dm.close()
    with tempfile.TemporaryDirectory() as tmp, Context(L.TT_DEVICE_DRYRUN, n_streams=streams, window=4096) as dctx:
        dctx.record(True)
        dm = GPT2(dctx, w.shape, w.tiles, family=family_of(w.name))
        dm.step(None, **hp)
        depth = dag_depth(dctx.dump_dag(os.path.join(tmp, "step.jsonl")))
        dm.close()
    ctx.profile("*", every=1)
    for _ in range(busy_steps):
        model.step(tok, **hp)
    busy = ctx.profile_busy()
    ctx.profile_take()
    ctx.profile(None)
    span = busy["span_ms"]
    return {
        "tasks_per_step": ntask,
        "gpu_us_per_task": round(1e3 * ms / ntask, 2),
        "host_graph_ms_per_step": round(1e3 * dry, 3),
        "host_graph_us_per_task": round(1e6 * dry / ntask, 2),
        "host_submit_ms_per_step": round(1e3 * st["submit_seconds"] / steps, 3),
        "gpu_idle_frac": round(1.0 - busy["busy_ms"] / span, 4) if span > 0 else None,
        "timed_tasks": busy["tasks"], "timed_span_ms_per_step": round(span / busy_steps, 3),
        **depth,
    }


def dag_depth(dag) -> dict:
    """Depth of one step's task graph (a dry-run dump): the longest chain of
    dependent tasks, and the flops on the costliest chain over all flops (1 /
    that bounds the speedup any launch order or stream count could get from
    running independent tasks side by side, at equal throughput per flop)."""
    cp, dp = {}, {}
    for r in dag:  # ids ascend in submission order, a topological order
        ds = [d for d in r["deps"] if d in cp]
        cp[r["id"]] = r.get("cost", 0.0) + max((cp[d] for d in ds), default=0.0)
        dp[r["id"]] = 1 + max((dp[d] for d in ds), default=0)
    total = sum(r.get("cost", 0.0) for r in dag)
    levels = {}
    for v in dp.values():
        levels[v] = levels.get(v, 0) + 1
    return {"dag_depth_tasks": max(dp.values(), default=0), "dag_max_width": max(levels.values(), default=0),
            "critical_path_flop_frac": round(max(cp.values(), default=0.0) / total, 4) if total else None}


if __name__ == "__main__":
    sys.exit(main())
