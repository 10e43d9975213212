"""Seeded synthetic inputs shared by the oracle and the GPU harness.

This module draws random numbers and describes workload shapes. It holds
none of the method's arithmetic: no layer, loss, gradient or optimiser
formula lives here, so the oracle and the HIP path can both take their
inputs from it without sharing any computation.

Workloads follow the GPT2 training example of the NNTile README
("Minimal working GPT example": a GPT2 JSON config, seq/embd/inner/head and
minibatch tile flags, fused AdamW with eps 1e-8, weight decay 0.1, lr 3e-4,
mean loss over the batch's tokens), with synthetic stand-ins for the
WikiText-103 / uint16 ``train.bin`` token streams the README trains on.

Conventions (readings of what the pages leave open):
  * weights and embeddings ~ N(0, 0.02), drawn in float64 and rounded to
    float32; biases 0; LayerNorm gains 1 and shifts 0;
  * each parameter tensor has its own PCG64 stream seeded by
    ``[seed, index]`` so any subset (one block, one slice) can be drawn
    alone and still equals the full draw;
  * token ids are uniform in [0, vocab), stored as uint16 like ``train.bin``.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Tuple

import numpy as np

__all__ = [
    "GPT2Shape", "Tiles", "Workload", "WORKLOADS", "LLAMA_WORKLOADS", "param_specs", "llama_param_specs",
    "init_params", "init_param", "token_stream", "split_tokens",
    "rand_normal", "rand_uniform",
]


@dataclasses.dataclass(frozen=True)
class GPT2Shape:
    n_layer: int
    vocab: int
    n_embd: int
    n_head: int
    n_inner: int
    seq: int
    batch: int

    @property
    def head_dim(self) -> int:
        return self.n_embd // self.n_head

    @property
    def tokens(self) -> int:
        return self.batch * self.seq


@dataclasses.dataclass(frozen=True)
class Tiles:
    """Tile sizes per axis (README flags --minibatch-tile, --seq-tile,
    --embd-tile, --inner-tile, --head-tile; the vocab tile has no flag there
    and defaults to the embd tile)."""
    batch: int
    seq: int
    embd: int
    inner: int
    head: int
    vocab: int


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    shape: GPT2Shape
    tiles: Tiles
    lr: float = 3e-4
    beta1: float = 0.9
    beta2: float = 0.999
    eps: float = 1e-8
    weight_decay: float = 0.1
    ln_eps: float = 1e-5


WORKLOADS: Dict[str, Workload] = {
    # tiny 1-block step, tiles of 32 on every axis, clamped to the axis
    "tiny": Workload("tiny", GPT2Shape(1, 256, 64, 4, 256, 32, 2),
                     Tiles(2, 32, 32, 32, 4, 32)),
    # GPT2-small shape with the README example's tile flags
    "gpt2_small": Workload("gpt2_small", GPT2Shape(12, 50257, 768, 12, 3072, 1024, 4),
                           Tiles(4, 1024, 768, 3072, 12, 768)),
    # wide 4-block model, large tiles
    "wide4": Workload("wide4", GPT2Shape(4, 50257, 8192, 64, 32768, 1024, 4),
                      Tiles(4, 1024, 2048, 8192, 16, 2048)),
    # same model, small tiles (about 16x more tasks)
    "wide4_small_tiles": Workload("wide4_small_tiles", GPT2Shape(4, 50257, 8192, 64, 32768, 1024, 4),
                                  Tiles(4, 256, 512, 2048, 8, 512)),
    # out-of-core wide 8-block model
    "wide8_ooc": Workload("wide8_ooc", GPT2Shape(8, 50257, 16384, 128, 65536, 1024, 2),
                          Tiles(2, 1024, 2048, 8192, 16, 2048)),
}


# LLaMA-style models (RMSNorm, rotary embedding, SwiGLU MLP, untied head):
# n_inner is the SwiGLU hidden width (about 8/3 d, a multiple of 256)
LLAMA_WORKLOADS: Dict[str, Workload] = {
    "llama_tiny": Workload("llama_tiny", GPT2Shape(1, 256, 64, 4, 176, 32, 2),
                           Tiles(2, 32, 32, 32, 4, 32)),
    # GPT2-small's width and depth with a LLaMA block and a 32000-token vocabulary
    "llama_small": Workload("llama_small", GPT2Shape(12, 32000, 768, 12, 2048, 1024, 4),
                            Tiles(4, 1024, 768, 2048, 12, 768)),
    # the wide model's width with a LLaMA block (inner 22016, as LLaMA's d 8192 models)
    "llama_wide4": Workload("llama_wide4", GPT2Shape(4, 32000, 8192, 64, 22016, 1024, 4),
                            Tiles(4, 1024, 2048, 8192, 16, 2048)),
}


def param_specs(s: GPT2Shape) -> List[Tuple[str, Tuple[int, ...], str]]:
    """Ordered GPT2 parameter list: (name, shape, init kind).

    Kinds: "normal" = N(0, 0.02); "zeros"; "ones". The QKV weight is one
    [d, 3d] matrix whose column blocks are q | k | v, head j taking columns
    j*hd .. (j+1)*hd-1 of each block. The LM head is tied to wte.
    """
    d, i_, v, t = s.n_embd, s.n_inner, s.vocab, s.seq
    specs: List[Tuple[str, Tuple[int, ...], str]] = [
        ("wte", (v, d), "normal"),
        ("wpe", (t, d), "normal"),
    ]
    for l in range(s.n_layer):
        p = f"h{l}."
        specs += [
            (p + "ln1_g", (d,), "ones"), (p + "ln1_b", (d,), "zeros"),
            (p + "w_qkv", (d, 3 * d), "normal"), (p + "b_qkv", (3 * d,), "zeros"),
            (p + "w_o", (d, d), "normal"), (p + "b_o", (d,), "zeros"),
            (p + "ln2_g", (d,), "ones"), (p + "ln2_b", (d,), "zeros"),
            (p + "w_fc", (d, i_), "normal"), (p + "b_fc", (i_,), "zeros"),
            (p + "w_p", (i_, d), "normal"), (p + "b_p", (d,), "zeros"),
        ]
    specs += [("lnf_g", (d,), "ones"), ("lnf_b", (d,), "zeros")]
    return specs


def llama_param_specs(s: GPT2Shape) -> List[Tuple[str, Tuple[int, ...], str]]:
    """Ordered LLaMA-style parameter list: (name, shape, init kind).

    wte, then per block the attention RMSNorm gain, the [d, 3d] QKV weight
    (column blocks q | k | v as for GPT2), w_o, the MLP RMSNorm gain, the
    SwiGLU gate and up weights [d, I] and the down weight [I, d], then the
    final RMSNorm gain and the untied head [V, d]. No biases, no position
    table. `n_inner` is the SwiGLU hidden width.
    """
    d, i_, v = s.n_embd, s.n_inner, s.vocab
    specs: List[Tuple[str, Tuple[int, ...], str]] = [("wte", (v, d), "normal")]
    for l in range(s.n_layer):
        p = f"h{l}."
        specs += [
            (p + "attn_norm_g", (d,), "ones"), (p + "w_qkv", (d, 3 * d), "normal"),
            (p + "w_o", (d, d), "normal"), (p + "mlp_norm_g", (d,), "ones"),
            (p + "w_gate", (d, i_), "normal"), (p + "w_up", (d, i_), "normal"),
            (p + "w_down", (i_, d), "normal"),
        ]
    specs += [("norm_f_g", (d,), "ones"), ("w_head", (v, d), "normal")]
    return specs


def init_param(spec: Tuple[str, Tuple[int, ...], str], index: int, seed: int = 0,
               std: float = 0.02) -> np.ndarray:
    """One parameter tensor as float32 (normal draws are made in float64)."""
    _, shape, kind = spec
    if kind == "zeros":
        return np.zeros(shape, np.float32)
    if kind == "ones":
        return np.ones(shape, np.float32)
    rng = np.random.default_rng([seed, index])
    return (rng.standard_normal(shape) * std).astype(np.float32)


def init_params(s: GPT2Shape, seed: int = 0, std: float = 0.02, threads: int = 1,
                specs=None) -> Dict[str, np.ndarray]:
    """Every parameter, in param_specs order (or the order of `specs`, e.g.
    llama_param_specs). Each tensor has its own seeded stream, so `threads`
    (drawing several tensors at once) changes nothing but the wall time."""
    specs = param_specs(s) if specs is None else specs
    if threads <= 1:
        return {spec[0]: init_param(spec, i, seed, std) for i, spec in enumerate(specs)}
    from concurrent.futures import ThreadPoolExecutor
    with ThreadPoolExecutor(threads) as ex:
        arrs = list(ex.map(lambda a: init_param(a[1], a[0], seed, std), enumerate(specs)))
    return {spec[0]: arr for spec, arr in zip(specs, arrs)}


def token_stream(s: GPT2Shape, seed: int = 1) -> np.ndarray:
    """uint16 token windows [B, T+1], ids uniform in [0, vocab)."""
    if s.vocab > 65536:
        raise ValueError("uint16 stream needs vocab <= 65536")
    rng = np.random.default_rng(seed)
    return rng.integers(0, s.vocab, size=(s.batch, s.seq + 1)).astype(np.uint16)


def split_tokens(stream: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Inputs are the window without its last id, labels the window shifted by one."""
    s = stream.astype(np.int32)
    return np.ascontiguousarray(s[:, :-1]), np.ascontiguousarray(s[:, 1:])


def rand_normal(shape, seed: int, std: float = 1.0, dtype=np.float32) -> np.ndarray:
    rng = np.random.default_rng(seed)
    return (rng.standard_normal(shape) * std).astype(dtype)


def rand_uniform(shape, seed: int, lo: float = -1.0, hi: float = 1.0, dtype=np.float32) -> np.ndarray:
    rng = np.random.default_rng(seed)
    return rng.uniform(lo, hi, size=shape).astype(dtype)
