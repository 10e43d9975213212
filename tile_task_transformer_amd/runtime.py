"""Tiled tensors, the task executor and the GPT2 step: thin object wrappers
over the C ABI (tt_ctx_*, tt_tensor_*, tt_submit_*, tt_gpt2_*)."""
from __future__ import annotations

import ctypes as C
import json
from typing import Dict, List, Sequence

import numpy as np

from . import _lib as L
from ._lib import check, lib


class Context:
    """Executor context: `device` = GPU ordinal, or L.TT_DEVICE_DRYRUN to
    record tasks without a GPU."""

    def __init__(self, device: int = 0, n_streams: int = 4, window: int = 0, device_budget: int = 0,
                 streams=None):
        """streams: optional sequence of n_streams caller-owned streams (torch
        streams or raw hipStream_t handles) for the tasks
        (tt_ctx_create_on_streams); they must outlive the context."""
        h = C.c_void_p()
        if streams is not None:
            handles = (C.c_void_p * max(1, len(streams)))(*[L.stream_handle(x) for x in streams])
            check(lib.tt_ctx_create_on_streams(device, len(streams), handles, window, device_budget, C.byref(h)))
            n_streams = len(streams)
        else:
            check(lib.tt_ctx_create(device, n_streams, window, device_budget, C.byref(h)))
        self.h = h
        self.n_streams = n_streams
        self.dryrun = device == L.TT_DEVICE_DRYRUN
        self._tensors: List["Tensor"] = []

    def close(self):
        if self.h:
            for t in self._tensors:
                t.h = None  # destroyed with the context
            # the context is freed even when destroy reports a latched error
            h, self.h = self.h, None
            check(lib.tt_ctx_destroy(h))

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def stream(self, i: int = 0) -> int:
        s = C.c_void_p()
        check(lib.tt_ctx_stream(self.h, i, C.byref(s)))
        return s.value or 0

    def streams_active(self, n: int):
        """Launch later tasks on streams 0..n-1 only (1 = one stream, in order)."""
        check(lib.tt_ctx_streams_active(self.h, n))

    def heavy_lane(self, min_flops: float):
        """Tasks of at least min_flops on stream 0 in order, the rest on the
        other streams (0 = off)."""
        check(lib.tt_ctx_heavy_lane(self.h, float(min_flops)))

    def priorities(self, on: bool = True):
        """Launch each window by critical-path priority (device homes only)."""
        check(lib.tt_ctx_priorities(self.h, int(on)))

    def record(self, on: bool = True):
        check(lib.tt_ctx_record(self.h, int(on)))

    def tensor(self, shape: Sequence[int], tile: Sequence[int], dtype: int = L.TT_F32,
               home: int = L.TT_HOME_DEVICE) -> "Tensor":
        t = Tensor(self, shape, tile, dtype, home)
        self._tensors.append(t)
        return t

    def submit_nop(self, label: str, accesses):
        """accesses: iterable of (Tensor, tile index tuple, mode)."""
        acc = list(accesses)
        arr = (L.tt_access * max(1, len(acc)))()
        for i, (t, idx, mode) in enumerate(acc):
            arr[i].tensor = t.h
            for j, v in enumerate(idx):
                arr[i].tile[j] = v
            arr[i].mode = mode
        check(lib.tt_submit_nop(self.h, label.encode(), arr, len(acc)))

    def submit_gemm(self, transA, transB, alpha, A, ia, B, ib, beta, Cc, ic):
        check(lib.tt_submit_gemm(self.h, transA, transB, alpha, A.h, L.i64_array(ia), B.h, L.i64_array(ib), beta,
                                 Cc.h, L.i64_array(ic)))

    def submit_fill(self, t, idx, value: float):
        check(lib.tt_submit_fill(self.h, t.h, L.i64_array(idx), value))

    def submit(self, op: int, tiles, scalars=None):
        """Generic task submission (tt_submit): `tiles` is a sequence of
        (Tensor, tile index tuple) in the op's order, `scalars` the op's
        ctypes scalar struct (L.tt_op_*) or None."""
        tl = list(tiles)
        arr = (L.tt_tile * max(1, len(tl)))()
        for i, (t, idx) in enumerate(tl):
            arr[i].tensor = t.h
            for j, v in enumerate(idx):
                arr[i].tile[j] = int(v)
        sp = C.cast(C.byref(scalars), C.c_void_p) if scalars is not None else None
        check(lib.tt_submit(self.h, op, arr, len(tl), sp, C.sizeof(scalars) if scalars is not None else 0))

    def wait_stream(self, stream):
        """Tasks launched from now on run after the work queued on `stream`
        (a torch stream or a raw hipStream_t) so far (device-side)."""
        check(lib.tt_ctx_wait_stream(self.h, L.stream_handle(stream)))

    def join_stream(self, stream):
        """Work queued on `stream` from now on runs after every task the
        context has launched (device-side)."""
        check(lib.tt_ctx_join_stream(self.h, L.stream_handle(stream)))

    def wait(self):
        check(lib.tt_wait(self.h))

    def dump_dag(self, path: str) -> List[dict]:
        check(lib.tt_dump_dag(self.h, path.encode()))
        with open(path) as f:
            return [json.loads(line) for line in f if line.strip()]

    def stats(self) -> Dict[str, float]:
        s = L.tt_stats()
        check(lib.tt_get_stats(self.h, C.byref(s)))
        return {k: getattr(s, k) for k, _ in L.tt_stats._fields_}

    def reset_stats(self):
        check(lib.tt_reset_stats(self.h))

    def profile(self, label_filter, every: int = 1):
        """Time tasks with this label ("*" = all, None = off) with event
        pairs; every > 1 times only each every-th matching task."""
        check(lib.tt_ctx_profile_every(self.h, every))
        check(lib.tt_ctx_profile(self.h, None if label_filter is None else label_filter.encode()))

    def profile_take(self) -> Dict[str, dict]:
        """Wait, return {label: {count, total_ms, min_ms, max_ms}} and clear."""
        buf = (L.tt_profile_entry * 256)()
        n = C.c_int()
        check(lib.tt_profile_read(self.h, buf, 256, C.byref(n)))
        return {buf[i].label.decode(): dict(count=buf[i].count, total_ms=buf[i].total_ms, min_ms=buf[i].min_ms,
                                            max_ms=buf[i].max_ms) for i in range(min(n.value, 256))}


    def profile_busy(self) -> dict:
        """Wait; {busy_ms, span_ms, tasks} of the tasks timed since profile()
        (busy = union of their GPU intervals), and clear them."""
        busy, span, n = C.c_double(), C.c_double(), C.c_int64()
        check(lib.tt_profile_busy(self.h, C.byref(busy), C.byref(span), C.byref(n)))
        return dict(busy_ms=busy.value, span_ms=span.value, tasks=n.value)


class Tensor:
    def __init__(self, ctx: Context, shape, tile, dtype=L.TT_F32, home=L.TT_HOME_DEVICE, handle=None):
        self.ctx = ctx
        self.shape = tuple(int(s) for s in shape)
        self.tile = tuple(int(s) for s in tile)
        self.dtype = dtype
        if handle is None:
            h = C.c_void_p()
            check(lib.tt_tensor_create(ctx.h, len(self.shape), L.i64_array(self.shape), L.i64_array(self.tile),
                                       dtype, home, C.byref(h)))
            self.h = h
        else:
            self.h = handle

    @property
    def np_dtype(self):
        return np.float32 if self.dtype == L.TT_F32 else np.int32

    def grid(self):
        g = L.i64_array([0] * L.TT_MAX_DIMS)
        n = C.c_int64()
        check(lib.tt_tensor_grid(self.h, g, C.byref(n)))
        return tuple(g[i] for i in range(len(self.shape))), n.value

    def set_matrix_split(self, k: int):
        """Rows of a tile's matrix view = product of the first k extents."""
        check(lib.tt_tensor_set_matrix_split(self.h, k))
        return self

    def nbytes(self) -> int:
        return lib.tt_tensor_bytes(self.h)

    def tile_ptr(self, idx):
        p = C.c_void_p()
        ext = L.i64_array([0] * L.TT_MAX_DIMS)
        check(lib.tt_tensor_tile(self.h, L.i64_array(idx), C.byref(p), ext))
        return p.value, tuple(ext[i] for i in range(len(self.shape)))

    def copy_in(self, dense: np.ndarray):
        a = np.ascontiguousarray(dense, dtype=self.np_dtype)
        if a.size != int(np.prod(self.shape)):
            raise ValueError(f"copy_in: {a.shape} does not match {self.shape}")
        check(lib.tt_tensor_copy_in(self.h, a.ctypes.data))

    def copy_out(self) -> np.ndarray:
        a = np.empty(self.shape, dtype=self.np_dtype)
        check(lib.tt_tensor_copy_out(self.h, a.ctypes.data))
        return a

    def destroy(self):
        if self.h:
            check(lib.tt_tensor_destroy(self.h))
            self.h = None


class GPT2:
    """The GPT2 training step of libtiletask. `shape`/`tiles` are synth.GPT2Shape
    / synth.Tiles-like objects (attribute access)."""

    def __init__(self, ctx: Context, shape, tiles, param_home: int = L.TT_HOME_DEVICE, ln_eps: float = 1e-5,
                 family: str = "gpt2"):
        """family "gpt2" (tt_gpt2_create) or "llama" (tt_llama_create: the
        LLaMA-style block; ln_eps is then the RMSNorm eps)."""
        self.ctx = ctx
        self.shape = shape
        self.family = family
        create = {"gpt2": lib.tt_gpt2_create, "llama": lib.tt_llama_create}[family]
        cfg = L.tt_gpt2_config(shape.n_layer, shape.vocab, shape.n_embd, shape.n_head, shape.n_inner, shape.seq,
                               shape.batch, ln_eps)
        tl = L.tt_gpt2_tiles(tiles.batch, tiles.seq, tiles.embd, tiles.inner, tiles.head, tiles.vocab)
        h = C.c_void_p()
        check(create(ctx.h, C.byref(cfg), C.byref(tl), param_home, C.byref(h)))
        self.h = h
        n = C.c_int()
        check(lib.tt_gpt2_num_params(self.h, C.byref(n)))
        self.n_params = n.value

    def tensors(self, index: int):
        """(param, grad, m, v) Tensor wrappers of parameter `index`."""
        hs = [C.c_void_p() for _ in range(4)]
        check(lib.tt_gpt2_param(self.h, index, *[C.byref(x) for x in hs]))
        return [Tensor(self.ctx, (), (), L.TT_F32, handle=x) for x in hs]

    def _wrap(self, index: int, which: int, shape) -> Tensor:
        t = self.tensors(index)[which]
        t.shape = tuple(shape)
        return t

    def set_params(self, params: Dict[str, np.ndarray], specs):
        for i, (name, shp, _) in enumerate(specs):
            self._wrap(i, 0, shp).copy_in(params[name])

    def get(self, specs, which: int) -> Dict[str, np.ndarray]:
        """which: 0 params, 1 grads, 2 first moments, 3 second moments."""
        return {name: self._wrap(i, which, shp).copy_out() for i, (name, shp, _) in enumerate(specs)}

    def step(self, tokens_dev, lr=3e-4, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.1, update=True,
             n_micro=1, start_lr=None, full_lr_iter=1, optimizer="adamw"):
        """One optimiser step. tokens_dev: int32 [n_micro * batch, seq + 1] on
        the GPU (n_micro minibatches whose gradients accumulate); warm-up:
        start_lr at the first update, lr from update full_lr_iter on;
        optimizer "adamw" or "sgd" (plain p -= lr*g)."""
        opt = {"adamw": L.TT_OPT_ADAMW, "sgd": L.TT_OPT_SGD}[optimizer]
        cur = None
        if hasattr(tokens_dev, "device") and getattr(tokens_dev.device, "type", "") == "cuda":
            # the executor's streams do not order after torch's: they wait (on
            # the device, the host does not block) for the work torch has
            # queued so far, which includes whatever wrote the token buffer
            import torch
            cur = torch.cuda.current_stream(tokens_dev.device)
            self.ctx.wait_stream(cur)
        hp = L.tt_adamw_hparams(lr, beta1, beta2, eps, weight_decay, lr if start_lr is None else start_lr,
                                full_lr_iter, opt)
        check(lib.tt_gpt2_step_accum(self.h, L.ptr(tokens_dev), n_micro, C.byref(hp), int(update)))
        if cur is not None:
            # the step's copy of the token buffer is queued on an executor
            # stream when the call returns; torch's later work (which may
            # reuse the buffer's memory once the caller drops it) runs after it
            self.ctx.join_stream(cur)

    def loss(self) -> float:
        f = C.c_float()
        check(lib.tt_gpt2_loss(self.h, C.byref(f)))
        return f.value

    def set_replay(self, on: bool = True):
        """Record the step into a HIP graph once and replay it (same tokens
        buffer and hyperparameters)."""
        check(lib.tt_gpt2_set_replay(self.h, int(on)))

    def row_losses(self) -> np.ndarray:
        """Per-token losses [batch, seq] of the last step's forward."""
        out = np.empty((self.shape.batch, self.shape.seq), np.float32)
        check(lib.tt_gpt2_row_losses(self.h, out.ctypes.data_as(C.POINTER(C.c_float))))
        return out

    def task_count(self) -> int:
        n = C.c_int64()
        check(lib.tt_gpt2_task_count(self.h, C.byref(n)))
        return n.value

    def close(self):
        if self.h:
            h, self.h = self.h, None
            check(lib.tt_gpt2_destroy(h))
