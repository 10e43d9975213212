"""tile_task_transformer_amd: a GPT2 training step as tile tasks on one MI355X.

Python face of libtiletask (include/tiletask.h). Three levels, same names as
the C ABI:
  * tile ops   -- tile_gemm, tile_layernorm_fwd/bwd, tile_softmax,
                  tile_xentropy, tile_attention_fwd/bwd, tile_fused_adamw and
                  the auxiliary embedding / reduction / fill ops;
  * tasks      -- Context, Tensor (tiled tensors) and the sequential-task-flow
                  executor (tt_submit_*, tt_wait, tt_dump_dag);
  * the model  -- GPT2, whose step() submits forward, backward and AdamW as
                  tile tasks.
Every compute step runs in the HIP library; this package only marshals
arguments. Importing it fails if libtiletask.so has not been built.
"""
from ._lib import TTError, lib  # noqa: F401
from .ops import *  # noqa: F401,F403
from .runtime import Context, Tensor, GPT2  # noqa: F401
