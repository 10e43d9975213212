"""The oracle: plain, slow, untiled float64 CPU training steps (GPT2 and a
LLaMA-style model).

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or
execute anything in this package: only the tests, the smoke check and the
CPU-baseline leg of the benchmark use it. It shares no code with the HIP
library or its Python binding; both take their inputs from ``synth``.

Modules:
  gpt2   -- untiled fp64 forward, backward, cross-entropy and AdamW step
  llama  -- the same for a LLaMA-style block (RMSNorm, rotary embedding,
            SwiGLU MLP, untied head)
  tiled  -- fp64 tile decompositions of each layer (K-split sums, LayerNorm
            statistic merges, softmax (max, sum-exp) merges, online attention
            over key tiles) that must reproduce the untiled results

Every function is pinned by tests to something other than itself (finite
differences, closed forms, invariants, torch/transformers fp64 routines).
"""
from . import gpt2, llama, tiled  # noqa: F401
