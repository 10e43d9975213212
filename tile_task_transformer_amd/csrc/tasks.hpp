// Task-level tile ops: one call builds the access list (which tiles a task
// reads and writes) and the launch of one tile op over tiled tensors, and
// hands both to the sequential-task-flow executor. tt_submit (the C ABI)
// and the GPT2 step both submit their tasks through submit_op.
#pragma once

#include "runtime.hpp"

namespace tt {

struct TileArg {
  tt_tensor* t = nullptr;
  int64_t lin = -1;
};

// Submits task-level op `op` (TT_OP_*) over `tiles` with its scalar block
// (`size` must equal the op's scalar struct size). label = task label for
// timing and the DAG dump (NULL = the op's name). grow_ws: enlarge the
// context's per-stream workspaces when the op could use more (split-K,
// partial sums); otherwise the op uses what the context has and fails at
// launch only where a workspace is required and too small.
int submit_op(tt_ctx* ctx, int op, const TileArg* tiles, int n, const void* scalars, size_t size,
              const char* label = nullptr, bool grow_ws = true);

// Workspace bytes op TT_OP_LAYERNORM_FWD / _BWD needs for n feature tiles
// of `rows` rows, the widest `cols` columns.
size_t layernorm_fwd_workspace(int64_t n, int64_t rows);
size_t layernorm_bwd_workspace(int64_t n, int64_t rows, int64_t cols);

}  // namespace tt
