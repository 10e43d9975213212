"""ctypes binding of libtiletask (include/tiletask.h), same names as the C ABI.

Argument marshalling only: device buffers may be passed as torch tensors
(their data_ptr() is used), integers (raw addresses) or None; streams as
torch.cuda.Stream, integers (hipStream_t) or None (default stream). Every
call checks the return code and raises TTError with tt_last_error().
There is no fallback: if libtiletask.so is missing the import fails.
"""
from __future__ import annotations

import ctypes as C
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("TILETASK_LIB", os.path.join(_HERE, "libtiletask.so"))

if not os.path.exists(LIB_PATH):
    raise ImportError(f"libtiletask.so not found at {LIB_PATH}: build it with "
                      "`python tile_task_transformer_amd/build.py` (hipcc, gfx950)")
# One HIP runtime per process. PyTorch-ROCm ships its own libamdhip64 and
# asks for it as "libamdhip64.so"; this library asks for "libamdhip64.so.7".
# Loaded after torch, ours resolves to torch's copy (same soname); loaded
# first, torch would bring a second runtime, and whichever initialised
# second would find no device. So torch, when present, is loaded first.
try:
    import torch  # noqa: F401
except ImportError:
    pass
lib = C.CDLL(LIB_PATH)

# ---- constants (mirror include/tiletask.h)
TT_OK, TT_ERR_ARG, TT_ERR_SHAPE, TT_ERR_OOM, TT_ERR_HIP, TT_ERR_STATE, TT_ERR_UNSUPPORTED = 0, -1, -2, -3, -4, -5, -6
TT_EPI_NONE, TT_EPI_BIAS, TT_EPI_RES, TT_EPI_GELU, TT_EPI_GELU_BWD, TT_EPI_XSTATS = 0, 1, 2, 4, 8, 16
TT_LN_PARTIAL, TT_LN_MERGE, TT_LN_APPLY, TT_LN_FUSED = 0, 1, 2, 3
TT_SM_STATS, TT_SM_MERGE, TT_SM_APPLY = 0, 1, 2
TT_XE_LOSS, TT_XE_GRAD, TT_XE_STATS = 0, 1, 2
TT_ATT_PREP, TT_ATT_GRAD = 0, 1
TT_EMB_TOKEN, TT_EMB_POS = 0, 1
TT_PROBE_READ, TT_PROBE_WRITE, TT_PROBE_COPY, TT_PROBE_NONTEMPORAL = 0, 1, 2, 4
TT_MAX_DIMS = 6
TT_F32, TT_I32 = 0, 1
TT_HOME_DEVICE, TT_HOME_PINNED_HOST, TT_HOME_PINNED_STATE = 0, 1, 2
TT_DEVICE_DRYRUN = -1
TT_R, TT_W, TT_RW = 1, 2, 3
TT_OPT_ADAMW, TT_OPT_SGD = 0, 1
TT_ADAMW_MAX_TILES = TT_SGD_MAX_TILES = TT_FILL_MAX_TILES = 16
(TT_OP_FILL, TT_OP_GEMM, TT_OP_GEMM_BATCH, TT_OP_GEMM_KSUM, TT_OP_LAYERNORM_FWD, TT_OP_LAYERNORM_BWD,
 TT_OP_ATTENTION_FWD, TT_OP_ATTENTION_PREP, TT_OP_ATTENTION_BWD, TT_OP_XENTROPY_STATS, TT_OP_XENTROPY_MERGE,
 TT_OP_XENTROPY_LOSS, TT_OP_XENTROPY_GRAD, TT_OP_ADAMW, TT_OP_ADAMW_ADVANCE, TT_OP_SGD, TT_OP_EMBEDDING_FWD,
 TT_OP_EMBEDDING_INDEX, TT_OP_EMBEDDING_BWD, TT_OP_EMBEDDING_POS_BWD, TT_OP_REDUCE_ROWS, TT_OP_SPLIT_TOKENS,
 TT_OP_COPY_IN) = range(1, 24)
(TT_OP_RMSNORM_FWD, TT_OP_RMSNORM_BWD, TT_OP_ROPE, TT_OP_ROPE_TABLE, TT_OP_SWIGLU_FWD, TT_OP_SWIGLU_BWD,
 TT_OP_EMBEDDING_TOKEN_FWD) = range(24, 31)

_ERRNAMES = {-1: "TT_ERR_ARG", -2: "TT_ERR_SHAPE", -3: "TT_ERR_OOM", -4: "TT_ERR_HIP", -5: "TT_ERR_STATE",
             -6: "TT_ERR_UNSUPPORTED"}


class TTError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{_ERRNAMES.get(code, code)}: {msg}")
        self.code = code


class tt_access(C.Structure):
    _fields_ = [("tensor", C.c_void_p), ("tile", C.c_int64 * TT_MAX_DIMS), ("mode", C.c_int)]


class tt_tile(C.Structure):
    _fields_ = [("tensor", C.c_void_p), ("tile", C.c_int64 * TT_MAX_DIMS)]


class tt_op_fill(C.Structure):
    _fields_ = [("value", C.c_float)]


class tt_op_gemm(C.Structure):
    _fields_ = [("transA", C.c_int), ("transB", C.c_int), ("epilogue", C.c_int), ("alpha", C.c_float),
                ("beta", C.c_float), ("split_k", C.c_int)]


class tt_op_layernorm(C.Structure):
    _fields_ = [("eps", C.c_float), ("dx_acc", C.c_int)]


class tt_op_attention(C.Structure):
    _fields_ = [("q_off", C.c_int64), ("k_off", C.c_int64), ("first", C.c_int), ("last", C.c_int),
                ("acc_dq", C.c_int), ("acc_dkv", C.c_int), ("scale", C.c_float)]


class tt_op_xentropy(C.Structure):
    _fields_ = [("accumulate", C.c_int), ("inv_n", C.c_float)]


class tt_op_xe_groups(C.Structure):
    _fields_ = [("vocab", C.c_int64), ("v_tile", C.c_int64), ("group", C.c_int)]


class tt_op_optim(C.Structure):
    _fields_ = [("lr", C.c_float), ("beta1", C.c_float), ("beta2", C.c_float), ("eps", C.c_float),
                ("weight_decay", C.c_float)]


class tt_op_embedding(C.Structure):
    _fields_ = [("seq_len", C.c_int64)]


class tt_op_reduce(C.Structure):
    _fields_ = [("beta", C.c_int)]


class tt_op_copy(C.Structure):
    _fields_ = [("src", C.c_void_p)]


class tt_op_rope(C.Structure):
    _fields_ = [("pos_off", C.c_int64), ("inverse", C.c_int), ("base", C.c_double)]


class tt_stats(C.Structure):
    _fields_ = [("tasks", C.c_int64), ("edges", C.c_int64), ("cross_stream_waits", C.c_int64),
                ("events_recorded", C.c_int64), ("submit_seconds", C.c_double), ("h2d_bytes", C.c_int64),
                ("d2h_bytes", C.c_int64), ("evictions", C.c_int64), ("prefetches", C.c_int64)]


class tt_profile_entry(C.Structure):
    _fields_ = [("label", C.c_char * 32), ("count", C.c_int64), ("total_ms", C.c_double), ("min_ms", C.c_double),
                ("max_ms", C.c_double)]


class tt_gpt2_config(C.Structure):
    _fields_ = [("n_layer", C.c_int), ("vocab", C.c_int), ("n_embd", C.c_int), ("n_head", C.c_int),
                ("n_inner", C.c_int), ("seq", C.c_int), ("batch", C.c_int), ("ln_eps", C.c_float)]


class tt_gpt2_tiles(C.Structure):
    _fields_ = [("batch", C.c_int), ("seq", C.c_int), ("embd", C.c_int), ("inner", C.c_int), ("head", C.c_int),
                ("vocab", C.c_int)]


class tt_adamw_hparams(C.Structure):
    _fields_ = [("lr", C.c_float), ("beta1", C.c_float), ("beta2", C.c_float), ("eps", C.c_float),
                ("weight_decay", C.c_float), ("start_lr", C.c_float), ("full_lr_iter", C.c_int),
                ("optimizer", C.c_int)]


P, I, I64, F, SZ = C.c_void_p, C.c_int, C.c_int64, C.c_float, C.c_size_t
PP = C.POINTER(C.c_void_p)

# name -> (restype, argtypes)
SIGNATURES = {
    "tt_last_error": (C.c_char_p, []),
    "tt_version": (C.c_char_p, []),
    "tt_probe_mfma_f32": (I, [P, I64, I64, P, C.POINTER(C.c_double)]),
    "tt_probe_hbm": (I, [P, I, P, P, I64, I64, C.POINTER(C.c_double)]),
    "tile_gemm": (I, [P, I, I, I64, I64, I64, F, P, I64, P, I64, F, P, I64, I, P, P, I64, P, I64]),
    "tile_gemm_ws": (I, [P, I, I, I64, I64, I64, F, P, I64, P, I64, F, P, I64, I, P, P, I64, P, I64, P, SZ]),
    "tile_gemm_workspace": (SZ, [I64, I64, I64]),
    "tile_gemm_ksum": (I, [P, I, I, I64, I64, P, F, P, P, P, P, F, P, I64]),
    "tile_gemm_ksum_ex": (I, [P, I, I, I64, I64, P, F, P, P, P, P, F, P, I64, I, P, P, I64, P, I64]),
    "tile_gemm_ksum_ws": (I, [P, I, I, I64, I64, P, F, P, P, P, P, F, P, I64, I, P, P, I64, P, I64, P, SZ]),
    "tile_gemm_ksum_workspace": (SZ, [I64, I64]),
    "tile_gemm_batch": (I, [P, I, I, I, P, P, I64, F, P, P, P, P, F, P, P]),
    "tile_gemm_batch_ws": (I, [P, I, I, I, P, P, I64, F, P, P, P, P, F, P, P, P, SZ]),
    "tile_gemm_batch_workspace": (SZ, [I, P, P, I64]),
    "tile_xentropy_multi": (I, [P, I, I, I64, P, P, P, P, P, P, I64, P, F]),
    "tile_xentropy_merge_groups": (I, [P, I64, I, P, I, P, I64, P, P]),
    "tile_gemm_batch_xstats": (I, [P, I, I, I64, P, I64, F, P, P, P, P, F, P, P, P, I64, I64, P, I64]),
    "tile_layernorm_fwd": (I, [P, I, I64, I64, P, I64, P, P, P, I64, I64, P, P, I64, F]),
    "tile_layernorm_bwd": (I, [P, I, I64, I64, I64, P, I64, P, I64, P, P, P, I64, I64, P, I64, I, P, P, P]),
    "tile_layernorm_bwd_workspace": (SZ, [I64, I64]),
    "tile_layernorm_bwd_noalloc": (I, [P, I, I64, I64, I64, P, I64, P, I64, P, P, P, I64, I64, P, I64, I, P, P]),
    "tile_layernorm_bwd_noalloc_max_bytes": (SZ, []),
    "tile_layernorm_fwd_multi": (I, [P, I, I64, P, P, P, P, P, P, F]),
    "tile_layernorm_bwd_multi": (I, [P, I, I64, P, P, P, P, P, P, I, P, P, P, SZ]),
    "tile_layernorm_bwd_multi_workspace": (SZ, [I64, I64]),
    "tile_rmsnorm_fwd": (I, [P, I, I64, P, P, P, P, P, F]),
    "tile_rmsnorm_bwd": (I, [P, I, I64, P, P, P, P, P, P, I, P, P, SZ]),
    "tile_rmsnorm_bwd_workspace": (SZ, [I64, I64]),
    "tile_rope_table": (I, [P, I64, I64, C.c_double, P]),
    "tile_rope": (I, [P, P, I64, I64, I64, I64, I64, P, I64, I]),
    "tile_rope_multi": (I, [P, I, P, I64, I64, I64, I64, I64, P, I64, I]),
    "tile_swiglu_fwd": (I, [P, I64, P, P, P]),
    "tile_swiglu_bwd": (I, [P, I64, P, P, P, P, P]),
    "tile_softmax": (I, [P, I, I64, I64, I64, I64, F, I, P, I64, P, P, I64, I64, P, P, P, I64, F]),
    "tile_xentropy": (I, [P, I, I64, I64, I64, P, P, I64, P, P, P, I, F]),
    "tile_attention_fwd": (I, [P, I64, I64, I64, I64, I64, I64, I64, P, P, P, P, P, P, I, I, F]),
    "tile_attention_bwd": (I, [P, I, I64, I64, I64, I64, I64, I64, I64, P, P, P, P, P, P, P, P, P, P, I, I, F]),
    "tile_attention_bwd_workspace": (SZ, [I64, I64, I64, I64]),
    "tile_attention_bwd_ws": (I, [P, I, I64, I64, I64, I64, I64, I64, I64, P, P, P, P, P, P, P, P, P, P, I, I, F, P,
                                  SZ]),
    "tile_fused_adamw": (I, [P, I64, P, P, P, P, F, F, F, F, F, P]),
    "tile_fused_adamw_multi": (I, [P, I, P, P, P, P, P, F, F, F, F, F, P]),
    "tile_adamw_advance": (I, [P, P, P, F, F]),
    "tile_sgd": (I, [P, I64, P, P, F]),
    "tile_sgd_multi": (I, [P, I, P, P, P, F]),
    "tile_embedding_fwd": (I, [P, I64, I64, P, I64, I64, I64, P, I64, P, I64, I64, I64, P, I64]),
    "tile_embedding_index": (I, [P, I64, P, P, P]),
    "tile_embedding_bwd": (I, [P, I, I64, I64, P, P, I64, I64, I64, P, I64, P, I64]),
    "tile_reduce_rows": (I, [P, I64, I64, P, I64, P, I, P]),
    "tile_reduce_rows_workspace": (SZ, [I64, I64]),
    "tile_reduce_rows_multi": (I, [P, I, I64, P, P, P, P, I, P, SZ]),
    "tile_fill": (I, [P, I64, P, F]),
    "tile_fill_multi": (I, [P, I, P, P, F]),
    "tile_split_tokens": (I, [P, I64, I64, P, P, P]),
    "tt_ctx_create": (I, [I, I, I, SZ, PP]),
    "tt_ctx_create_on_streams": (I, [I, I, PP, I, SZ, PP]),
    "tt_ctx_destroy": (I, [P]),
    "tt_ctx_stream": (I, [P, I, PP]),
    "tt_ctx_record": (I, [P, I]),
    "tt_ctx_streams_active": (I, [P, I]),
    "tt_ctx_heavy_lane": (I, [P, C.c_double]),
    "tt_ctx_priorities": (I, [P, I]),
    "tt_tensor_create": (I, [P, I, C.POINTER(I64), C.POINTER(I64), I, I, PP]),
    "tt_tensor_wrap": (I, [P, I, C.POINTER(I64), C.POINTER(I64), I, P, PP]),
    "tt_tensor_destroy": (I, [P]),
    "tt_tensor_bytes": (I64, [P]),
    "tt_tensor_set_matrix_split": (I, [P, I]),
    "tt_tensor_grid": (I, [P, C.POINTER(I64), C.POINTER(I64)]),
    "tt_tensor_tile": (I, [P, C.POINTER(I64), PP, C.POINTER(I64)]),
    "tt_tensor_copy_in": (I, [P, P]),
    "tt_tensor_copy_out": (I, [P, P]),
    "tt_submit_nop": (I, [P, C.c_char_p, C.POINTER(tt_access), I]),
    "tt_submit_gemm": (I, [P, I, I, F, P, C.POINTER(I64), P, C.POINTER(I64), F, P, C.POINTER(I64)]),
    "tt_submit_fill": (I, [P, P, C.POINTER(I64), F]),
    "tt_submit": (I, [P, I, C.POINTER(tt_tile), I, P, SZ]),
    "tt_ctx_wait_stream": (I, [P, P]),
    "tt_ctx_join_stream": (I, [P, P]),
    "tt_wait": (I, [P]),
    "tt_dump_dag": (I, [P, C.c_char_p]),
    "tt_get_stats": (I, [P, C.POINTER(tt_stats)]),
    "tt_ctx_profile": (I, [P, C.c_char_p]),
    "tt_profile_read": (I, [P, C.POINTER(tt_profile_entry), I, C.POINTER(I)]),
    "tt_profile_busy": (I, [P, C.POINTER(C.c_double), C.POINTER(C.c_double), C.POINTER(I64)]),
    "tt_ctx_profile_every": (I, [P, I]),
    "tt_reset_stats": (I, [P]),
    "tt_gpt2_create": (I, [P, C.POINTER(tt_gpt2_config), C.POINTER(tt_gpt2_tiles), I, PP]),
    "tt_llama_create": (I, [P, C.POINTER(tt_gpt2_config), C.POINTER(tt_gpt2_tiles), I, PP]),
    "tt_gpt2_destroy": (I, [P]),
    "tt_gpt2_num_params": (I, [P, C.POINTER(I)]),
    "tt_gpt2_param": (I, [P, I, PP, PP, PP, PP]),
    "tt_gpt2_step": (I, [P, P, C.POINTER(tt_adamw_hparams), I]),
    "tt_gpt2_loss": (I, [P, C.POINTER(F)]),
    "tt_gpt2_task_count": (I, [P, C.POINTER(I64)]),
    "tt_gpt2_row_losses": (I, [P, C.POINTER(F)]),
    "tt_gpt2_set_replay": (I, [P, I]),
    "tt_gpt2_step_accum": (I, [P, P, I, C.POINTER(tt_adamw_hparams), I]),
}

for _name, (_res, _args) in SIGNATURES.items():
    _fn = getattr(lib, _name)
    _fn.restype = _res
    _fn.argtypes = _args


def last_error() -> str:
    return lib.tt_last_error().decode()


def check(rc: int) -> int:
    if rc != TT_OK:
        raise TTError(rc, last_error())
    return rc


def ptr(x) -> int | None:
    """Device/host address of a torch tensor, numpy array, int or None."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if hasattr(x, "data_ptr"):
        return x.data_ptr()
    if hasattr(x, "ctypes"):
        return x.ctypes.data
    raise TypeError(f"cannot take the address of {type(x)}")


def stream_handle(s) -> int | None:
    if s is None:
        return None
    if isinstance(s, int):
        return s
    if hasattr(s, "cuda_stream"):
        return s.cuda_stream
    raise TypeError(f"not a stream: {type(s)}")


def i64_array(vals):
    arr = (C.c_int64 * TT_MAX_DIMS)()
    for i, v in enumerate(vals):
        arr[i] = int(v)
    return arr
