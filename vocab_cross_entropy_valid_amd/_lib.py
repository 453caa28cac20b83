"""ctypes binding of liblce.so: same names and arguments as include/lce.h.

Argument marshalling only.  Pointers are passed as integers (device
addresses from torch tensors or any other allocator); streams as the raw
hipStream_t handle.  Loading fails loudly when the library is missing: there
is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
import threading

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("LCE_LIBRARY", os.path.join(_HERE, "liblce.so"))

LCE_OK = 0
LCE_ERR_INVALID_ARG = 1
LCE_ERR_UNSUPPORTED = 2
LCE_ERR_WORKSPACE = 3
LCE_ERR_LABEL_RANGE = 4
LCE_ERR_HIP = 5

LCE_OPT_SGD = 1
LCE_OPT_ADAMW = 2

LCE_F32 = 0
LCE_BF16 = 1
LCE_MEAN = 0
LCE_SUM = 1

KERNEL_CLASSES = ("compact", "fwd", "merge", "reduce", "zero", "transpose",
                  "bwd_g", "dh", "dw", "gemm", "embed", "attn", "attn_dq", "attn_dkv",
                  "dh_dw", "cast", "mfma", "opt")

class LceOptimizer(ctypes.Structure):
    """lce_optimizer of include/lce.h."""
    _fields_ = [("kind", ctypes.c_int), ("lr", ctypes.c_float), ("weight_decay", ctypes.c_float),
                ("beta1", ctypes.c_float), ("beta2", ctypes.c_float), ("eps", ctypes.c_float),
                ("step", ctypes.c_int64)]


# name -> (restype, argtypes), in the order of include/lce.h
_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_INT = ctypes.c_int
_SZ = ctypes.c_size_t
SIGNATURES = {
    "lce_workspace_bytes": (_SZ, [_I64, _I64, _I64, _INT]),
    "lce_forward": (_INT, [_P, _P, _P, _I64, _I64, _I64, _I64, _INT, _P, _P, _P, _P, _P, _P,
                           _P, _P, _SZ, _P]),
    "lce_forward_noalloc": (_INT, [_P, _P, _P, _I64, _I64, _I64, _I64, _INT, _P, _P, _P, _P, _P,
                                   _P, _P, _P]),
    "lce_backward": (_INT, [_P, _P, _P, _I64, _P, _P, _P, _I64, _I64, _I64, _INT, _P, _INT,
                            _P, _P, _INT, _P, _SZ, _P]),
    "lce_cast_bf16": (_INT, [_P, _P, _I64, _P]),
    "lce_step_workspace_bytes": (_SZ, [_I64, _I64, _I64, _INT]),
    "lce_backward_step": (_INT, [_P, _P, _P, _I64, _P, _P, _P, _I64, _I64, _I64, _INT, _P, _INT,
                                 _P, _P, _P, _P, ctypes.POINTER(LceOptimizer), _P, _SZ, _P]),
    "lce_forward_shard": (_INT, [_P, _P, _P, _I64, _I64, _I64, _I64, _I64, _I64, _INT, _P, _P, _P,
                                 _P, _P, _P, _P, _SZ, _P]),
    "lce_lse_merge": (_INT, [_P, _P, _P, _I64, _I64, _I64, _P, _P, _P, _P, _P, _P, _P]),
    "lce_backward_shard": (_INT, [_P, _P, _P, _I64, _P, _P, _P, _I64, _I64, _I64, _I64, _I64, _INT,
                                  _P, _INT, _P, _INT, _P, _INT, _P, _SZ, _P]),
    "lce_embed_forward": (_INT, [_P, _P, _I64, _I64, _I64, _I64, _INT, _P, _P, _P, _P, _P]),
    "lce_embed_workspace_bytes": (_SZ, [_I64, _I64, _I64]),
    "lce_embed_backward": (_INT, [_P, _P, _P, _P, _I64, _I64, _I64, _P, _INT, _P, _SZ, _P]),
    "lce_attention_forward": (_INT, [_P, _P, _P, _I64, _I64, _I64, _I64, _INT, ctypes.c_float,
                                     _P, _P, _P]),
    "lce_attention_backward": (_INT, [_P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, _INT,
                                      ctypes.c_float, _P, _P, _P, _P, _P]),
    "lce_check_error": (_INT, [_P, _P]),
    "lce_status_string": (ctypes.c_char_p, [_INT]),
    "lce_last_error": (ctypes.c_char_p, []),
    "lce_gemm_nt": (_INT, [_P, _P, _P, _I64, _I64, _I64, _INT, _P]),
    "lce_mfma_peak": (_INT, [_P, _I64, _I64, _P]),
    "lce_timing_enable": (_INT, [_INT]),
    "lce_timing_reset": (_INT, []),
    "lce_timing_query": (_INT, [_INT, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(_I64)]),
}

_lib = None
_lock = threading.Lock()


class LceError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


def load(path: str = None) -> ctypes.CDLL:
    """Load liblce.so (once) and declare every exported signature."""
    global _lib
    with _lock:
        if _lib is not None and path is None:
            return _lib
        p = path or LIB_PATH
        if not os.path.exists(p):
            raise RuntimeError(
                f"liblce.so not found at {p}: build it first "
                "(python -c 'import __graft_entry__ as g; g.build()' or "
                "python vocab_cross_entropy_valid_amd/build.py)")
        lib = ctypes.CDLL(p)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        if path is None:
            _lib = lib
        return lib


def _check(status: int, what: str) -> None:
    if status != LCE_OK:
        lib = load()
        msg = lib.lce_last_error().decode() or lib.lce_status_string(status).decode()
        raise LceError(status, f"{what}: {msg}")


# ------------------------------------------------------------ thin wrappers

def lce_workspace_bytes(N: int, d: int, V: int, dtype: int) -> int:
    return int(load().lce_workspace_bytes(N, d, V, dtype))


def lce_cast_bf16(src, dst, n, stream) -> None:
    _check(load().lce_cast_bf16(src, dst, n, stream), "lce_cast_bf16")


def lce_step_workspace_bytes(N: int, d: int, V: int, dtype: int) -> int:
    return int(load().lce_step_workspace_bytes(N, d, V, dtype))


def lce_forward(H, W, labels, ignore_index, N, d, V, dtype, loss, lse, valid_idx,
                valid_count, loss_sum, loss_mean, err_flag, workspace, workspace_bytes,
                stream) -> None:
    _check(load().lce_forward(H, W, labels, ignore_index, N, d, V, dtype, loss, lse,
                              valid_idx, valid_count, loss_sum, loss_mean, err_flag,
                              workspace, workspace_bytes, stream), "lce_forward")


def lce_forward_noalloc(H, W, labels, ignore_index, N, d, V, dtype, loss, lse, valid_idx,
                        valid_count, loss_sum, loss_mean, err_flag, stream) -> None:
    _check(load().lce_forward_noalloc(H, W, labels, ignore_index, N, d, V, dtype, loss, lse,
                                      valid_idx, valid_count, loss_sum, loss_mean, err_flag,
                                      stream), "lce_forward_noalloc")


def lce_backward(H, W, labels, ignore_index, lse, valid_idx, valid_count, N, d, V, dtype,
                 grad_out, reduction, dH, dW, accumulate_dW, workspace, workspace_bytes,
                 stream) -> None:
    _check(load().lce_backward(H, W, labels, ignore_index, lse, valid_idx, valid_count, N, d,
                               V, dtype, grad_out, reduction, dH, dW, accumulate_dW,
                               workspace, workspace_bytes, stream), "lce_backward")


def lce_backward_step(H, W, labels, ignore_index, lse, valid_idx, valid_count, N, d, V, dtype,
                      grad_out, reduction, dH, W_master, exp_avg, exp_avg_sq, opt, workspace,
                      workspace_bytes, stream) -> None:
    _check(load().lce_backward_step(H, W, labels, ignore_index, lse, valid_idx, valid_count, N, d,
                                    V, dtype, grad_out, reduction, dH, W_master, exp_avg,
                                    exp_avg_sq, ctypes.byref(opt), workspace, workspace_bytes,
                                    stream), "lce_backward_step")


def lce_forward_shard(H, W_shard, labels, ignore_index, N, d, V_total, v_begin, V_shard, dtype,
                      part_max, part_sum, part_target, valid_idx, valid_count, err_flag,
                      workspace, workspace_bytes, stream) -> None:
    _check(load().lce_forward_shard(H, W_shard, labels, ignore_index, N, d, V_total, v_begin,
                                    V_shard, dtype, part_max, part_sum, part_target, valid_idx,
                                    valid_count, err_flag, workspace, workspace_bytes, stream),
           "lce_forward_shard")


def lce_lse_merge(part_max, part_sum, part_target, n_shards, shard_stride, N, valid_idx,
                  valid_count, loss, lse, loss_sum, loss_mean, stream) -> None:
    _check(load().lce_lse_merge(part_max, part_sum, part_target, n_shards, shard_stride, N,
                                valid_idx, valid_count, loss, lse, loss_sum, loss_mean, stream),
           "lce_lse_merge")


def lce_backward_shard(H, W_shard, labels, ignore_index, lse, valid_idx, valid_count, N, d,
                       V_total, v_begin, V_shard, dtype, grad_out, reduction, dH, accumulate_dH,
                       dW_shard, accumulate_dW, workspace, workspace_bytes, stream) -> None:
    _check(load().lce_backward_shard(H, W_shard, labels, ignore_index, lse, valid_idx,
                                     valid_count, N, d, V_total, v_begin, V_shard, dtype,
                                     grad_out, reduction, dH, accumulate_dH, dW_shard,
                                     accumulate_dW, workspace, workspace_bytes, stream),
           "lce_backward_shard")


def lce_embed_forward(W, input_ids, pad_id, N, d, V, dtype, X, valid_idx, valid_count, err_flag,
                      stream) -> None:
    _check(load().lce_embed_forward(W, input_ids, pad_id, N, d, V, dtype, X, valid_idx,
                                    valid_count, err_flag, stream), "lce_embed_forward")


def lce_embed_workspace_bytes(N: int, d: int, V: int) -> int:
    return int(load().lce_embed_workspace_bytes(N, d, V))


def lce_embed_backward(dX, input_ids, valid_idx, valid_count, N, d, V, dW, accumulate_dW,
                       workspace, workspace_bytes, stream) -> None:
    _check(load().lce_embed_backward(dX, input_ids, valid_idx, valid_count, N, d, V, dW,
                                     accumulate_dW, workspace, workspace_bytes, stream),
           "lce_embed_backward")


def lce_attention_forward(Q, K, V, B, H, S, D, causal, scale, O, lse, stream) -> None:
    _check(load().lce_attention_forward(Q, K, V, B, H, S, D, causal, scale, O, lse, stream),
           "lce_attention_forward")


def lce_attention_backward(Q, K, V, O, lse, dO, B, H, S, D, causal, scale, dQ, dK, dV, delta,
                           stream) -> None:
    _check(load().lce_attention_backward(Q, K, V, O, lse, dO, B, H, S, D, causal, scale, dQ, dK,
                                         dV, delta, stream), "lce_attention_backward")


def lce_check_error(err_flag, stream) -> None:
    _check(load().lce_check_error(err_flag, stream), "lce_check_error")


def lce_status_string(status: int) -> str:
    return load().lce_status_string(status).decode()


def lce_last_error() -> str:
    return load().lce_last_error().decode()


def lce_gemm_nt(A, B, C, M, N, K, dtype, stream) -> None:
    _check(load().lce_gemm_nt(A, B, C, M, N, K, dtype, stream), "lce_gemm_nt")


def lce_mfma_peak(out, n_out, iters, stream) -> None:
    _check(load().lce_mfma_peak(out, n_out, iters, stream), "lce_mfma_peak")


def lce_timing_enable(on: bool) -> None:
    _check(load().lce_timing_enable(1 if on else 0), "lce_timing_enable")


def lce_timing_reset() -> None:
    _check(load().lce_timing_reset(), "lce_timing_reset")


def lce_timing_query(kernel_class: int):
    """(total_ms, launches) for one kernel class; synchronises."""
    ms = ctypes.c_double()
    n = ctypes.c_int64()
    _check(load().lce_timing_query(kernel_class, ctypes.byref(ms), ctypes.byref(n)),
           "lce_timing_query")
    return ms.value, n.value
