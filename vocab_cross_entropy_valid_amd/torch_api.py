"""PyTorch-facing wrapper over the C ABI.

PyTorch supplies device memory and the current stream; every step of the
computation runs in liblce's HIP kernels.  ``linear_cross_entropy`` has the
semantics of ``F.cross_entropy(H @ W.T, labels, ignore_index=..., reduction=...)``
without materialising ``H @ W.T``.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import torch

from . import _lib

_DTYPES = {torch.bfloat16: _lib.LCE_BF16, torch.float32: _lib.LCE_F32}
_RED = {"mean": _lib.LCE_MEAN, "sum": _lib.LCE_SUM}


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _check_inputs(H: torch.Tensor, W: torch.Tensor, labels: torch.Tensor):
    if H.dim() != 2 or W.dim() != 2 or labels.dim() != 1:
        raise ValueError("H must be [N, d], W [V, d] and labels [N]")
    if H.shape[1] != W.shape[1] or H.shape[0] != labels.shape[0]:
        raise ValueError(f"shape mismatch: H {tuple(H.shape)}, W {tuple(W.shape)}, "
                         f"labels {tuple(labels.shape)}")
    if H.dtype != W.dtype or H.dtype not in _DTYPES:
        raise ValueError("H and W must both be bfloat16 or both float32")
    if labels.dtype != torch.int64:
        raise ValueError("labels must be int64")
    for t in (H, W, labels):
        if not t.is_cuda:
            raise ValueError("all tensors must be on the GPU")
        if not t.is_contiguous():
            raise ValueError("all tensors must be contiguous")
    if not (H.device == W.device == labels.device):
        raise ValueError("all tensors must be on the same device")


def workspace_bytes(N: int, d: int, V: int, dtype: torch.dtype) -> int:
    return _lib.lce_workspace_bytes(N, d, V, _DTYPES[dtype])


def step_workspace_bytes(N: int, d: int, V: int, dtype: torch.dtype) -> int:
    return _lib.lce_step_workspace_bytes(N, d, V, _DTYPES[dtype])


def alloc_workspace(N: int, d: int, V: int, dtype: torch.dtype, device,
                    step: bool = False) -> torch.Tensor:
    """Workspace for lce_forward / lce_backward (step=True: also lce_backward_step)."""
    n = (step_workspace_bytes if step else workspace_bytes)(N, d, V, dtype)
    if n == 0:
        raise ValueError(f"unsupported sizes N={N} d={d} V={V}")
    return torch.empty(n, dtype=torch.uint8, device=device)


@dataclasses.dataclass
class ForwardOut:
    loss: torch.Tensor         # f32 [N], 0 on ignored rows
    lse: torch.Tensor          # f32 [N], 0 on ignored rows
    valid_idx: torch.Tensor    # int32 [N]; first valid_count entries meaningful
    valid_count: torch.Tensor  # int32 [1]
    loss_sum: torch.Tensor     # f64 [1]
    loss_mean: torch.Tensor    # f32 [1]
    err_flag: torch.Tensor     # int32 [1]


def forward(H: torch.Tensor, W: torch.Tensor, labels: torch.Tensor, ignore_index: int = -100,
            workspace: Optional[torch.Tensor] = None, check: bool = True) -> ForwardOut:
    """lce_forward on the current stream.  With check=True the error flag is
    read back (one synchronisation) and a bad label raises ValueError."""
    _check_inputs(H, W, labels)
    N, d = H.shape
    V = W.shape[0]
    dev = H.device
    dt = _DTYPES[H.dtype]
    if workspace is None:
        workspace = alloc_workspace(N, d, V, H.dtype, dev)
    f32 = dict(dtype=torch.float32, device=dev)
    out = ForwardOut(
        loss=torch.empty(N, **f32), lse=torch.empty(N, **f32),
        valid_idx=torch.empty(N, dtype=torch.int32, device=dev),
        valid_count=torch.empty(1, dtype=torch.int32, device=dev),
        loss_sum=torch.empty(1, dtype=torch.float64, device=dev),
        loss_mean=torch.empty(1, **f32),
        err_flag=torch.empty(1, dtype=torch.int32, device=dev))
    s = _stream(dev)
    _lib.lce_forward(_ptr(H), _ptr(W), _ptr(labels), int(ignore_index), N, d, V, dt,
                     _ptr(out.loss), _ptr(out.lse), _ptr(out.valid_idx), _ptr(out.valid_count),
                     _ptr(out.loss_sum), _ptr(out.loss_mean), _ptr(out.err_flag),
                     _ptr(workspace), workspace.numel(), s)
    if check:
        try:
            _lib.lce_check_error(_ptr(out.err_flag), s)
        except _lib.LceError as e:
            if e.status == _lib.LCE_ERR_LABEL_RANGE:
                raise ValueError(str(e)) from e
            raise
    return out


def backward(H: torch.Tensor, W: torch.Tensor, labels: torch.Tensor, fwd: ForwardOut,
             grad_out: Optional[torch.Tensor] = None, reduction: str = "mean",
             ignore_index: int = -100, dH: Optional[torch.Tensor] = None,
             dW: Optional[torch.Tensor] = None, accumulate_dW: bool = False,
             workspace: Optional[torch.Tensor] = None):
    """lce_backward on the current stream; returns (dH, dW) in float32."""
    _check_inputs(H, W, labels)
    N, d = H.shape
    V = W.shape[0]
    dev = H.device
    if reduction not in _RED:
        raise ValueError("reduction must be 'mean' or 'sum'")
    if grad_out is None:
        grad_out = torch.ones(1, dtype=torch.float32, device=dev)
    grad_out = grad_out.reshape(1).to(device=dev, dtype=torch.float32).contiguous()
    if workspace is None:
        workspace = alloc_workspace(N, d, V, H.dtype, dev)
    if dH is None:
        dH = torch.empty(N, d, dtype=torch.float32, device=dev)
    if dW is None:
        if accumulate_dW:
            raise ValueError("accumulate_dW needs dW")
        dW = torch.empty(V, d, dtype=torch.float32, device=dev)
    for t, shp in ((dH, (N, d)), (dW, (V, d))):
        if t.dtype != torch.float32 or tuple(t.shape) != shp or not t.is_contiguous():
            raise ValueError("dH and dW must be contiguous float32 of shapes [N, d] and [V, d]")
    _lib.lce_backward(_ptr(H), _ptr(W), _ptr(labels), int(ignore_index), _ptr(fwd.lse),
                      _ptr(fwd.valid_idx), _ptr(fwd.valid_count), N, d, V, _DTYPES[H.dtype],
                      _ptr(grad_out), _RED[reduction], _ptr(dH), _ptr(dW),
                      1 if accumulate_dW else 0, _ptr(workspace), workspace.numel(),
                      _stream(dev))
    return dH, dW


# ----------------------------------------------- fused optimizer update

def backward_step(H: torch.Tensor, W: torch.Tensor, labels: torch.Tensor, fwd: ForwardOut,
                  kind: str, lr: float, weight_decay: float = 0.0, betas=(0.9, 0.999),
                  eps: float = 1e-8, step: int = 1, W_master: Optional[torch.Tensor] = None,
                  exp_avg: Optional[torch.Tensor] = None,
                  exp_avg_sq: Optional[torch.Tensor] = None,
                  grad_out: Optional[torch.Tensor] = None, reduction: str = "mean",
                  ignore_index: int = -100, dH: Optional[torch.Tensor] = None,
                  workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """lce_backward_step: dH is returned, W (and W_master, exp_avg, exp_avg_sq)
    are updated in place by SGD (kind='sgd') or AdamW (kind='adamw')."""
    _check_inputs(H, W, labels)
    N, d = H.shape
    V = W.shape[0]
    dev = H.device
    if reduction not in _RED:
        raise ValueError("reduction must be 'mean' or 'sum'")
    kinds = {"sgd": _lib.LCE_OPT_SGD, "adamw": _lib.LCE_OPT_ADAMW}
    if kind not in kinds:
        raise ValueError("kind must be 'sgd' or 'adamw'")
    for t in (W_master, exp_avg, exp_avg_sq):
        if t is not None and (t.dtype != torch.float32 or tuple(t.shape) != (V, d)
                              or not t.is_contiguous()):
            raise ValueError("W_master, exp_avg and exp_avg_sq must be contiguous float32 [V, d]")
    if grad_out is None:
        grad_out = torch.ones(1, dtype=torch.float32, device=dev)
    grad_out = grad_out.reshape(1).to(device=dev, dtype=torch.float32).contiguous()
    if workspace is None:
        workspace = alloc_workspace(N, d, V, H.dtype, dev, step=True)
    if dH is None:
        dH = torch.empty(N, d, dtype=torch.float32, device=dev)
    opt = _lib.LceOptimizer(kind=kinds[kind], lr=lr, weight_decay=weight_decay,
                            beta1=betas[0], beta2=betas[1], eps=eps, step=step)
    _lib.lce_backward_step(_ptr(H), _ptr(W), _ptr(labels), int(ignore_index), _ptr(fwd.lse),
                           _ptr(fwd.valid_idx), _ptr(fwd.valid_count), N, d, V, _DTYPES[H.dtype],
                           _ptr(grad_out), _RED[reduction], _ptr(dH), _ptr(W_master),
                           _ptr(exp_avg), _ptr(exp_avg_sq), opt, _ptr(workspace),
                           workspace.numel(), _stream(dev))
    return dH


# ------------------------------------------------------ vocabulary shards

@dataclasses.dataclass
class ShardPartials:
    part_max: torch.Tensor     # f32 [N]: largest logit over the shard (0 on ignored rows)
    part_sum: torch.Tensor     # f32 [N]: sum over the shard of exp(logit - part_max)
    part_target: torch.Tensor  # f32 [N]: target logit if the label is in the shard, else -inf
    valid_idx: torch.Tensor
    valid_count: torch.Tensor
    err_flag: torch.Tensor


def forward_shard(H: torch.Tensor, W_shard: torch.Tensor, labels: torch.Tensor, V_total: int,
                  v_begin: int, ignore_index: int = -100,
                  workspace: Optional[torch.Tensor] = None,
                  out: Optional[ShardPartials] = None) -> ShardPartials:
    """lce_forward_shard: W_shard holds vocabulary rows [v_begin, v_begin + V_shard)."""
    _check_inputs(H, W_shard, labels)
    N, d = H.shape
    Vs = W_shard.shape[0]
    dev = H.device
    if workspace is None:
        workspace = alloc_workspace(N, d, Vs, H.dtype, dev)
    if out is None:
        f32 = dict(dtype=torch.float32, device=dev)
        out = ShardPartials(
            part_max=torch.empty(N, **f32), part_sum=torch.empty(N, **f32),
            part_target=torch.empty(N, **f32),
            valid_idx=torch.empty(N, dtype=torch.int32, device=dev),
            valid_count=torch.empty(1, dtype=torch.int32, device=dev),
            err_flag=torch.empty(1, dtype=torch.int32, device=dev))
    _lib.lce_forward_shard(_ptr(H), _ptr(W_shard), _ptr(labels), int(ignore_index), N, d,
                           int(V_total), int(v_begin), Vs, _DTYPES[H.dtype], _ptr(out.part_max),
                           _ptr(out.part_sum), _ptr(out.part_target), _ptr(out.valid_idx),
                           _ptr(out.valid_count), _ptr(out.err_flag), _ptr(workspace),
                           workspace.numel(), _stream(dev))
    return out


def lse_merge(part_max: torch.Tensor, part_sum: torch.Tensor, part_target: torch.Tensor,
              valid_idx: torch.Tensor, valid_count: torch.Tensor) -> ForwardOut:
    """lce_lse_merge over stacked shard partials of shape [n_shards, N]."""
    if part_max.dim() != 2 or part_max.shape != part_sum.shape or part_max.shape != part_target.shape:
        raise ValueError("partials must be three [n_shards, N] tensors")
    for t in (part_max, part_sum, part_target):
        if t.dtype != torch.float32 or not t.is_contiguous() or not t.is_cuda:
            raise ValueError("partials must be contiguous float32 GPU tensors")
    n_shards, N = part_max.shape
    dev = part_max.device
    f32 = dict(dtype=torch.float32, device=dev)
    out = ForwardOut(
        loss=torch.empty(N, **f32), lse=torch.empty(N, **f32), valid_idx=valid_idx,
        valid_count=valid_count, loss_sum=torch.empty(1, dtype=torch.float64, device=dev),
        loss_mean=torch.empty(1, **f32), err_flag=torch.zeros(1, dtype=torch.int32, device=dev))
    _lib.lce_lse_merge(_ptr(part_max), _ptr(part_sum), _ptr(part_target), n_shards, N, N,
                       _ptr(valid_idx), _ptr(valid_count), _ptr(out.loss), _ptr(out.lse),
                       _ptr(out.loss_sum), _ptr(out.loss_mean), _stream(dev))
    return out


def backward_shard(H: torch.Tensor, W_shard: torch.Tensor, labels: torch.Tensor, V_total: int,
                   v_begin: int, merged: ForwardOut, dH: torch.Tensor, accumulate_dH: bool,
                   grad_out: Optional[torch.Tensor] = None, reduction: str = "mean",
                   ignore_index: int = -100, dW_shard: Optional[torch.Tensor] = None,
                   accumulate_dW: bool = False, workspace: Optional[torch.Tensor] = None):
    """lce_backward_shard; returns dW_shard (dH is updated in place)."""
    _check_inputs(H, W_shard, labels)
    N, d = H.shape
    Vs = W_shard.shape[0]
    dev = H.device
    if reduction not in _RED:
        raise ValueError("reduction must be 'mean' or 'sum'")
    if grad_out is None:
        grad_out = torch.ones(1, dtype=torch.float32, device=dev)
    grad_out = grad_out.reshape(1).to(device=dev, dtype=torch.float32).contiguous()
    if workspace is None:
        workspace = alloc_workspace(N, d, Vs, H.dtype, dev)
    if dW_shard is None:
        if accumulate_dW:
            raise ValueError("accumulate_dW needs dW_shard")
        dW_shard = torch.empty(Vs, d, dtype=torch.float32, device=dev)
    for t, shp in ((dH, (N, d)), (dW_shard, (Vs, d))):
        if t.dtype != torch.float32 or tuple(t.shape) != shp or not t.is_contiguous():
            raise ValueError("dH and dW_shard must be contiguous float32 [N, d] and [V_shard, d]")
    _lib.lce_backward_shard(_ptr(H), _ptr(W_shard), _ptr(labels), int(ignore_index),
                            _ptr(merged.lse), _ptr(merged.valid_idx), _ptr(merged.valid_count),
                            N, d, int(V_total), int(v_begin), Vs, _DTYPES[H.dtype],
                            _ptr(grad_out), _RED[reduction], _ptr(dH), 1 if accumulate_dH else 0,
                            _ptr(dW_shard), 1 if accumulate_dW else 0, _ptr(workspace),
                            workspace.numel(), _stream(dev))
    return dW_shard


# -------------------------------------------- tied table: input side

@dataclasses.dataclass
class EmbedOut:
    X: torch.Tensor            # [N, d], dtype of W; zero rows at padding positions
    valid_idx: torch.Tensor    # int32 [N]; first valid_count entries meaningful
    valid_count: torch.Tensor  # int32 [1]
    err_flag: torch.Tensor     # int32 [1]


def embed_forward(W: torch.Tensor, input_ids: torch.Tensor, pad_id: int) -> EmbedOut:
    """lce_embed_forward: X = W[input_ids] where input_ids != pad_id, else 0."""
    if W.dim() != 2 or input_ids.dim() != 1 or input_ids.dtype != torch.int64:
        raise ValueError("W must be [V, d] and input_ids int64 [N]")
    if W.dtype not in _DTYPES or not (W.is_cuda and input_ids.is_cuda):
        raise ValueError("W must be a bfloat16 or float32 GPU tensor, input_ids on the GPU")
    if not (W.is_contiguous() and input_ids.is_contiguous()):
        raise ValueError("W and input_ids must be contiguous")
    V, d = W.shape
    N = input_ids.shape[0]
    dev = W.device
    out = EmbedOut(X=torch.empty(N, d, dtype=W.dtype, device=dev),
                   valid_idx=torch.empty(N, dtype=torch.int32, device=dev),
                   valid_count=torch.empty(1, dtype=torch.int32, device=dev),
                   err_flag=torch.empty(1, dtype=torch.int32, device=dev))
    _lib.lce_embed_forward(_ptr(W), _ptr(input_ids), int(pad_id), N, d, V, _DTYPES[W.dtype],
                           _ptr(out.X), _ptr(out.valid_idx), _ptr(out.valid_count),
                           _ptr(out.err_flag), _stream(dev))
    return out


def embed_backward(dX: torch.Tensor, input_ids: torch.Tensor, emb: EmbedOut, dW: torch.Tensor,
                   accumulate_dW: bool = True,
                   workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """lce_embed_backward: dW (+)= scatter-sum of dX rows by input id."""
    if dX.dtype != torch.float32 or dW.dtype != torch.float32:
        raise ValueError("dX and dW must be float32")
    if not (dX.is_contiguous() and dW.is_contiguous()):
        raise ValueError("dX and dW must be contiguous")
    N, d = dX.shape
    V = dW.shape[0]
    if dW.shape[1] != d or input_ids.shape[0] != N:
        raise ValueError("shape mismatch")
    dev = dX.device
    if workspace is None:
        n = _lib.lce_embed_workspace_bytes(N, d, V)
        if n == 0:
            raise ValueError(f"unsupported sizes N={N} d={d} V={V}")
        workspace = torch.empty(n, dtype=torch.uint8, device=dev)
    _lib.lce_embed_backward(_ptr(dX), _ptr(input_ids), _ptr(emb.valid_idx), _ptr(emb.valid_count),
                            N, d, V, _ptr(dW), 1 if accumulate_dW else 0, _ptr(workspace),
                            workspace.numel(), _stream(dev))
    return dW


def cast_bf16(x: torch.Tensor, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """lce_cast_bf16: a float32 GPU tensor rounded to bfloat16 (nearest, ties to even)."""
    if x.dtype != torch.float32 or not x.is_cuda or not x.is_contiguous():
        raise ValueError("x must be a contiguous float32 GPU tensor")
    if out is None:
        out = torch.empty(x.shape, dtype=torch.bfloat16, device=x.device)
    if out.dtype != torch.bfloat16 or out.shape != x.shape or not out.is_contiguous():
        raise ValueError("out must be a contiguous bfloat16 tensor of x's shape")
    _lib.lce_cast_bf16(_ptr(x), _ptr(out), x.numel(), _stream(x.device))
    return out


def _as_param_dtype(g: torch.Tensor, dtype: torch.dtype) -> torch.Tensor:
    return cast_bf16(g) if dtype == torch.bfloat16 else g


class _LinearCrossEntropy(torch.autograd.Function):
    @staticmethod
    def forward(ctx, H, W, labels, ignore_index, reduction, check):
        fwd = forward(H, W, labels, ignore_index, check=check)
        ctx.save_for_backward(H, W, labels, fwd.lse, fwd.valid_idx, fwd.valid_count)
        ctx.ignore_index = ignore_index
        ctx.reduction = reduction
        ctx.mark_non_differentiable(fwd.loss, fwd.lse, fwd.valid_count)
        out = fwd.loss_mean if reduction == "mean" else fwd.loss_sum.to(torch.float32)
        return out.reshape(()), fwd.loss, fwd.lse, fwd.valid_count

    @staticmethod
    def backward(ctx, g, *unused):
        H, W, labels, lse, valid_idx, valid_count = ctx.saved_tensors
        fwd = ForwardOut(None, lse, valid_idx, valid_count, None, None, None)
        dH, dW = backward(H, W, labels, fwd, grad_out=g, reduction=ctx.reduction,
                          ignore_index=ctx.ignore_index)
        # bf16 parameters take the fp32 gradients through the library's cast kernel
        gH = _as_param_dtype(dH, H.dtype) if ctx.needs_input_grad[0] else None
        gW = _as_param_dtype(dW, W.dtype) if ctx.needs_input_grad[1] else None
        return gH, gW, None, None, None, None


def linear_cross_entropy(H: torch.Tensor, W: torch.Tensor, labels: torch.Tensor,
                         ignore_index: int = -100, reduction: str = "mean",
                         return_aux: bool = False, check: bool = True):
    """Cross-entropy of the projection H @ W^T against labels, streamed.

    Returns the reduced loss (a 0-d float32 tensor; NaN for "mean" when every
    label is ignored).  With return_aux=True also (per-token loss, lse,
    valid_count).  Gradients flow to H and W (fp32, rounded to bf16 by the
    library's cast kernel for bf16 parameters).
    """
    if reduction not in _RED:
        raise ValueError("reduction must be 'mean' or 'sum'")
    loss, per_tok, lse, cnt = _LinearCrossEntropy.apply(H, W, labels, ignore_index, reduction,
                                                        check)
    if return_aux:
        return loss, (per_tok, lse, cnt)
    return loss


@dataclasses.dataclass
class AttentionOut:
    O: torch.Tensor    # f32 [B, H, S, D]
    lse: torch.Tensor  # f32 [B, H, S], natural log


def attention_forward(Q: torch.Tensor, K: torch.Tensor, V: torch.Tensor, causal: bool = True,
                      scale: Optional[float] = None, out: Optional[AttentionOut] = None
                      ) -> AttentionOut:
    """lce_attention_forward: online-softmax attention over bf16 [B, H, S, D] tensors."""
    for t in (Q, K, V):
        if t.dtype != torch.bfloat16 or not t.is_cuda or not t.is_contiguous() or t.dim() != 4:
            raise ValueError("Q, K and V must be contiguous bf16 [B, H, S, D] GPU tensors")
    if Q.shape != K.shape or Q.shape != V.shape:
        raise ValueError("Q, K and V must have the same shape")
    B, H, S, D = Q.shape
    dev = Q.device
    if out is None:
        out = AttentionOut(O=torch.empty(B, H, S, D, dtype=torch.float32, device=dev),
                           lse=torch.empty(B, H, S, dtype=torch.float32, device=dev))
    _lib.lce_attention_forward(_ptr(Q), _ptr(K), _ptr(V), B, H, S, D, 1 if causal else 0,
                               0.0 if scale is None else float(scale), _ptr(out.O), _ptr(out.lse),
                               _stream(dev))
    return out


@dataclasses.dataclass
class AttentionGrads:
    dQ: torch.Tensor  # f32 [B, H, S, D]
    dK: torch.Tensor
    dV: torch.Tensor


def attention_backward(Q: torch.Tensor, K: torch.Tensor, V: torch.Tensor, fwd: AttentionOut,
                       dO: torch.Tensor, causal: bool = True, scale: Optional[float] = None,
                       out: Optional[AttentionGrads] = None,
                       delta: Optional[torch.Tensor] = None) -> AttentionGrads:
    """lce_attention_backward: dQ, dK, dV for an upstream bf16 dO."""
    for t in (Q, K, V, dO):
        if t.dtype != torch.bfloat16 or not t.is_cuda or not t.is_contiguous() or t.dim() != 4:
            raise ValueError("Q, K, V and dO must be contiguous bf16 [B, H, S, D] GPU tensors")
    if Q.shape != K.shape or Q.shape != V.shape or Q.shape != dO.shape:
        raise ValueError("Q, K, V and dO must have the same shape")
    B, H, S, D = Q.shape
    dev = Q.device
    if out is None:
        f32 = dict(dtype=torch.float32, device=dev)
        out = AttentionGrads(dQ=torch.empty(B, H, S, D, **f32), dK=torch.empty(B, H, S, D, **f32),
                             dV=torch.empty(B, H, S, D, **f32))
    if delta is None:
        delta = torch.empty(B, H, S, dtype=torch.float32, device=dev)
    _lib.lce_attention_backward(_ptr(Q), _ptr(K), _ptr(V), _ptr(fwd.O), _ptr(fwd.lse), _ptr(dO),
                                B, H, S, D, 1 if causal else 0,
                                0.0 if scale is None else float(scale), _ptr(out.dQ),
                                _ptr(out.dK), _ptr(out.dV), _ptr(delta), _stream(dev))
    return out
