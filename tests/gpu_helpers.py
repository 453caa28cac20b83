"""Shared helpers of the GPU parity tests (calls go through the C ABI)."""
from __future__ import annotations

import sys

import numpy as np

TORCH_DTYPES = {"bf16": "bfloat16", "f32": "float32"}


def announce(msg: str) -> None:
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def to_dev(H, W, y, dtype):
    import torch
    dt = getattr(torch, TORCH_DTYPES[dtype])
    dev = torch.device("cuda:0")
    return (torch.from_numpy(np.ascontiguousarray(H)).to(dev, dt),
            torch.from_numpy(np.ascontiguousarray(W)).to(dev, dt),
            torch.from_numpy(np.ascontiguousarray(y)).to(dev))


def run_path(H, W, y, dtype, ignore_index=-100, reduction="mean", grad=1.0, check=True,
             backward=True):
    """Forward (+ backward) through torch_api -> C ABI; returns numpy results."""
    import torch
    from vocab_cross_entropy_valid_amd import torch_api
    Ht, Wt, yt = to_dev(H, W, y, dtype)
    fwd = torch_api.forward(Ht, Wt, yt, ignore_index, check=check)
    out = dict(
        loss=fwd.loss.cpu().numpy(), lse=fwd.lse.cpu().numpy(),
        valid_count=int(fwd.valid_count.item()),
        valid_idx=fwd.valid_idx.cpu().numpy(),
        loss_sum=float(fwd.loss_sum.item()), loss_mean=float(fwd.loss_mean.item()),
        err_flag=int(fwd.err_flag.item()))
    if backward:
        g = torch.full((1,), grad, dtype=torch.float32, device=Ht.device)
        dH, dW = torch_api.backward(Ht, Wt, yt, fwd, grad_out=g, reduction=reduction,
                                    ignore_index=ignore_index)
        torch.cuda.synchronize()
        out["dH"] = dH.cpu().numpy()
        out["dW"] = dW.cpu().numpy()
    return out


def rel_l2(got, exp):
    got = np.asarray(got, dtype=np.float64)
    exp = np.asarray(exp, dtype=np.float64)
    den = np.linalg.norm(exp)
    return float(np.linalg.norm(got - exp) / (den if den > 0 else 1.0))
