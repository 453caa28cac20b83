"""The fp32 -> bf16 output cast (lce_cast_bf16) and the autograd path that
uses it, against the oracle's round-to-nearest-even (oracle.round_to_bf16,
pinned to PyTorch's CPU conversion and to closed forms).  Bit-exact."""
import numpy as np
import pytest

import oracle
import workloads
from tests.gpu_helpers import announce, rel_l2
from tests.oracle_pins import _bf16_sweep

pytestmark = pytest.mark.gpu


def _bits(a):
    return np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)


@pytest.mark.parametrize("n", [1, 7, 8, 9, 4099, 1000003])
def test_cast_matches_round_to_nearest_even(n):
    import torch
    from vocab_cross_entropy_valid_amd import torch_api
    announce(f"cast_bf16 n={n}")
    sweep = _bf16_sweep()
    x = np.resize(sweep, n).astype(np.float32)
    if n > 8:
        x[3] = np.nan
    xt = torch.from_numpy(x).cuda()
    y = torch_api.cast_bf16(xt)
    torch.cuda.synchronize()
    got = y.float().cpu().numpy()
    ref = oracle.round_to_bf16(x)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(_bits(got[~nan]), _bits(ref[~nan]))


def test_cast_rejects_misaligned_and_overlapping():
    import torch
    from vocab_cross_entropy_valid_amd import _lib
    x = torch.zeros(64, device="cuda:0")
    out = torch.empty(64, dtype=torch.bfloat16, device="cuda:0")
    lib = _lib.load()
    assert lib.lce_cast_bf16(x.data_ptr() + 4, out.data_ptr(), 8, None) == _lib.LCE_ERR_INVALID_ARG
    assert lib.lce_cast_bf16(x.data_ptr(), x.data_ptr() + 16, 8, None) == _lib.LCE_ERR_INVALID_ARG
    assert lib.lce_cast_bf16(x.data_ptr(), out.data_ptr(), -1, None) == _lib.LCE_ERR_INVALID_ARG
    assert lib.lce_cast_bf16(None, None, 0, None) == _lib.LCE_OK


def test_autograd_gradients_are_the_rounded_fp32_outputs():
    """linear_cross_entropy's bf16 gradients are bit-identical to round to
    nearest even of lce_backward's fp32 dH and dW, which themselves match
    the oracle's gradients to the bf16 tolerance; two cast launches per
    backward, both in the library."""
    import torch
    from vocab_cross_entropy_valid_amd import _lib, torch_api
    announce("autograd bf16 gradients through the cast kernel")
    H, W, y = workloads.custom(700, 192, 3000, dtype="bf16", seed=91, ignore_frac=0.15)
    dev = torch.device("cuda:0")
    Ht = torch.from_numpy(H).to(dev, torch.bfloat16).requires_grad_(True)
    Wt = torch.from_numpy(W).to(dev, torch.bfloat16).requires_grad_(True)
    yt = torch.from_numpy(y).to(dev)
    loss = torch_api.linear_cross_entropy(Ht, Wt, yt)
    _lib.lce_timing_reset()
    _lib.lce_timing_enable(True)
    try:
        loss.backward()
        torch.cuda.synchronize()
    finally:
        _lib.lce_timing_enable(False)
    casts = _lib.lce_timing_query(_lib.KERNEL_CLASSES.index("cast"))[1]
    _lib.lce_timing_reset()
    assert casts == 2
    fwd = torch_api.forward(Ht.detach(), Wt.detach(), yt)
    dH, dW = torch_api.backward(Ht.detach(), Wt.detach(), yt, fwd)
    torch.cuda.synchronize()
    for g, f32 in ((Ht.grad, dH), (Wt.grad, dW)):
        assert g.dtype == torch.bfloat16
        got = g.float().cpu().numpy()
        ref = oracle.round_to_bf16(f32.cpu().numpy())
        assert np.array_equal(_bits(got), _bits(ref))
    rdH, rdW = oracle.backward(H, W, y, -100)
    assert rel_l2(Ht.grad.float().cpu().numpy(), rdH) <= 1e-2
    assert rel_l2(Wt.grad.float().cpu().numpy(), rdW) <= 1e-2
