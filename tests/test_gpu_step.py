"""Backward with the optimizer fused into the dW epilogue (no dW table)."""
import numpy as np
import pytest

import oracle
import workloads
from tests.gpu_helpers import announce, rel_l2, to_dev

pytestmark = pytest.mark.gpu

IGN = -100


@pytest.mark.parametrize("kind,dtype,N,d,V,seed", [
    ("sgd", "bf16", 700, 128, 5000, 71),
    ("adamw", "bf16", 700, 128, 5000, 72),
    ("adamw", "f32", 333, 64, 1500, 73),
    ("sgd", "f32", 300, 64, 20000, 74),          # several vocabulary blocks
])
def test_fused_update(kind, dtype, N, d, V, seed):
    import torch
    from vocab_cross_entropy_valid_amd import torch_api
    announce(f"fused {kind} {dtype} N={N} d={d} V={V}")
    H, W, y = workloads.custom(N, d, V, dtype=dtype, seed=seed, ignore_frac=0.2)
    Ht, Wt, yt = to_dev(H, W, y, dtype)
    rng = np.random.default_rng(seed + 1)
    hp = dict(lr=2e-2, weight_decay=0.05, betas=(0.8, 0.95), eps=1e-7, step=3)
    fwd = torch_api.forward(Ht, Wt, yt, IGN)
    # reference gradient: the unfused path (same kernels, same G)
    g2 = torch.full((1,), 1.7, device=Ht.device)
    dH0, dW0 = torch_api.backward(Ht, Wt, yt, fwd, grad_out=g2)
    p0 = Wt.float().cpu().numpy().astype(np.float64)
    g = dW0.cpu().numpy().astype(np.float64)
    m0 = rng.standard_normal((V, d)) * 1e-4 if kind == "adamw" else None
    v0 = rng.random((V, d)) * 1e-8 if kind == "adamw" else None
    master = Wt.float().clone() if dtype == "bf16" else None
    ea = torch.from_numpy(m0.astype(np.float32)).to(Ht.device) if kind == "adamw" else None
    eas = torch.from_numpy(v0.astype(np.float32)).to(Ht.device) if kind == "adamw" else None
    Wupd = Wt.clone()
    dH = torch_api.backward_step(Ht, Wupd, yt, fwd, kind, hp["lr"], hp["weight_decay"],
                                 hp["betas"], hp["eps"], hp["step"], W_master=master,
                                 exp_avg=ea, exp_avg_sq=eas, grad_out=g2)
    torch.cuda.synchronize()
    # dH is the unfused dH, bit for bit
    assert torch.equal(dH, dH0)
    # the update arithmetic against fp64 on the same gradient
    p_ref, m_ref, v_ref = oracle.optimizer_step(
        p0, g, kind, hp["lr"], hp["weight_decay"], hp["betas"][0], hp["betas"][1], hp["eps"],
        hp["step"], m0.astype(np.float32).astype(np.float64) if m0 is not None else None,
        v0.astype(np.float32).astype(np.float64) if v0 is not None else None)
    p_gpu = (master if master is not None else Wupd).cpu().numpy()
    np.testing.assert_allclose(p_gpu, p_ref, rtol=1e-5, atol=1e-6)
    if kind == "adamw":
        np.testing.assert_allclose(ea.cpu().numpy(), m_ref, rtol=1e-5, atol=1e-10)
        np.testing.assert_allclose(eas.cpu().numpy(), v_ref, rtol=1e-5, atol=1e-14)
    if dtype == "bf16":
        # the operand copy is the master rounded to nearest even
        assert torch.equal(Wupd, master.to(torch.bfloat16))
    # end to end against the oracle's gradient and update
    dW_o = oracle.backward(H, W, y, IGN, grad=1.7)[1]
    p_o, _, _ = oracle.optimizer_step(
        p0, dW_o, kind, hp["lr"], hp["weight_decay"], hp["betas"][0], hp["betas"][1], hp["eps"],
        hp["step"], m0, v0)
    assert rel_l2(p_gpu - p0, p_o - p0) <= (1e-2 if dtype == "bf16" else 1e-4)


def test_fused_update_config3_sampled_rows():
    """The metric's head (d = 4096, V = 128256, 3903 valid tokens): AdamW step,
    sampled vocabulary rows against fp64 on the unfused gradient."""
    import torch
    from vocab_cross_entropy_valid_amd import torch_api
    announce("fused adamw config 3")
    H, W, y = workloads.generate(3)
    Ht, Wt, yt = to_dev(H, W, y, "bf16")
    fwd = torch_api.forward(Ht, Wt, yt, IGN)
    ws = torch_api.alloc_workspace(8192, 4096, 128256, torch.bfloat16, Ht.device)
    _, dW0 = torch_api.backward(Ht, Wt, yt, fwd, workspace=ws)
    rows = torch.tensor([0, 1, 2, 100, 64000, 128255, 70001], device=Ht.device)
    g = dW0[rows].cpu().numpy().astype(np.float64)
    del dW0
    master = Wt.float()
    ea = torch.zeros_like(master)
    eas = torch.zeros_like(master)
    p0 = master[rows].cpu().numpy().astype(np.float64)
    torch_api.backward_step(Ht, Wt, yt, fwd, "adamw", 1e-3, 0.01, step=1, W_master=master,
                            exp_avg=ea, exp_avg_sq=eas, workspace=ws)
    torch.cuda.synchronize()
    p_ref, m_ref, v_ref = oracle.optimizer_step(p0, g, "adamw", 1e-3, 0.01, step=1,
                                                exp_avg=np.zeros_like(g), exp_avg_sq=np.zeros_like(g))
    np.testing.assert_allclose(master[rows].cpu().numpy(), p_ref, rtol=1e-5, atol=1e-6)
    np.testing.assert_allclose(ea[rows].cpu().numpy(), m_ref, rtol=1e-5, atol=1e-12)
    assert torch.equal(Wt[rows], master[rows].to(torch.bfloat16))
