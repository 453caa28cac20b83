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
    # more valid rows (8400) than one token chunk (8192): the first chunk's
    # dW goes to the block accumulator, the second adds it and applies
    ("sgd", "bf16", 10500, 128, 3000, 75),
    ("adamw", "bf16", 10500, 64, 20000, 76),     # ... with two vocabulary blocks
    ("adamw", "f32", 10500, 64, 1500, 77),
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


@pytest.mark.parametrize("n_valid", [8192, 16384, 16385])
def test_fused_update_chunk_boundaries(n_valid):
    """Valid rows ending exactly at a token-chunk boundary (the chunk after
    them holds none and must do nothing), and one row past it (a third chunk
    with a single row applies the update).  16800 positions = three chunks."""
    import torch
    from vocab_cross_entropy_valid_amd import torch_api
    announce(f"fused sgd chunk boundaries: {n_valid} valid of 16800")
    N, d, V = 16800, 64, 900
    H, W, y = workloads.custom(N, d, V, dtype="bf16", seed=n_valid, ignore_frac=0.0)
    drop = np.random.default_rng(n_valid).choice(N, N - n_valid, replace=False)
    y[drop] = IGN
    Ht, Wt, yt = to_dev(H, W, y, "bf16")
    fwd = torch_api.forward(Ht, Wt, yt, IGN)
    assert int(fwd.valid_count.item()) == n_valid
    dH0, dW0 = torch_api.backward(Ht, Wt, yt, fwd)
    master = Wt.float().clone()
    Wupd = Wt.clone()
    dH = torch_api.backward_step(Ht, Wupd, yt, fwd, "sgd", 0.5, 0.1, W_master=master)
    torch.cuda.synchronize()
    assert torch.equal(dH, dH0)
    p0 = Wt.float().cpu().numpy().astype(np.float64)
    p_ref, _, _ = oracle.optimizer_step(p0, dW0.cpu().numpy(), "sgd", 0.5, 0.1)
    np.testing.assert_allclose(master.cpu().numpy(), p_ref, rtol=1e-5, atol=1e-6)
    dW_o = oracle.backward(H, W, y, IGN)[1]
    p_o, _, _ = oracle.optimizer_step(p0, dW_o, "sgd", 0.5, 0.1)
    assert rel_l2(master.cpu().numpy() - p0, p_o - p0) <= 1e-2


@pytest.mark.parametrize("kind", ["sgd", "adamw"])
def test_fused_update_config3_sampled_rows(kind):
    """The metric's head (d = 4096, V = 128256, 3903 valid tokens): sampled
    vocabulary rows of the updated weights against the oracle's gradient
    (oracle.rows_dW with the stored fp64 lse of every valid row) and the
    oracle's update (oracle.optimizer_step).  AdamW starts from a second
    moment well above g^2, so that its update is linear in g and the bf16
    gradient tolerance carries over to the weight change (from zero moments
    the first step is lr * sign(g), which flips on entries whose exact value
    lies within rounding of 0)."""
    import os
    import torch
    from vocab_cross_entropy_valid_amd import torch_api
    announce(f"fused {kind} config 3, sampled rows vs the oracle")
    g_path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                          "full_config3.npz")
    gold = np.load(g_path, allow_pickle=False)
    H, W, y = workloads.generate(3)
    assert workloads.checksum(H, W, y) == str(gold["checksum"]), "input generator drifted"
    idx, n_valid, _ = oracle.compact_valid(y, IGN, W.shape[0])
    rows = np.array([0, 1, 2, 100, 64000, 70001, 128255])
    g_ref = oracle.rows_dW(H, W, y, idx, gold["lse_valid"], rows, 1.0 / n_valid)
    Ht, Wt, yt = to_dev(H, W, y, "bf16")
    fwd = torch_api.forward(Ht, Wt, yt, IGN)
    master = Wt.float()
    rt = torch.from_numpy(rows).to(Ht.device)
    p0 = master[rt].cpu().numpy().astype(np.float64)
    hp = dict(lr=1e-3, weight_decay=0.01, betas=(0.9, 0.999), eps=1e-8, step=1)
    ea = eas = None
    m0 = v0 = None
    if kind == "adamw":
        ea = torch.zeros_like(master)
        eas = torch.full_like(master, 1e-4)
        m0 = np.zeros_like(p0)
        v0 = np.full_like(p0, np.float64(np.float32(1e-4)))
    torch_api.backward_step(Ht, Wt, yt, fwd, kind, hp["lr"], hp["weight_decay"], hp["betas"],
                            hp["eps"], hp["step"], W_master=master, exp_avg=ea, exp_avg_sq=eas)
    torch.cuda.synchronize()
    p_ref, m_ref, _ = oracle.optimizer_step(p0, g_ref, kind, hp["lr"], hp["weight_decay"],
                                            hp["betas"][0], hp["betas"][1], hp["eps"],
                                            hp["step"], m0, v0)
    p_gpu = master[rt].cpu().numpy().astype(np.float64)
    assert rel_l2(p_gpu - p0, p_ref - p0) <= 1e-2, rel_l2(p_gpu - p0, p_ref - p0)
    if kind == "adamw":
        assert rel_l2(ea[rt].cpu().numpy(), m_ref) <= 1e-2
    # the bf16 operand is the updated master rounded to nearest even
    assert torch.equal(Wt[rt], master[rt].to(torch.bfloat16))


def test_fused_update_config4_sampled_rows():
    """The 260K vocabulary (16384 positions, 6800 valid, d = 4096): the case
    whose fp32 dW table (4.26 GB) the fused update never stores.  AdamW, the
    second moment started above g^2 as in the config 3 case; sampled rows
    against oracle.rows_dW (stored fp64 lse) and oracle.optimizer_step."""
    import os
    import torch
    from vocab_cross_entropy_valid_amd import torch_api
    announce("fused adamw config 4, sampled rows vs the oracle")
    gold = np.load(os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                                "full_config4.npz"), allow_pickle=False)
    H, W, y = workloads.generate(4)
    assert workloads.checksum(H, W, y) == str(gold["checksum"]), "input generator drifted"
    idx, n_valid, _ = oracle.compact_valid(y, IGN, W.shape[0])
    rows = np.array([0, 1, 5, 1000, 16383, 16384, 130000, 259999])
    g_ref = oracle.rows_dW(H, W, y, idx, gold["lse_valid"], rows, 1.0 / n_valid)
    Ht, Wt, yt = to_dev(H, W, y, "bf16")
    del H
    fwd = torch_api.forward(Ht, Wt, yt, IGN)
    master = Wt.float()
    ea = torch.zeros_like(master)
    eas = torch.full_like(master, 1e-4)
    rt = torch.from_numpy(rows).to(Ht.device)
    p0 = master[rt].cpu().numpy().astype(np.float64)
    v0 = np.full_like(p0, np.float64(np.float32(1e-4)))
    torch_api.backward_step(Ht, Wt, yt, fwd, "adamw", 1e-3, 0.01, step=1, W_master=master,
                            exp_avg=ea, exp_avg_sq=eas)
    torch.cuda.synchronize()
    p_ref, m_ref, _ = oracle.optimizer_step(p0, g_ref, "adamw", 1e-3, 0.01, step=1,
                                            exp_avg=np.zeros_like(p0), exp_avg_sq=v0)
    p_gpu = master[rt].cpu().numpy().astype(np.float64)
    assert rel_l2(p_gpu - p0, p_ref - p0) <= 1e-2, rel_l2(p_gpu - p0, p_ref - p0)
    assert rel_l2(ea[rt].cpu().numpy(), m_ref) <= 1e-2
    assert torch.equal(Wt[rt], master[rt].to(torch.bfloat16))
