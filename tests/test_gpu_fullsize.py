"""Full-size configurations on the GPU, in the launch configuration the
benchmark times (default workspace, one lce_forward + lce_backward).

The fp64 oracle cannot redo a 62K x 128K x 4K forward in a test, so:
  * valid_count / valid_idx: bit-exact against the oracle's compaction;
  * mean loss: within 2e-3 of the stored oracle value (tests/golden, written
    by make_golden.py from the oracle only);
  * per-row loss and lse of every valid row (1e-4 absolute) against the
    stored oracle values;
  * dH rows (1e-2 relative L2) on sampled rows, recomputed live by the
    oracle row by row;
  * dW rows (1e-2 relative L2) on stored sampled vocabulary rows;
  * properties at any size: dH rows of ignored tokens are exactly 0, the
    columns of dW sum to ~0 (rows of softmax - onehot sum to 0), and
    <dW, W> = <dH, H> (both equal sum G * logits for the same rounded G).
"""
import os

import numpy as np
import pytest

import oracle
import workloads
from tests.gpu_helpers import announce, rel_l2, to_dev

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


@pytest.mark.parametrize("cid", [2, 3, 4, 5])
def test_full_size_config(cid):
    import torch
    from vocab_cross_entropy_valid_amd import torch_api
    wl = workloads.CONFIGS[cid]
    path = os.path.join(GOLDEN, f"full_config{cid}.npz")
    g = np.load(path, allow_pickle=False)
    announce(f"full size config {cid} {wl.name}: generating inputs")
    H, W, y = workloads.generate(cid)
    assert workloads.checksum(H, W, y) == str(g["checksum"]), "input generator drifted"
    idx, n_valid, _ = oracle.compact_valid(y, -100, wl.V)
    assert n_valid == int(g["n_valid"])

    announce(f"full size config {cid}: GPU forward + backward")
    Ht, Wt, yt = to_dev(H, W, y, wl.dtype)
    fwd = torch_api.forward(Ht, Wt, yt)
    dH, dW = torch_api.backward(Ht, Wt, yt, fwd)
    torch.cuda.synchronize()

    assert int(fwd.valid_count.item()) == n_valid
    np.testing.assert_array_equal(fwd.valid_idx[:n_valid].cpu().numpy(), idx)
    mean_ref = float(g["loss_sum"]) / n_valid
    assert abs(float(fwd.loss_mean.item()) - mean_ref) <= 2e-3
    assert abs(float(fwd.loss_sum.item()) - float(g["loss_sum"])) <= 1e-5 * float(g["loss_sum"])

    # every valid row's loss and lse against the stored oracle values
    loss = fwd.loss.cpu().numpy()
    lse = fwd.lse.cpu().numpy()
    np.testing.assert_allclose(loss[idx], g["loss_valid"], rtol=0, atol=1e-4)
    np.testing.assert_allclose(lse[idx], g["lse_valid"], rtol=0, atol=1e-4)
    # sampled rows, recomputed live by the oracle (also checks the stored values)
    rng = np.random.default_rng(100 + cid)
    rows = np.unique(np.concatenate([idx[:2], idx[-2:], rng.choice(idx, 12, replace=False)]))
    lse_ref, loss_ref, _ = oracle.rows_forward(H, W, y, rows)
    np.testing.assert_allclose(loss[rows], loss_ref, rtol=0, atol=1e-4)
    np.testing.assert_allclose(lse[rows], lse_ref, rtol=0, atol=1e-4)
    dH_ref = oracle.rows_dH(H, W, y, rows, 1.0 / n_valid)
    rows_t = torch.from_numpy(rows).to(dH.device)
    assert rel_l2(dH[rows_t].cpu().numpy(), dH_ref) <= 1e-2

    vid = g["vocab_ids"]
    dW_rows = dW[torch.from_numpy(vid).to(dW.device)].cpu().numpy()
    assert rel_l2(dW_rows, g["dW_rows"]) <= 1e-2

    # properties over the whole outputs
    ign = np.ones(wl.N, dtype=bool)
    ign[idx] = False
    if ign.any():
        assert float(dH[torch.from_numpy(np.flatnonzero(ign)).to(dH.device)].abs().max()) == 0.0
    colsum = dW.double().sum(0)
    assert float(colsum.norm() / dW.double().norm()) <= 1e-2
    a = float((dW.double() * Wt.double()).sum())
    b = float((dH.double() * Ht.double()).sum())
    assert abs(a - b) <= 1e-3 * max(abs(a), abs(b)), (a, b)
    announce(f"full size config {cid}: ok (mean loss {float(fwd.loss_mean.item()):.6f}, "
             f"oracle {mean_ref:.6f})")
