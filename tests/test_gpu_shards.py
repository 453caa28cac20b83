"""Vocabulary-sharded mode on the GPU against the oracle and the unsharded
path: per-shard partials (max, scaled sum, target logit), their merge, and
the per-shard backward (dH shares summed, dW rows stacked)."""
import numpy as np
import pytest

import oracle
import workloads
from tests.gpu_helpers import announce, rel_l2, to_dev

pytestmark = pytest.mark.gpu

IGN = -100


def _bounds(V, cuts):
    edges = [0] + list(cuts) + [V]
    return list(zip(edges[:-1], edges[1:]))


def _run_shards(Ht, Wt, yt, V, shards, grad=1.0, reduction="mean", backward=True):
    import torch
    from vocab_cross_entropy_valid_amd import torch_api
    N = Ht.shape[0]
    dev = Ht.device
    pm = torch.empty(len(shards), N, dtype=torch.float32, device=dev)
    ps = torch.empty_like(pm)
    pt = torch.empty_like(pm)
    parts = []
    for k, (a, b) in enumerate(shards):
        out = torch_api.ShardPartials(pm[k], ps[k], pt[k],
                                      torch.empty(N, dtype=torch.int32, device=dev),
                                      torch.empty(1, dtype=torch.int32, device=dev),
                                      torch.empty(1, dtype=torch.int32, device=dev))
        parts.append(torch_api.forward_shard(Ht, Wt[a:b].contiguous(), yt, V, a, IGN, out=out))
    merged = torch_api.lse_merge(pm, ps, pt, parts[0].valid_idx, parts[0].valid_count)
    res = dict(parts=parts, merged=merged, pm=pm, ps=ps, pt=pt)
    if backward:
        g = torch.full((1,), grad, dtype=torch.float32, device=dev)
        dH = torch.empty(N, Ht.shape[1], dtype=torch.float32, device=dev)
        dWs = []
        for k, (a, b) in enumerate(shards):
            dWs.append(torch_api.backward_shard(Ht, Wt[a:b].contiguous(), yt, V, a, merged, dH,
                                                accumulate_dH=k > 0, grad_out=g,
                                                reduction=reduction, ignore_index=IGN))
        res["dH"] = dH
        res["dW"] = torch.cat(dWs)
    torch.cuda.synchronize()
    return res


@pytest.mark.parametrize("N,d,V,dtype,cuts,seed", [
    (700, 128, 5000, "bf16", (1234, 1300), 51),      # ragged shards, one of 66 entries
    (300, 64, 20000, "bf16", (7, 16391), 52),         # a 7-entry shard, one past a block
    (333, 64, 1500, "f32", (512,), 53),               # fp32
])
def test_shard_partials_merge_and_backward(N, d, V, dtype, cuts, seed):
    import torch
    from vocab_cross_entropy_valid_amd import torch_api
    announce(f"shards N={N} d={d} V={V} {dtype} cuts={cuts}")
    H, W, y = workloads.custom(N, d, V, dtype=dtype, seed=seed, ignore_frac=0.2)
    shards = _bounds(V, cuts)
    Ht, Wt, yt = to_dev(H, W, y, dtype)
    r = _run_shards(Ht, Wt, yt, V, shards, grad=1.3)

    # per-shard partials against the oracle's definitions
    f = oracle.forward(H, W, y, IGN)
    v = f.valid_idx
    ign = np.setdiff1d(np.arange(N), v)
    for k, (a, b) in enumerate(shards):
        po = oracle.shard_partials(H, W[a:b], y, a, V, IGN)
        pm = r["pm"][k].cpu().numpy()
        ps = r["ps"][k].cpu().numpy()
        pt = r["pt"][k].cpu().numpy()
        np.testing.assert_allclose(pm[v], po.part_max[v], rtol=0, atol=1e-4)
        np.testing.assert_allclose(ps[v], po.part_sum[v], rtol=1e-4)
        fin = np.isfinite(po.part_target[v])
        assert np.array_equal(np.isfinite(pt[v]), fin)
        np.testing.assert_allclose(pt[v][fin], po.part_target[v][fin], rtol=0, atol=1e-4)
        assert np.all(ps[ign] == 0.0) and np.all(pm[ign] == 0.0)
        assert int(r["parts"][k].valid_count.item()) == f.valid_count
        assert int(r["parts"][k].err_flag.item()) == 0

    # merged forward: oracle and the unsharded GPU path
    m = r["merged"]
    loss = m.loss.cpu().numpy()
    lse = m.lse.cpu().numpy()
    np.testing.assert_allclose(loss, f.loss, rtol=1e-5, atol=1e-5)
    np.testing.assert_allclose(lse, f.lse, rtol=1e-5, atol=1e-5)
    assert np.all(loss[ign] == 0.0) and np.all(lse[ign] == 0.0)
    assert abs(float(m.loss_sum.item()) - f.loss_sum) <= 1e-5 * abs(f.loss_sum)
    assert abs(float(m.loss_mean.item()) - f.loss_mean) <= 1e-5 * abs(f.loss_mean)
    full = torch_api.forward(Ht, Wt, yt, IGN)
    np.testing.assert_allclose(loss, full.loss.cpu().numpy(), rtol=0, atol=2e-5)

    # backward: dH shares summed over shards, dW rows stacked
    dH_ref, dW_ref = oracle.backward(H, W, y, IGN, grad=1.3)
    tol = 1e-2 if dtype == "bf16" else 1e-4
    assert rel_l2(r["dH"].cpu().numpy(), dH_ref) <= tol
    assert rel_l2(r["dW"].cpu().numpy(), dW_ref) <= tol
    assert float(r["dH"][torch.from_numpy(ign).to(Ht.device)].abs().max()) == 0.0
    dH_full, dW_full = torch_api.backward(Ht, Wt, yt, full, grad_out=torch.full(
        (1,), 1.3, device=Ht.device))
    assert rel_l2(r["dH"].cpu().numpy(), dH_full.cpu().numpy()) <= 1e-5
    assert rel_l2(r["dW"].cpu().numpy(), dW_full.cpu().numpy()) <= 1e-5


def test_single_shard_equals_unsharded():
    """One shard holding the whole vocabulary reproduces lce_forward."""
    from vocab_cross_entropy_valid_amd import torch_api
    announce("single shard")
    H, W, y = workloads.custom(500, 128, 3000, seed=54, ignore_frac=0.1)
    Ht, Wt, yt = to_dev(H, W, y, "bf16")
    r = _run_shards(Ht, Wt, yt, 3000, [(0, 3000)], backward=False)
    full = torch_api.forward(Ht, Wt, yt, IGN)
    np.testing.assert_allclose(r["merged"].loss.cpu().numpy(), full.loss.cpu().numpy(),
                               rtol=0, atol=2e-5)
    pm, ps = r["pm"][0].cpu().numpy(), r["ps"][0].cpu().numpy()
    v = full.valid_idx[:int(full.valid_count.item())].cpu().numpy()
    np.testing.assert_allclose(pm[v] + np.log(ps[v]), full.lse.cpu().numpy()[v], rtol=0,
                               atol=2e-5)


def test_shard_label_range_is_checked_against_the_whole_vocabulary():
    """A label past V_total sets err_flag in every shard; labels of other
    shards are not errors."""
    from vocab_cross_entropy_valid_amd import torch_api
    announce("shard label range")
    H, W, y = workloads.custom(200, 64, 900, seed=55, ignore_frac=0.0)
    y[7] = 900
    Ht, Wt, yt = to_dev(H, W, y, "bf16")
    p = torch_api.forward_shard(Ht, Wt[:300].contiguous(), yt, 900, 0, IGN)
    assert int(p.err_flag.item()) == 1 and int(p.valid_count.item()) == 199
    y[7] = 899
    Ht, Wt, yt = to_dev(H, W, y, "bf16")
    p = torch_api.forward_shard(Ht, Wt[:300].contiguous(), yt, 900, 0, IGN)
    assert int(p.err_flag.item()) == 0 and int(p.valid_count.item()) == 200
