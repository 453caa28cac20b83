"""Input side of a tied table on the GPU: the masked gather (bit-exact) and
the deterministic scatter-sum of dX into dW, against the oracle."""
import numpy as np
import pytest

import oracle
from tests.gpu_helpers import announce, rel_l2

pytestmark = pytest.mark.gpu


def _ids(N, V, pad, pad_frac, seed, zipf_s=1.1, hot=None):
    rng = np.random.default_rng(seed)
    k = np.arange(1, V + 1, dtype=np.float64)
    cdf = np.cumsum(k ** -zipf_s)
    cdf /= cdf[-1]
    ids = np.minimum(np.searchsorted(cdf, rng.random(N), side="right"), V - 1).astype(np.int64)
    if hot is not None:                       # one id repeated across many 64-row chunks
        ids[rng.choice(N, hot[1], replace=False)] = hot[0]
    if pad_frac:
        ids[rng.choice(N, int(pad_frac * N), replace=False)] = pad
    return ids


def _dev(a, dtype=None):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a)).to("cuda:0")
    return t if dtype is None else t.to(dtype)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_embed_forward_is_an_exact_masked_gather(dtype):
    import torch
    from vocab_cross_entropy_valid_amd import torch_api
    announce(f"embed forward {dtype}")
    V, d, N, pad = 5000, 256, 3000, 2
    rng = np.random.default_rng(60)
    W = rng.standard_normal((V, d)).astype(np.float32)
    ids = _ids(N, V, pad, 0.2, 61)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    Wt = _dev(W, tdt)
    out = torch_api.embed_forward(Wt, _dev(ids), pad)
    X = out.X.float().cpu().numpy()
    Wr = Wt.float().cpu().numpy()
    Xo, idx = oracle.embed_forward(Wr, ids, pad)
    assert np.array_equal(X, Xo)                       # a copy: bit-exact
    assert int(out.valid_count.item()) == idx.size
    assert np.array_equal(out.valid_idx[:idx.size].cpu().numpy(), idx)
    assert int(out.err_flag.item()) == 0


@pytest.mark.parametrize("N,d,V,hot,seed", [
    (3000, 256, 5000, (17, 700), 62),      # one id over 11 chunks of 64 rows
    (1000, 128, 300, None, 63),            # small vocabulary: long segments everywhere
    (257, 64, 100000, None, 64),           # mostly single-row segments
])
def test_embed_backward_scatter_sum(N, d, V, hot, seed):
    import torch
    from vocab_cross_entropy_valid_amd import torch_api
    announce(f"embed backward N={N} d={d} V={V} hot={hot}")
    pad = 0
    ids = _ids(N, V, pad, 0.15, seed, hot=hot)
    rng = np.random.default_rng(seed + 100)
    dX = rng.standard_normal((N, d)).astype(np.float32)
    ref = oracle.embed_backward(dX, ids, pad, V)
    Wt = torch.zeros(V, d, dtype=torch.bfloat16, device="cuda:0")
    idt = _dev(ids)
    emb = torch_api.embed_forward(Wt, idt, pad)
    dXt = _dev(dX)
    # overwrite: rows without an occurrence become 0
    dW = torch.full((V, d), 7.0, dtype=torch.float32, device="cuda:0")
    torch_api.embed_backward(dXt, idt, emb, dW, accumulate_dW=False)
    got = dW.cpu().numpy()
    np.testing.assert_allclose(got, ref, rtol=1e-5, atol=1e-5)
    assert rel_l2(got, ref) <= 1e-6
    untouched = np.setdiff1d(np.arange(V), ids[ids != pad])
    assert not got[untouched].any()
    # accumulate: added to what dW holds
    base = rng.standard_normal((V, d)).astype(np.float32)
    dW2 = _dev(base)
    torch_api.embed_backward(dXt, idt, emb, dW2, accumulate_dW=True)
    np.testing.assert_allclose(dW2.cpu().numpy(), base + ref, rtol=1e-5, atol=1e-5)
    # bitwise reproducible
    dW3 = torch.empty_like(dW)
    torch_api.embed_backward(dXt, idt, emb, dW3, accumulate_dW=False)
    assert torch.equal(dW3, dW)


def test_embed_bad_id_sets_flag():
    import torch
    from vocab_cross_entropy_valid_amd import torch_api
    announce("embed bad id")
    ids = _ids(500, 300, 0, 0.1, 65)
    ids[11] = 300
    Wt = torch.randn(300, 64, device="cuda:0").to(torch.bfloat16)
    out = torch_api.embed_forward(Wt, _dev(ids), 0)
    assert int(out.err_flag.item()) == 1
    assert not out.X[11].float().abs().sum().item()          # treated as padding
    assert 11 not in out.valid_idx[:int(out.valid_count.item())].cpu().numpy()


@pytest.mark.slow
def test_embed_full_size_rows():
    """Shapes of the long-context workload (65536 positions, d = 4096,
    V = 128256, Zipf ids, 5% padding): dW on sampled rows (the hottest ids
    and random ones) against the oracle; X exact on sampled rows."""
    import torch
    from vocab_cross_entropy_valid_amd import torch_api
    announce("embed full size")
    N, d, V, pad = 65536, 4096, 128256, 0
    ids = _ids(N, V, pad, 0.05, 66)
    rng = np.random.default_rng(67)
    dX = rng.standard_normal((N, d), dtype=np.float32)
    Wt = torch.randn(V, d, device="cuda:0").to(torch.bfloat16)
    idt = _dev(ids)
    emb = torch_api.embed_forward(Wt, idt, pad)
    rows = np.concatenate([np.arange(8), rng.choice(N, 8, replace=False)])
    Xs = emb.X[_dev(rows)].float().cpu().numpy()
    Wr = Wt[_dev(np.where(ids[rows] == pad, 0, ids[rows]))].float().cpu().numpy()
    Wr[ids[rows] == pad] = 0
    assert np.array_equal(Xs, Wr)
    dW = torch.empty(V, d, dtype=torch.float32, device="cuda:0")
    torch_api.embed_backward(_dev(dX), idt, emb, dW, accumulate_dW=False)
    uniq, cnt = np.unique(ids[ids != pad], return_counts=True)
    sample = np.unique(np.concatenate([uniq[np.argsort(-cnt)[:4]],
                                       rng.choice(uniq, 6, replace=False)]))
    # The oracle's backward on the positions holding a sampled id, with the
    # ids renumbered 0, 1, ... (rows of the table are independent, so these are
    # exactly the sampled rows of the full dW); every other position is padding.
    sel = np.flatnonzero(np.isin(ids, sample))
    local = np.searchsorted(sample, ids[sel])
    ref = oracle.embed_backward(dX[sel], local, -1, sample.size)
    got = dW[_dev(sample)].cpu().numpy()
    np.testing.assert_allclose(got, ref, rtol=1e-4, atol=1e-3)
