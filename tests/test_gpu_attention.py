"""Online-softmax attention on the GPU against the fp64 oracle.

Inputs are bf16-representable (workloads.attention_inputs); the oracle runs
in fp64 on those same values.  Tolerance, from the arithmetic of the kernel:
scores are exact bf16 products summed in fp32 (relative error ~1e-6), the
probabilities are rounded to bf16 before the second product (relative error
<= 2^-9 each, independent across keys), and the normaliser sums the same
rounded values.  The output is then a weighted mean whose weights carry
<= 0.2% relative error, so

  * O:   relative L2 error over each case <= 1e-2 (same bar as the
         bf16 gradients of the loss path), and finite everywhere;
  * lse: absolute error <= 2e-3 (the normaliser's relative error <= 2^-9
         bounds the log's absolute error by ~2e-3).

At full size (batch 8, 32 heads, 2048 positions, head_dim 128, causal) the
oracle recomputes sampled rows through the causal-prefix identity (row q of
causal attention equals unmasked attention over keys 0..q; pinned in
tests/oracle_pins.py), and V = 1 must give O = 1 everywhere (rows of a
softmax sum to one; the normaliser sums exactly the rounded values the MFMA
multiplies, so only fp32 summation order separates the two, ~sqrt(S) * 6e-8).
"""
import numpy as np
import pytest

import oracle
import workloads
from tests.gpu_helpers import announce, rel_l2

pytestmark = pytest.mark.gpu


def _run(Q, K, V, causal, scale=None):
    import torch
    from vocab_cross_entropy_valid_amd import torch_api
    dev = torch.device("cuda:0")
    t = [torch.from_numpy(x).to(dev).to(torch.bfloat16).contiguous() for x in (Q, K, V)]
    r = torch_api.attention_forward(*t, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return r.O.cpu().numpy(), r.lse.cpu().numpy()


CASES = [
    # B, H, S, D, causal, seed
    (1, 2, 200, 64, False, 601),
    (2, 3, 257, 128, True, 602),     # ragged key block and query block
    (1, 1, 1, 128, True, 603),       # a single position
    (1, 2, 64, 64, True, 604),       # exactly one key block
    (1, 1, 300, 128, False, 605),
    (2, 2, 130, 128, True, 606),     # second query block holds 2 queries
    (1, 4, 512, 128, True, 607),     # several query blocks, diagonal skips
    # B * H a multiple of 8: the blocks of a group of heads run interleaved,
    # heaviest first, on one XCD (group of 8 heads per XCD for the forward,
    # shrunk to the largest power of two dividing B * H / 8)
    (2, 4, 300, 128, True, 608),
    (1, 8, 130, 64, False, 609),
    (2, 32, 260, 128, True, 610),    # groups of 8
    (3, 16, 200, 64, True, 611),     # B * H / 8 = 6: groups of 2
]


@pytest.mark.parametrize("B,H,S,D,causal,seed", CASES)
def test_attention_matches_oracle(B, H, S, D, causal, seed):
    announce(f"attention B{B} H{H} S{S} D{D} causal={causal}")
    Q, K, V = workloads.attention_inputs(B, H, S, D, seed)
    O, lse = _run(Q, K, V, causal)
    ref = oracle.attention_forward(Q, K, V, causal=causal)
    assert np.all(np.isfinite(O)) and np.all(np.isfinite(lse))
    assert rel_l2(O, ref.O) <= 1e-2, rel_l2(O, ref.O)
    np.testing.assert_allclose(lse, ref.lse, rtol=0, atol=2e-3)


def test_attention_explicit_scale_and_large_scores():
    """A scale far from 1/sqrt(D) and inputs of std 4 (scores of order 100):
    the running max must keep exp2 in range."""
    announce("attention explicit scale")
    Q, K, V = workloads.attention_inputs(1, 2, 190, 128, 611, std=4.0)
    O, lse = _run(Q, K, V, True, scale=0.3)
    ref = oracle.attention_forward(Q, K, V, causal=True, scale=0.3)
    assert rel_l2(O, ref.O) <= 1e-2
    np.testing.assert_allclose(lse, ref.lse, rtol=1e-4, atol=2e-3)


def test_attention_rows_sum_to_one():
    announce("attention V = 1")
    Q, K, _ = workloads.attention_inputs(1, 2, 333, 128, 612, std=2.0)
    V = np.ones_like(Q)
    O, _ = _run(Q, K, V, True)
    np.testing.assert_allclose(O, 1.0, rtol=0, atol=1e-5)


def test_attention_deterministic_and_empty():
    import torch
    from vocab_cross_entropy_valid_amd import torch_api
    announce("attention determinism, empty")
    Q, K, V = workloads.attention_inputs(1, 2, 400, 128, 613)
    a = _run(Q, K, V, True)
    b = _run(Q, K, V, True)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    dev = torch.device("cuda:0")
    e = torch.empty(2, 3, 0, 128, dtype=torch.bfloat16, device=dev)
    r = torch_api.attention_forward(e, e, e, causal=True)
    torch.cuda.synchronize()
    assert r.O.shape == (2, 3, 0, 128) and r.lse.shape == (2, 3, 0)


@pytest.mark.slow
def test_attention_full_size_sampled_rows():
    """The benchmarked shape; the oracle recomputes sampled rows."""
    import torch
    from vocab_cross_entropy_valid_amd import torch_api
    wl = workloads.ATTENTION
    announce(f"attention full size {wl.name}: inputs")
    Q, K, V = workloads.attention_inputs(wl.B, wl.H, wl.S, wl.D, wl.seed)
    dev = torch.device("cuda:0")
    t = [torch.from_numpy(x).to(dev).to(torch.bfloat16).contiguous() for x in (Q, K, V)]
    announce("attention full size: GPU")
    r = torch_api.attention_forward(*t, causal=wl.causal)
    torch.cuda.synchronize()
    O = r.O
    lse = r.lse
    assert bool(torch.isfinite(O).all()) and bool(torch.isfinite(lse).all())
    rng = np.random.default_rng(614)
    picks = [(0, 0, 0), (wl.B - 1, wl.H - 1, wl.S - 1), (3, 17, 127), (3, 17, 128),
             (5, 2, 1000)] + [(int(rng.integers(wl.B)), int(rng.integers(wl.H)),
                               int(rng.integers(wl.S))) for _ in range(11)]
    for b, h, q in picks:
        ref = oracle.attention_forward(Q[b, h, q:q + 1], K[b, h, :q + 1], V[b, h, :q + 1],
                                       causal=False)
        got = O[b, h, q].cpu().numpy()
        assert rel_l2(got[None], ref.O) <= 1e-2, (b, h, q, rel_l2(got[None], ref.O))
        assert abs(float(lse[b, h, q]) - float(ref.lse[0])) <= 2e-3, (b, h, q)
    announce("attention full size: V = 1")
    ones = torch.ones_like(t[2])
    r1 = torch_api.attention_forward(t[0], t[1], ones, causal=wl.causal)
    torch.cuda.synchronize()
    assert float((r1.O - 1.0).abs().max()) <= 1e-5


# ------------------------------------------------------------------ backward
#
# dQ, dK, dV against the fp64 oracle's exact gradient for the same bf16
# inputs and an upstream dO rounded to bf16.  Tolerance 1e-2 relative L2 per
# gradient (derived like the loss path's dH / dW: the probabilities and dS
# enter the products rounded to bf16, <= 2^-9 relative each, and every
# gradient is a sum of many such products).  The forward's O and lse feed
# the backward as they would in training.

def _run_bwd(Q, K, V, dO, causal, scale=None):
    import torch
    from vocab_cross_entropy_valid_amd import torch_api
    dev = torch.device("cuda:0")
    t = [torch.from_numpy(x).to(dev).to(torch.bfloat16).contiguous() for x in (Q, K, V, dO)]
    fwd = torch_api.attention_forward(*t[:3], causal=causal, scale=scale)
    g = torch_api.attention_backward(*t[:3], fwd, t[3], causal=causal, scale=scale)
    torch.cuda.synchronize()
    return g.dQ.cpu().numpy(), g.dK.cpu().numpy(), g.dV.cpu().numpy()


BWD_CASES = [
    # B, H, S, D, causal, seed
    (1, 2, 200, 64, False, 621),
    (2, 2, 257, 128, True, 622),     # ragged query, key and 32-query blocks
    (1, 1, 1, 128, True, 623),
    (1, 2, 130, 128, False, 624),
    (1, 3, 512, 128, True, 625),     # several key groups of 128, diagonal skips
    (1, 2, 40, 64, False, 628),      # two query blocks: the pipeline's shortest loop
    (2, 1, 96, 128, True, 629),      # three query blocks (every LDS slot used once)
    (1, 2, 700, 128, True, 630),     # 11 blocks of 64 queries: odd count, ragged tail
    (1, 1, 384, 128, False, 631),    # non-causal, 6 blocks of 64 (no masked path)
    # B * H a multiple of 8: the blocks of a group of heads (4 per XCD,
    # shrunk as in the forward) run interleaved, heaviest first, on one XCD
    (2, 4, 300, 128, True, 632),
    (1, 8, 200, 64, True, 633),
    (1, 16, 257, 128, False, 634),
    (2, 16, 260, 128, True, 635),    # groups of 4
    (1, 40, 130, 64, True, 636),     # B * H / 8 = 5: one head per group
]


@pytest.mark.parametrize("B,H,S,D,causal,seed", BWD_CASES)
def test_attention_backward_matches_oracle(B, H, S, D, causal, seed):
    announce(f"attention backward B{B} H{H} S{S} D{D} causal={causal}")
    Q, K, V = workloads.attention_inputs(B, H, S, D, seed)
    dO = workloads.attention_inputs(B, H, S, D, seed + 1000)[0]
    dQ, dK, dV = _run_bwd(Q, K, V, dO, causal)
    ref = oracle.attention_backward(Q, K, V, dO, causal=causal)
    for name, got, exp in (("dQ", dQ, ref.dQ), ("dK", dK, ref.dK), ("dV", dV, ref.dV)):
        assert np.all(np.isfinite(got)), name
        assert rel_l2(got, exp) <= 1e-2, (name, rel_l2(got, exp))


def test_attention_backward_explicit_scale_and_determinism():
    announce("attention backward explicit scale, determinism")
    Q, K, V = workloads.attention_inputs(1, 2, 190, 128, 626, std=2.0)
    dO = workloads.attention_inputs(1, 2, 190, 128, 627)[0]
    a = _run_bwd(Q, K, V, dO, True, scale=0.2)
    ref = oracle.attention_backward(Q, K, V, dO, causal=True, scale=0.2)
    for got, exp in zip(a, (ref.dQ, ref.dK, ref.dV)):
        assert rel_l2(got, exp) <= 1e-2
    b = _run_bwd(Q, K, V, dO, True, scale=0.2)
    assert all(np.array_equal(x, y) for x, y in zip(a, b))


@pytest.mark.slow
def test_attention_backward_full_size_sampled_heads():
    """The benchmarked shape; the oracle recomputes whole sampled heads."""
    import torch
    from vocab_cross_entropy_valid_amd import torch_api
    wl = workloads.ATTENTION
    announce("attention backward full size: inputs")
    Q, K, V = workloads.attention_inputs(wl.B, wl.H, wl.S, wl.D, wl.seed)
    dO = workloads.attention_inputs(wl.B, wl.H, wl.S, wl.D, wl.seed + 1)[0]
    dev = torch.device("cuda:0")
    t = [torch.from_numpy(x).to(dev).to(torch.bfloat16).contiguous() for x in (Q, K, V, dO)]
    announce("attention backward full size: GPU")
    fwd = torch_api.attention_forward(*t[:3], causal=wl.causal)
    g = torch_api.attention_backward(*t[:3], fwd, t[3], causal=wl.causal)
    torch.cuda.synchronize()
    for b, hh in ((0, 0), (wl.B - 1, wl.H - 1), (3, 17)):
        ref = oracle.attention_backward(Q[b, hh], K[b, hh], V[b, hh], dO[b, hh], causal=wl.causal)
        for name, got, exp in (("dQ", g.dQ, ref.dQ), ("dK", g.dK, ref.dK), ("dV", g.dV, ref.dV)):
            r = rel_l2(got[b, hh].cpu().numpy(), exp)
            assert r <= 1e-2, (name, b, hh, r)
