"""Pins that tie the fp64 oracle to facts outside itself.

Each pin checks the oracle against something the mathematics fixes: closed
forms (W = 0, H = 0, V = 1, V = 2), invariants (rows of softmax - onehot sum
to zero, shift invariance, permutation equivariance, independence from
ignored rows), central finite differences of the loss, a 50-digit evaluation
of -log softmax from the exact rational logits, and PyTorch's CPU float64
cross_entropy (a library routine the oracle does not use).  ``run_pins`` is
reused by the mutation tests, which plant one plausible mistake at a time in
the oracle and require at least one pin to fail.
"""
from __future__ import annotations

import math
from fractions import Fraction

import numpy as np

IGN = -100


def _case(seed, N=9, d=6, V=11, n_ign=2, scale=1.0):
    rng = np.random.default_rng(seed)
    H = rng.standard_normal((N, d)) * scale
    W = rng.standard_normal((V, d)) * scale
    y = rng.integers(0, V, N).astype(np.int64)
    y[rng.choice(N, n_ign, replace=False)] = IGN
    return H, W, y


# ---------------------------------------------------------------- closed forms

def pin_w_zero(o):
    """W = 0: every valid loss is ln V, dH = 0 and
    dW[v] = w (sum_valid H_n / V - sum_{valid, y_n = v} H_n)."""
    H, _, y = _case(1)
    V = 11
    W = np.zeros((V, H.shape[1]))
    f = o.forward(H, W, y, IGN)
    dH, dW = o.backward(H, W, y, IGN)
    valid = y != IGN
    nv = int(valid.sum())
    assert f.valid_count == nv
    np.testing.assert_allclose(f.loss[valid], math.log(V), rtol=0, atol=4e-16)
    assert np.all(f.loss[~valid] == 0)
    assert np.all(dH == 0)
    w = 1.0 / nv
    exp = np.tile(H[valid].sum(0) / V, (V, 1))
    for n in np.flatnonzero(valid):
        exp[y[n]] -= H[n]
    np.testing.assert_allclose(dW, w * exp, rtol=1e-13, atol=1e-15)
    assert abs(f.loss_mean - math.log(V)) < 1e-15


def pin_h_zero(o):
    """H = 0: every valid loss is ln V, dW = 0 and
    dH[n] = w (sum_v W_v / V - W[y_n]) on valid rows, 0 on ignored rows."""
    _, W, y = _case(2)
    H = np.zeros((y.size, W.shape[1]))
    V = W.shape[0]
    f = o.forward(H, W, y, IGN)
    dH, dW = o.backward(H, W, y, IGN, reduction="sum", grad=0.5)
    valid = y != IGN
    np.testing.assert_allclose(f.loss[valid], math.log(V), rtol=0, atol=4e-16)
    assert np.all(dW == 0)
    for n in range(y.size):
        if valid[n]:
            np.testing.assert_allclose(dH[n], 0.5 * (W.mean(0) - W[y[n]]),
                                       rtol=1e-13, atol=1e-15)
        else:
            assert np.all(dH[n] == 0)


def pin_v_one(o):
    """V = 1: the only class has probability 1, so loss and gradients vanish."""
    H, W, y = _case(3, V=1)
    y[y != IGN] = 0
    f = o.forward(H, W, y, IGN)
    dH, dW = o.backward(H, W, y, IGN)
    assert np.all(np.abs(f.loss) <= 1e-15)
    assert np.abs(dH).max() <= 1e-15 and np.abs(dW).max() <= 1e-15


def pin_two_class(o):
    """V = 2 is logistic regression: loss = log(1 + exp(z_o - z_y)) and
    dloss/dH_n = sigma(z_o - z_y) (W_o - W_y) (sum reduction, grad 1)."""
    H, W, y = _case(4, V=2, n_ign=1)
    f = o.forward(H, W, y, IGN)
    dH, _ = o.backward(H, W, y, IGN, reduction="sum")
    for n in range(y.size):
        if y[n] == IGN:
            continue
        other = 1 - y[n]
        t = float(H[n] @ W[other] - H[n] @ W[y[n]])
        exp_loss = math.log1p(math.exp(t)) if t < 30 else t + math.log1p(math.exp(-t))
        assert abs(f.loss[n] - exp_loss) <= 1e-13 * max(1.0, exp_loss)
        sig = 1.0 / (1.0 + math.exp(-t))
        np.testing.assert_allclose(dH[n], sig * (W[other] - W[y[n]]), rtol=1e-12, atol=1e-14)


# ---------------------------------------------------------------- invariants

def pin_dw_colsum(o):
    """Rows of softmax - onehot sum to 0, hence sum_v dW[v, :] = 0."""
    H, W, y = _case(5, N=13, d=7, V=17)
    _, dW = o.backward(H, W, y, IGN)
    assert np.abs(dW.sum(0)).max() <= 1e-14 * max(1.0, np.abs(dW).max())
    assert np.abs(dW).max() > 1e-3  # non-trivial


def pin_shift_invariance(o):
    """Adding c to every row of W adds H_n.c to every logit of row n, which
    leaves loss and dH unchanged; a huge common logit offset must stay finite."""
    H, W, y = _case(6)
    c = np.random.default_rng(60).standard_normal(W.shape[1])
    f0 = o.forward(H, W, y, IGN)
    f1 = o.forward(H, W + c, y, IGN)
    np.testing.assert_allclose(f1.loss, f0.loss, rtol=1e-10, atol=1e-12)
    dH0, _ = o.backward(H, W, y, IGN)
    dH1, _ = o.backward(H, W + c, y, IGN)
    np.testing.assert_allclose(dH1, dH0, rtol=1e-9, atol=1e-12)
    # large offset: append a feature of 1s to H and a column 1000 to W
    Hb = np.concatenate([H, np.ones((H.shape[0], 1))], 1)
    Wb = np.concatenate([W, np.full((W.shape[0], 1), 1000.0)], 1)
    f2 = o.forward(Hb, Wb, y, IGN)
    assert np.all(np.isfinite(f2.loss))
    np.testing.assert_allclose(f2.loss, f0.loss, rtol=1e-9, atol=1e-9)


def pin_permutation(o):
    """Permuting W's rows and relabelling permutes dW's rows the same way."""
    H, W, y = _case(7)
    V = W.shape[0]
    perm = np.random.default_rng(70).permutation(V)
    inv = np.argsort(perm)
    y2 = y.copy()
    y2[y != IGN] = inv[y[y != IGN]]          # new row inv[v] holds old row v
    W2 = W[perm]
    f0, f1 = o.forward(H, W, y, IGN), o.forward(H, W2, y2, IGN)
    np.testing.assert_allclose(f1.loss, f0.loss, rtol=1e-12, atol=1e-14)
    _, dW0 = o.backward(H, W, y, IGN)
    _, dW1 = o.backward(H, W2, y2, IGN)
    np.testing.assert_allclose(dW1, dW0[perm], rtol=1e-11, atol=1e-14)


def pin_ignored_rows(o):
    """Ignored rows contribute nothing: giving their H rows huge values changes
    no output, their loss and dH rows are 0, and the count excludes them."""
    H, W, y = _case(8, n_ign=3)
    ign = y == IGN
    H2 = H.copy()
    H2[ign] = 1e3
    f0, f1 = o.forward(H, W, y, IGN), o.forward(H2, W, y, IGN)
    assert f0.valid_count == int((~ign).sum()) == f1.valid_count
    np.testing.assert_array_equal(f0.loss, f1.loss)
    assert np.all(f0.loss[ign] == 0)
    dH0, dW0 = o.backward(H, W, y, IGN)
    dH1, dW1 = o.backward(H2, W, y, IGN)
    np.testing.assert_array_equal(dW0, dW1)
    assert np.all(dH1[ign] == 0)
    np.testing.assert_array_equal(dH0, dH1)
    assert np.all(f0.loss[~ign] > 0)


def pin_ignore_inside_range(o):
    """ignore_index may be a real class id: those rows are skipped."""
    H, W, y = _case(9, n_ign=0)
    y[[0, 3]] = 4
    f = o.forward(H, W, y, 4)
    keep = y != 4
    assert f.valid_count == int(keep.sum())
    assert np.all(f.loss[~keep] == 0)
    g = o.forward(H[keep], W, y[keep], IGN)
    np.testing.assert_allclose(f.loss[keep], g.loss, rtol=1e-14, atol=0)


def pin_bad_label(o):
    """A valid label outside [0, V) is an error, not an out-of-bounds read."""
    H, W, y = _case(10)
    y[np.flatnonzero(y != IGN)[0]] = W.shape[0]
    try:
        o.forward(H, W, y, IGN)
    except ValueError:
        pass
    else:
        raise AssertionError("label == V was accepted")
    y[np.flatnonzero(y != IGN)[0]] = -5
    try:
        o.backward(H, W, y, IGN)
    except ValueError:
        pass
    else:
        raise AssertionError("label -5 was accepted")


# ------------------------------------------------------------ finite differences

def pin_finite_differences(o):
    """Central differences of the mean loss match dH and dW entry by entry."""
    H, W, y = _case(11, N=5, d=4, V=7, n_ign=1)
    dH, dW = o.backward(H, W, y, IGN)

    def mean_loss(Hx, Wx):
        return o.forward(Hx, Wx, y, IGN).loss_mean

    for arr, grad, which in ((H, dH, 0), (W, dW, 1)):
        num = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            h = 1e-6 * max(1.0, abs(arr[idx]))
            a, b = arr.copy(), arr.copy()
            a[idx] += h
            b[idx] -= h
            fa = mean_loss(a, W) if which == 0 else mean_loss(H, a)
            fb = mean_loss(b, W) if which == 0 else mean_loss(H, b)
            num[idx] = (fa - fb) / (2 * h)
        np.testing.assert_allclose(grad, num, rtol=1e-6, atol=1e-9)
    assert np.all(dH[y == IGN] == 0)


# ---------------------------------------------------- high precision brute force

def pin_mpmath(o):
    """loss_n = -log(exp(z_y) / sum_v exp(z_v)) with z the exact rational dot
    product of the float inputs, evaluated with 50 significant digits."""
    import mpmath
    mpmath.mp.dps = 50
    H, W, y = _case(12, N=6, d=5, V=9, n_ign=1, scale=3.0)
    f = o.forward(H, W, y, IGN)
    total = mpmath.mpf(0)
    nv = 0
    for n in range(y.size):
        if y[n] == IGN:
            assert f.loss[n] == 0
            continue
        z = [sum(Fraction(float(H[n, k])) * Fraction(float(W[v, k]))
                 for k in range(H.shape[1])) for v in range(W.shape[0])]
        zs = [mpmath.mpf(q.numerator) / q.denominator for q in z]
        p = mpmath.exp(zs[y[n]]) / mpmath.fsum(mpmath.exp(t) for t in zs)
        ref = -mpmath.log(p)
        assert abs(f.loss[n] - float(ref)) <= 1e-13 * max(1.0, abs(float(ref)))
        total += ref
        nv += 1
    assert abs(f.loss_mean - float(total / nv)) <= 1e-13


# -------------------------------------------------------------- library routine

def pin_torch_cross_entropy(o):
    """PyTorch CPU float64 cross_entropy with ignore_index and autograd."""
    import torch
    import torch.nn.functional as F
    for seed, red in ((13, "mean"), (14, "sum")):
        H, W, y = _case(seed, N=23, d=8, V=19, n_ign=4)
        Ht = torch.tensor(H, requires_grad=True)
        Wt = torch.tensor(W, requires_grad=True)
        loss = F.cross_entropy(Ht @ Wt.T, torch.tensor(y), ignore_index=IGN, reduction=red)
        loss.backward()
        f = o.forward(H, W, y, IGN)
        dH, dW = o.backward(H, W, y, IGN, reduction=red)
        ref = f.loss_mean if red == "mean" else f.loss_sum
        assert abs(ref - loss.item()) <= 1e-13 * max(1.0, abs(loss.item()))
        per = F.cross_entropy(Ht.detach() @ Wt.detach().T, torch.tensor(y),
                              ignore_index=IGN, reduction="none").numpy()
        np.testing.assert_allclose(f.loss, per, rtol=1e-13, atol=1e-15)
        np.testing.assert_allclose(dH, Ht.grad.numpy(), rtol=1e-12, atol=1e-15)
        np.testing.assert_allclose(dW, Wt.grad.numpy(), rtol=1e-12, atol=1e-15)


# ----------------------------------------------------- row-sampled entry points

def pin_row_functions(o):
    """The per-row helpers used for sampled checks agree with the full pass
    (the full pass itself is pinned above)."""
    H, W, y = _case(15, N=17, d=5, V=13, n_ign=3)
    f = o.forward(H, W, y, IGN)
    dH, dW = o.backward(H, W, y, IGN)
    rows = f.valid_idx[::2]
    l, loss, _ = o.rows_forward(H, W, y, rows)
    np.testing.assert_allclose(l, f.lse[rows], rtol=1e-14)
    np.testing.assert_allclose(loss, f.loss[rows], rtol=1e-14)
    w = 1.0 / f.valid_count
    np.testing.assert_allclose(o.rows_dH(H, W, y, rows, w), dH[rows], rtol=1e-12, atol=1e-16)
    vr = np.array([0, 3, 12])
    got = o.rows_dW(H, W, y, f.valid_idx, f.lse[f.valid_idx], vr, w, row_block=4)
    np.testing.assert_allclose(got, dW[vr], rtol=1e-12, atol=1e-16)


def pin_compaction(o):
    """valid_idx is the ascending list of rows whose label is kept, found by a
    plain loop; out-of-range labels are reported, not kept."""
    rng = np.random.default_rng(16)
    y = rng.integers(-3, 40, 200).astype(np.int64)
    y[rng.choice(200, 50, replace=False)] = IGN
    idx, n, bad = o.compact_valid(y, IGN, 37)
    exp_idx, exp_bad = [], []
    for r in range(200):
        if y[r] == IGN:
            continue
        (exp_idx if 0 <= y[r] < 37 else exp_bad).append(r)
    assert n == len(exp_idx)
    assert idx.tolist() == exp_idx and idx.dtype == np.int32
    assert bad.tolist() == exp_bad


# ------------------------------------------------------- vocabulary shards

_PARTITIONS = ([(0, 11)], [(0, 3), (3, 4), (4, 11)], [(0, 5), (5, 11)],
               [(v, v + 1) for v in range(11)])


def pin_shard_merge_identity(o):
    """logsumexp over a union of disjoint slices equals the logsumexp of the
    slices' own (max, scaled sum) pairs: merging the partials of any
    partition of the vocabulary, in any shard order, reproduces the full
    forward (which the pins above tie to mpmath and PyTorch)."""
    H, W, y = _case(17, N=13, d=5, V=11, n_ign=3)
    f = o.forward(H, W, y, IGN)
    for part in _PARTITIONS:
        parts = [o.shard_partials(H, W[a:b], y, a, 11, IGN) for a, b in part]
        for order in (parts, parts[::-1]):
            loss, lse, loss_sum, mean = o.merge_partials(order, f.valid_idx)
            np.testing.assert_allclose(lse, f.lse, rtol=1e-13, atol=1e-13)
            np.testing.assert_allclose(loss, f.loss, rtol=1e-12, atol=1e-12)
            assert abs(loss_sum - f.loss_sum) <= 1e-12 * abs(f.loss_sum)


def pin_shard_partials_definition(o):
    """One shard holding the whole vocabulary: m + log s is the row's lse, t
    its target logit, s >= 1 on valid rows and 0 on ignored ones; a shard that
    does not hold the label reports -inf."""
    H, W, y = _case(18, N=12, d=4, V=9, n_ign=3)
    f = o.forward(H, W, y, IGN)
    p = o.shard_partials(H, W, y, 0, 9, IGN)
    v = f.valid_idx
    ign = np.setdiff1d(np.arange(12), v)
    np.testing.assert_allclose(p.part_max[v] + np.log(p.part_sum[v]), f.lse[v], rtol=1e-14)
    _, _, zt = o.rows_forward(H, W, y, v)
    np.testing.assert_allclose(p.part_target[v], zt, rtol=1e-14)
    assert np.all(p.part_sum[v] >= 1.0) and np.all(p.part_sum[ign] == 0.0)
    lo = o.shard_partials(H, W[:4], y, 0, 9, IGN)
    assert np.all(np.isneginf(lo.part_target[v[y[v] >= 4]]))
    assert np.all(np.isfinite(lo.part_target[v[y[v] < 4]]))


def pin_shard_backward_sum(o):
    """The shards' dH shares sum to the full dH and their dW rows stack to
    the full dW (G restricted to a shard's columns, with the global lse)."""
    H, W, y = _case(19, N=10, d=5, V=11, n_ign=2)
    f = o.forward(H, W, y, IGN)
    dH, dW = o.backward(H, W, y, IGN, grad=1.7)
    for part in _PARTITIONS[1:3]:
        sH = np.zeros_like(dH)
        rows = []
        for a, b in part:
            h, w_ = o.shard_backward(H, W[a:b], y, f.lse, a, 11, IGN, grad=1.7)
            sH += h
            rows.append(w_)
        np.testing.assert_allclose(sH, dH, rtol=1e-12, atol=1e-15)
        np.testing.assert_allclose(np.concatenate(rows), dW, rtol=1e-12, atol=1e-15)


# ------------------------------------------------ tied table: input side

def _ids_case(seed, N=40, V=13, pad=0, n_pad=9):
    rng = np.random.default_rng(seed)
    ids = rng.integers(0, V, N).astype(np.int64)
    ids[rng.choice(N, n_pad, replace=False)] = pad
    ids[:3] = 5                      # an id repeated at the start
    return ids


def pin_embed_adjoint(o):
    """The lookup is linear in W (X = E W with E the masked one-hot matrix),
    so its gradient is the adjoint: <dX, E W'> = <E^T dX, W'> for any W'."""
    rng = np.random.default_rng(20)
    ids = _ids_case(20)
    W = rng.standard_normal((13, 6))
    dX = rng.standard_normal((40, 6))
    X, _ = o.embed_forward(W, ids, 0)
    dW = o.embed_backward(dX, ids, 0, 13)
    lhs = float((dX * X).sum())
    rhs = float((dW * W).sum())
    assert abs(lhs - rhs) <= 1e-12 * (abs(lhs) + 1.0)


def pin_embed_dense(o):
    """Forward and backward against the dense one-hot matrix E [N, V] (E[n, v]
    = 1 when n is not padding and id[n] = v): X = E W and dW = E^T dX by
    numpy's matrix product; padding rows of X are zero."""
    rng = np.random.default_rng(21)
    ids = _ids_case(21, pad=3)
    W = rng.standard_normal((13, 5))
    dX = rng.standard_normal((40, 5))
    E = np.zeros((40, 13))
    keep = ids != 3
    E[np.flatnonzero(keep), ids[keep]] = 1.0
    X, idx = o.embed_forward(W, ids, 3)
    np.testing.assert_allclose(X, E @ W, rtol=0, atol=0)
    np.testing.assert_allclose(o.embed_backward(dX, ids, 3, 13), E.T @ dX, rtol=1e-13, atol=1e-13)
    assert idx.tolist() == np.flatnonzero(keep).tolist()
    assert not X[~keep].any()


def pin_embed_bad_id(o):
    """An id outside [0, V) that is not the padding id is an error."""
    ids = _ids_case(22)
    ids[7] = 13
    for fn in (lambda: o.embed_forward(np.zeros((13, 2)), ids, 0),
               lambda: o.embed_backward(np.zeros((40, 2)), ids, 0, 13)):
        try:
            fn()
        except ValueError:
            continue
        raise AssertionError("out-of-range id accepted")


# --------------------------------------------------- optimizer step

def pin_sgd_matches_torch(o):
    """One SGD step (weight decay, no momentum) equals torch.optim.SGD in fp64."""
    import torch
    rng = np.random.default_rng(23)
    p0 = rng.standard_normal((7, 5))
    g = rng.standard_normal((7, 5))
    t = torch.tensor(p0, dtype=torch.float64, requires_grad=True)
    t.grad = torch.tensor(g)
    torch.optim.SGD([t], lr=0.3, weight_decay=0.05).step()
    p1, _, _ = o.optimizer_step(p0, g, "sgd", 0.3, 0.05)
    np.testing.assert_allclose(p1, t.detach().numpy(), rtol=1e-14, atol=1e-15)


def pin_adamw_matches_torch(o):
    """AdamW at step t = 4 from given moment estimates equals torch.optim.AdamW
    in fp64 (decoupled weight decay, bias correction)."""
    import torch
    rng = np.random.default_rng(24)
    p0 = rng.standard_normal((6, 4))
    g = rng.standard_normal((6, 4)) * 1e-3
    m0 = rng.standard_normal((6, 4)) * 1e-3
    v0 = rng.random((6, 4)) * 1e-6
    t = torch.tensor(p0, dtype=torch.float64, requires_grad=True)
    opt = torch.optim.AdamW([t], lr=1e-2, betas=(0.8, 0.95), eps=1e-7, weight_decay=0.1)
    opt.state[t] = {"step": torch.tensor(3.0, dtype=torch.float64),
                    "exp_avg": torch.tensor(m0), "exp_avg_sq": torch.tensor(v0)}
    t.grad = torch.tensor(g)
    opt.step()
    p1, m1, v1 = o.optimizer_step(p0, g, "adamw", 1e-2, 0.1, 0.8, 0.95, 1e-7, 4, m0, v0)
    np.testing.assert_allclose(p1, t.detach().numpy(), rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(m1, opt.state[t]["exp_avg"].numpy(), rtol=1e-13)
    np.testing.assert_allclose(v1, opt.state[t]["exp_avg_sq"].numpy(), rtol=1e-13)


# ---------------------------------------------------------------- attention
#
# The attention oracle (online-softmax attention, "OjasX 0.6.1", section
# 核心技术 / "Core Technology"; softmax(Q K^T / sqrt(d)) V as the KV-cache page
# writes it) against closed forms, invariants and torch's own fp64 routine.

def _qkv(seed, B=2, H=3, S=7, D=8, scale=1.0):
    rng = np.random.default_rng(seed)
    return [rng.standard_normal((B, H, S, D)) * scale for _ in range(3)]


def pin_attn_uniform(o):
    """Q = 0: every allowed key has the same score, so O is the mean of the
    allowed V rows and lse = log(number of allowed keys)."""
    _, K, V = _qkv(501)
    Q = np.zeros_like(K)
    S = K.shape[-2]
    r = o.attention_forward(Q, K, V, causal=False)
    np.testing.assert_allclose(r.O, np.broadcast_to(V.mean(axis=-2, keepdims=True), V.shape),
                               rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(r.lse, np.full(r.lse.shape, np.log(S)), rtol=1e-14)
    r = o.attention_forward(Q, K, V, causal=True)
    counts = np.arange(1, S + 1, dtype=np.float64)
    prefix_mean = np.cumsum(V, axis=-2) / counts[:, None]
    np.testing.assert_allclose(r.O, prefix_mean, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(r.lse, np.broadcast_to(np.log(counts), r.lse.shape), rtol=1e-14)


def pin_attn_single_key(o):
    """One key: O = V and lse = the single scaled score, causal or not."""
    Q, K, V = _qkv(502, S=1, D=16)
    for causal in (False, True):
        r = o.attention_forward(Q, K, V, causal=causal)
        np.testing.assert_allclose(r.O, V, rtol=1e-14)
        np.testing.assert_allclose(r.lse, (Q * K).sum(-1) / 4.0, rtol=1e-13)


def pin_attn_key_shift(o):
    """Adding one vector u to every key adds scale q.u to each score of row q:
    O is unchanged, lse moves by exactly that amount."""
    Q, K, V = _qkv(503, S=9, D=16)
    u = np.random.default_rng(5031).standard_normal(16) * 3.0
    for causal in (False, True):
        a = o.attention_forward(Q, K, V, causal=causal)
        b = o.attention_forward(Q, K + u, V, causal=causal)
        np.testing.assert_allclose(b.O, a.O, rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(b.lse - a.lse, (Q @ u) / 4.0, rtol=1e-11, atol=1e-12)


def pin_attn_permutation(o):
    """Without a mask, permuting keys and values together changes nothing."""
    Q, K, V = _qkv(504, S=11)
    perm = np.random.default_rng(5041).permutation(11)
    a = o.attention_forward(Q, K, V)
    b = o.attention_forward(Q, K[..., perm, :], V[..., perm, :])
    np.testing.assert_allclose(b.O, a.O, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(b.lse, a.lse, rtol=1e-13)


def pin_attn_rows_sum_to_one(o):
    """V = 1: each output is a convex combination of ones, so exactly 1."""
    Q, K, _ = _qkv(505, S=13, scale=2.0)
    V = np.ones_like(Q)
    for causal in (False, True):
        np.testing.assert_allclose(o.attention_forward(Q, K, V, causal=causal).O, 1.0,
                                   rtol=1e-13)


def pin_attn_causal_prefix(o):
    """Causal row q equals unmasked attention over keys 0..q only."""
    Q, K, V = _qkv(506, S=10)
    r = o.attention_forward(Q, K, V, causal=True)
    for q in (0, 3, 9):
        p = o.attention_forward(Q[..., q:q + 1, :], K[..., :q + 1, :], V[..., :q + 1, :])
        np.testing.assert_allclose(r.O[..., q, :], p.O[..., 0, :], rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(r.lse[..., q], p.lse[..., 0], rtol=1e-13)


def pin_attn_dominant_key(o):
    """A key whose score exceeds all others by ~1e3 takes all the weight (and
    the scores are far beyond exp's range without the max shift)."""
    Q, K, V = _qkv(507, B=1, H=1, S=6, D=4)
    Q[..., :, :] = 0.0
    Q[..., :, 0] = 1.0
    K[..., :, 0] = 0.0
    K[..., 2, 0] = 2000.0     # score 1000 after scale 1/2
    r = o.attention_forward(Q, K, V)
    np.testing.assert_allclose(r.O, np.broadcast_to(V[..., 2:3, :], V.shape), rtol=1e-12,
                               atol=1e-300)
    assert np.all(np.isfinite(r.lse)) and np.allclose(r.lse, 1000.0, rtol=1e-12)


def pin_attn_torch_sdpa(o):
    """torch's scaled_dot_product_attention in float64 (a library routine),
    with and without the causal mask, default scale 1 / sqrt(D)."""
    import torch
    import torch.nn.functional as F
    Q, K, V = _qkv(508, S=17, D=16)
    for causal in (False, True):
        ref = F.scaled_dot_product_attention(torch.tensor(Q), torch.tensor(K), torch.tensor(V),
                                             is_causal=causal).numpy()
        np.testing.assert_allclose(o.attention_forward(Q, K, V, causal=causal).O, ref,
                                   rtol=1e-11, atol=1e-12)


def pin_attn_backward_finite_differences(o):
    """Central differences of L = sum(dO * O) for every entry of Q, K and V."""
    Q, K, V = _qkv(511, B=1, H=1, S=4, D=3)
    dO = np.random.default_rng(5111).standard_normal(Q.shape)
    h = 1e-6
    for causal in (False, True):
        g = o.attention_backward(Q, K, V, dO, causal=causal)
        for X, G in ((Q, g.dQ), (K, g.dK), (V, g.dV)):
            for idx in np.ndindex(X.shape):
                old = X[idx]
                X[idx] = old + h
                lp = (dO * o.attention_forward(Q, K, V, causal=causal).O).sum()
                X[idx] = old - h
                lm = (dO * o.attention_forward(Q, K, V, causal=causal).O).sum()
                X[idx] = old
                assert abs((lp - lm) / (2 * h) - G[idx]) <= 1e-7 * max(1.0, abs(G[idx])), idx


def pin_attn_backward_torch(o):
    """torch float64 autograd through scaled_dot_product_attention."""
    import torch
    import torch.nn.functional as F
    Q, K, V = _qkv(512, S=9, D=8)
    dO = np.random.default_rng(5121).standard_normal(Q.shape)
    for causal in (False, True):
        t = [torch.tensor(x, requires_grad=True) for x in (Q, K, V)]
        F.scaled_dot_product_attention(*t, is_causal=causal).backward(torch.tensor(dO))
        g = o.attention_backward(Q, K, V, dO, causal=causal)
        for got, ref in ((g.dQ, t[0].grad), (g.dK, t[1].grad), (g.dV, t[2].grad)):
            np.testing.assert_allclose(got, ref.numpy(), rtol=1e-11, atol=1e-12)


def pin_attn_backward_closed_forms(o):
    """Q = 0 and dO = 1: P is uniform over the allowed keys, so dV[k] = sum_q
    P[q, k] = 1 without a mask and H_S - H_k (harmonic numbers) with the
    causal mask.  Equal V rows: O does not depend on P, so dQ = dK = 0.  Rows
    of dS sum to zero, so the keys' dK sum to zero."""
    _, K, V = _qkv(513, S=7)
    Q = np.zeros_like(K)
    ones = np.ones_like(Q)
    S = K.shape[-2]
    g = o.attention_backward(Q, K, V, ones, causal=False)
    np.testing.assert_allclose(g.dV, 1.0, rtol=1e-13)
    g = o.attention_backward(Q, K, V, ones, causal=True)
    Hn = np.concatenate([[0.0], np.cumsum(1.0 / np.arange(1, S + 1))])
    expect = (Hn[S] - Hn[:S])[:, None]
    np.testing.assert_allclose(g.dV, np.broadcast_to(expect, g.dV.shape), rtol=1e-13)
    Q, K, _ = _qkv(514, S=6)
    Vc = np.broadcast_to(np.random.default_rng(5141).standard_normal(8), Q.shape).copy()
    dO = np.random.default_rng(5142).standard_normal(Q.shape)
    for causal in (False, True):
        g = o.attention_backward(Q, K, Vc, dO, causal=causal)
        np.testing.assert_allclose(g.dQ, 0.0, atol=1e-13)
        np.testing.assert_allclose(g.dK, 0.0, atol=1e-13)
        Q2, K2, V2 = _qkv(515, S=6)
        g = o.attention_backward(Q2, K2, V2, dO, causal=causal)
        np.testing.assert_allclose(g.dK.sum(axis=-2), 0.0, atol=1e-12)


# ------------------------------------------------------------- output cast

def _bf16_sweep():
    rng = np.random.default_rng(700)
    x = np.concatenate([
        rng.standard_normal(4000).astype(np.float32) * np.float32(3.0),
        (rng.standard_normal(2000) * 1e-3).astype(np.float32),
        np.ldexp(rng.random(500) + 1.0, rng.integers(-149, 128, 500)).astype(np.float32),
        np.array([0.0, -0.0, 1.0, -1.0, np.inf, -np.inf, 3.3895314e38, -3.3895314e38,
                  3.4028235e38, 1e-45, -1e-45, 1.1754944e-38], dtype=np.float32),
    ])
    # exact ties: a bfloat16 value plus half its step, for even and odd last bits
    base = rng.integers(0x3F000000, 0x40000000, 300, dtype=np.uint64) & 0xFFFF0000
    ties = (base + 0x8000).astype(np.uint32).view(np.float32)
    # one bit either side of a tie
    near = np.concatenate([(base + 0x7FFF).astype(np.uint32).view(np.float32),
                           (base + 0x8001).astype(np.uint32).view(np.float32)])
    return np.concatenate([x, ties, -ties, near])


def pin_bf16_matches_torch(o):
    """Round to nearest even against PyTorch's CPU float32 -> bfloat16
    conversion (a library routine the oracle does not use), on random values,
    subnormals, values near the overflow threshold, exact ties and values one
    bit off a tie; NaN stays NaN."""
    import torch
    x = _bf16_sweep()
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    got = o.round_to_bf16(x)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))
    assert np.isnan(o.round_to_bf16(np.array([np.nan], np.float32)))[0]


def pin_bf16_closed_forms(o):
    """Values with the low 16 bits zero are unchanged; 1 + 2^-8 lies halfway
    between 1 (even) and 1 + 2^-7 (odd) and goes to 1; 1 + 3 2^-8 lies halfway
    between 1 + 2^-7 (odd) and 1 + 2^-6 (even) and goes up; the error never
    exceeds half a bfloat16 step and the rounding is monotone."""
    f = np.float32
    assert o.round_to_bf16(np.array([1 + 2.0 ** -8], f))[0] == 1.0
    assert o.round_to_bf16(np.array([1 + 3 * 2.0 ** -8], f))[0] == f(1 + 2.0 ** -6)
    assert o.round_to_bf16(np.array([-(1 + 3 * 2.0 ** -8)], f))[0] == f(-(1 + 2.0 ** -6))
    assert o.round_to_bf16(np.array([1 + 2.0 ** -8 + 2.0 ** -20], f))[0] == f(1 + 2.0 ** -7)
    x = _bf16_sweep()
    x = x[np.isfinite(x) & (np.abs(x) < 3.3e38)]
    r = o.round_to_bf16(x)
    assert np.all((r.view(np.uint32) & 0xFFFF) == 0)
    ex = x[(x.view(np.uint32) & 0xFFFF) == 0]
    assert np.array_equal(o.round_to_bf16(ex), ex)
    e = np.frexp(np.abs(x.astype(np.float64)))[1]
    step = np.ldexp(1.0, np.maximum(e, -125) - 8)
    assert np.all(np.abs(r.astype(np.float64) - x) <= step / 2)
    srt = np.sort(x)
    assert np.all(np.diff(o.round_to_bf16(srt).astype(np.float64)) >= 0)


PINS = [
    pin_w_zero, pin_h_zero, pin_v_one, pin_two_class, pin_dw_colsum,
    pin_shift_invariance, pin_permutation, pin_ignored_rows,
    pin_ignore_inside_range, pin_bad_label, pin_finite_differences,
    pin_mpmath, pin_torch_cross_entropy, pin_row_functions, pin_compaction,
    pin_shard_merge_identity, pin_shard_partials_definition, pin_shard_backward_sum,
    pin_embed_adjoint, pin_embed_dense, pin_embed_bad_id,
    pin_sgd_matches_torch, pin_adamw_matches_torch,
    pin_attn_uniform, pin_attn_single_key, pin_attn_key_shift, pin_attn_permutation,
    pin_attn_rows_sum_to_one, pin_attn_causal_prefix, pin_attn_dominant_key,
    pin_attn_torch_sdpa, pin_attn_backward_finite_differences, pin_attn_backward_torch,
    pin_attn_backward_closed_forms, pin_bf16_matches_torch, pin_bf16_closed_forms,
]


def run_pins(o, pins=PINS):
    """Names of the pins that fail for oracle module ``o``."""
    failed = []
    for p in pins:
        try:
            p(o)
        except Exception:  # noqa: BLE001 -- any error counts as a failed pin
            failed.append(p.__name__)
    return failed
