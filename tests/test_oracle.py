"""The fp64 oracle against its pins, plus planted-mistake (mutation) checks.

A pin that still passes when a plausible mistake is planted in the oracle
tests nothing (the lesson of bug #138 on "6GB显卡预训练11亿参数模型", section
可证伪测试抓到的8个静默bug: a comparison that passes at zero difference).  Every
mutation below must make at least one pin fail.  Mistakes are planted in the
oracle, on the CPU.
"""
import math

import numpy as np
import pytest

import oracle.lce_oracle as O
from tests import oracle_pins as P


@pytest.mark.parametrize("pin", P.PINS, ids=lambda p: p.__name__)
def test_pin(pin):
    pin(O)


def _no_onehot(Z, lse, y, w):
    return np.exp(Z - lse[:, None]) * w


def _wrong_sign(Z, lse, y, w):
    P_ = np.exp(Z - lse[:, None])
    P_[np.arange(Z.shape[0]), y] -= 1.0
    return -P_ * w


def _unscaled(Z, lse, y, w):
    P_ = np.exp(Z - lse[:, None])
    P_[np.arange(Z.shape[0]), y] -= 1.0
    return P_


def _label_off_by_one(Z, y):
    return Z[np.arange(Z.shape[0]), (y + 1) % Z.shape[1]]


def _dropped_feature(Hb, W):
    Hb = np.asarray(Hb, dtype=np.float64)
    W = np.asarray(W, dtype=np.float64)
    return Hb[:, :-1] @ W[:, :-1].T


def _unshifted_lse(Z):
    with np.errstate(over="ignore"):
        return np.log(np.exp(Z).sum(axis=1))


def _max_only_lse(Z):
    return Z.max(axis=1)


def _keep_everything(labels, ignore_index):
    return np.ones(np.asarray(labels).shape, dtype=bool)


def _mean_over_all(reduction, grad, n_valid):
    return grad / (n_valid + 2)


def _softmax_wrong_axis(Z, lse, y, w):
    # normalise over the wrong axis (columns instead of rows)
    m = Z.max(axis=0)
    l0 = m + np.log(np.exp(Z - m[None, :]).sum(axis=0))
    P_ = np.exp(Z - l0[None, :])
    P_[np.arange(Z.shape[0]), y] -= 1.0
    return P_ * w


_orig_shard_partials = O.shard_partials
_orig_shard_backward = O.shard_backward


def _merge_without_rescale(parts, valid_idx):
    # sums the shards' s without bringing them to a common max
    N = parts[0].part_max.shape[0]
    loss = np.zeros(N)
    lse = np.zeros(N)
    v = np.asarray(valid_idx)
    M = np.stack([p.part_max[v] for p in parts]).max(axis=0)
    S = np.stack([p.part_sum[v] for p in parts]).sum(axis=0)
    lse[v] = M + np.log(S)
    loss[v] = lse[v] - np.stack([p.part_target[v] for p in parts]).max(axis=0)
    s = float(loss[v].sum())
    return loss, lse, s, s / max(v.size, 1)


def _shard_label_not_offset(H, W_shard, labels, v_begin, V_total, ignore_index=-100, **kw):
    # forgets that a shard's row 0 is vocabulary entry v_begin
    return _orig_shard_partials(H, W_shard, labels, 0, V_total, ignore_index, **kw)


def _shard_backward_local_lse(H, W_shard, labels, lse, v_begin, V_total, ignore_index=-100, **kw):
    # normalises by the shard's own logsumexp instead of the global one
    p = _orig_shard_partials(H, W_shard, labels, v_begin, V_total, ignore_index)
    local = np.where(p.part_sum > 0, p.part_max + np.log(np.maximum(p.part_sum, 1e-300)), 0.0)
    return _orig_shard_backward(H, W_shard, labels, local, v_begin, V_total, ignore_index, **kw)


def _embed_bwd_keeps_padding(dX, input_ids, pad_id, V):
    dX = np.asarray(dX, dtype=np.float64)
    ids = np.asarray(input_ids, dtype=np.int64)
    dW = np.zeros((V, dX.shape[1]))
    for n in range(ids.shape[0]):
        if 0 <= ids[n] < V:
            dW[ids[n]] += dX[n]
    return dW


def _embed_bwd_overwrites(dX, input_ids, pad_id, V):
    # a repeated id keeps only its last row instead of the sum
    dX = np.asarray(dX, dtype=np.float64)
    ids = np.asarray(input_ids, dtype=np.int64)
    dW = np.zeros((V, dX.shape[1]))
    for n in np.flatnonzero(ids != pad_id):
        dW[ids[n]] = dX[n]
    return dW


def _embed_fwd_off_by_one(W, input_ids, pad_id):
    W = np.asarray(W, dtype=np.float64)
    ids = np.asarray(input_ids, dtype=np.int64)
    idx = np.flatnonzero(ids != pad_id).astype(np.int32)
    X = np.zeros((ids.shape[0], W.shape[1]))
    X[idx] = W[(ids[idx] + 1) % W.shape[0]]
    return X, idx


_orig_opt = O.optimizer_step


def _adamw_without_bias_correction(p, g, kind, lr, weight_decay=0.0, beta1=0.9, beta2=0.999,
                                   eps=1e-8, step=1, exp_avg=None, exp_avg_sq=None):
    if kind != "adamw":
        return _orig_opt(p, g, kind, lr, weight_decay, beta1, beta2, eps, step, exp_avg,
                         exp_avg_sq)
    p = np.asarray(p, dtype=np.float64) * (1.0 - lr * weight_decay)
    m = beta1 * np.asarray(exp_avg) + (1.0 - beta1) * g
    v = beta2 * np.asarray(exp_avg_sq) + (1.0 - beta2) * g * g
    return p - lr * m / (np.sqrt(v) + eps), m, v


def _adamw_coupled_decay(p, g, kind, lr, weight_decay=0.0, beta1=0.9, beta2=0.999,
                         eps=1e-8, step=1, exp_avg=None, exp_avg_sq=None):
    # Adam with L2 decay folded into the gradient instead of AdamW's decoupled decay
    if kind != "adamw":
        return _orig_opt(p, g, kind, lr, weight_decay, beta1, beta2, eps, step, exp_avg,
                         exp_avg_sq)
    p = np.asarray(p, dtype=np.float64)
    return _orig_opt(p, np.asarray(g) + weight_decay * p, kind, lr, 0.0, beta1, beta2, eps, step,
                     exp_avg, exp_avg_sq)


def _sgd_ascends(p, g, kind, lr, weight_decay=0.0, *a, **k):
    if kind != "sgd":
        return _orig_opt(p, g, kind, lr, weight_decay, *a, **k)
    return np.asarray(p) + lr * (np.asarray(g) + weight_decay * np.asarray(p)), None, None


# attention
def _attn_scale_dropped(Q, K, scale):
    return np.asarray(Q, dtype=np.float64) @ np.swapaxes(np.asarray(K, dtype=np.float64), -1, -2)


def _attn_mask_transposed(S):
    return np.arange(S)[None, :] >= np.arange(S)[:, None]


def _attn_mask_strict(S):
    return np.arange(S)[None, :] < np.arange(S)[:, None]


_orig_attn = O.attention_forward


def _attn_softmax_over_queries(Q, K, V, causal=False, scale=None):
    Q = np.asarray(Q, dtype=np.float64)
    S, D = Q.shape[-2], Q.shape[-1]
    scale = 1.0 / np.sqrt(D) if scale is None else scale
    Z = O.attention_scores(Q, K, scale)
    if causal:
        Z = np.where(O.causal_allowed(S), Z, -np.inf)
    Zt = np.swapaxes(Z, -1, -2)
    lse = O.logsumexp_rows(Zt.reshape(-1, S)).reshape(Zt.shape[:-1])
    P = np.swapaxes(np.exp(Zt - lse[..., None]), -1, -2)
    return O.AttentionResult(O=P @ np.asarray(V, dtype=np.float64), lse=lse)


def _attn_lse_base2(Q, K, V, causal=False, scale=None):
    r = _orig_attn(Q, K, V, causal, scale)
    return O.AttentionResult(O=r.O, lse=r.lse / np.log(2.0))


def _attn_unshifted(Q, K, V, causal=False, scale=None):
    Q = np.asarray(Q, dtype=np.float64)
    S, D = Q.shape[-2], Q.shape[-1]
    scale = 1.0 / np.sqrt(D) if scale is None else scale
    Z = O.attention_scores(Q, K, scale)
    if causal:
        Z = np.where(O.causal_allowed(S), Z, -np.inf)
    with np.errstate(over="ignore", invalid="ignore"):
        E = np.exp(Z)
        lse = np.log(E.sum(-1))
        return O.AttentionResult(O=(E / E.sum(-1, keepdims=True)) @ np.asarray(V, dtype=np.float64),
                                 lse=lse)


_orig_attn_bwd = O.attention_backward


def _attn_bwd_no_rowdot(dO, Oo):
    return np.zeros(np.asarray(dO).shape[:-1])


def _attn_bwd_dk_unscaled(Q, K, V, dO, causal=False, scale=None):
    g = _orig_attn_bwd(Q, K, V, dO, causal, scale)
    D = np.asarray(Q).shape[-1]
    s = 1.0 / np.sqrt(D) if scale is None else scale
    return O.AttentionGrads(dQ=g.dQ, dK=g.dK / s, dV=g.dV)


def _attn_bwd_dv_untransposed(Q, K, V, dO, causal=False, scale=None):
    g = _orig_attn_bwd(Q, K, V, dO, causal, scale)
    Qd = np.asarray(Q, dtype=np.float64)
    s = 1.0 / np.sqrt(Qd.shape[-1]) if scale is None else scale
    Z = O.attention_scores(Qd, K, s)
    if causal:
        Z = np.where(O.causal_allowed(Qd.shape[-2]), Z, -np.inf)
    f = O.attention_forward(Q, K, V, causal, scale)
    P = np.exp(Z - f.lse[..., None])
    return O.AttentionGrads(dQ=g.dQ, dK=g.dK, dV=P @ np.asarray(dO, dtype=np.float64))


def _bf16_truncate(x):
    # rounds toward zero instead of to nearest
    x = np.asarray(x, dtype=np.float32)
    return (x.view(np.uint32) & np.uint32(0xFFFF0000)).view(np.float32)


def _bf16_ties_away(x):
    # a tie goes away from zero instead of to the even neighbour
    x = np.asarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    r = ((u + 0x8000) & 0xFFFF0000).astype(np.uint32).view(np.float32).copy()
    r[np.isnan(x)] = np.nan
    return r


def _bf16_ties_odd(x):
    # a tie goes to the odd neighbour
    x = np.asarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    odd = (u >> 16) & 1
    r = ((u + 0x8000 - odd) & 0xFFFF0000).astype(np.uint32).view(np.float32).copy()
    r[np.isnan(x)] = np.nan
    return r


MUTATIONS = {
    "bf16_truncates": ("round_to_bf16", _bf16_truncate),
    "bf16_ties_away_from_zero": ("round_to_bf16", _bf16_ties_away),
    "bf16_ties_to_odd": ("round_to_bf16", _bf16_ties_odd),
    "attn_bwd_without_row_dot": ("attention_row_dot", _attn_bwd_no_rowdot),
    "attn_bwd_dk_unscaled": ("attention_backward", _attn_bwd_dk_unscaled),
    "attn_bwd_dv_untransposed": ("attention_backward", _attn_bwd_dv_untransposed),
    "attn_scale_dropped": ("attention_scores", _attn_scale_dropped),
    "attn_mask_transposed": ("causal_allowed", _attn_mask_transposed),
    "attn_mask_excludes_diagonal": ("causal_allowed", _attn_mask_strict),
    "attn_softmax_over_queries": ("attention_forward", _attn_softmax_over_queries),
    "attn_lse_base2": ("attention_forward", _attn_lse_base2),
    "attn_without_max_shift": ("attention_forward", _attn_unshifted),
    "adamw_without_bias_correction": ("optimizer_step", _adamw_without_bias_correction),
    "adamw_coupled_weight_decay": ("optimizer_step", _adamw_coupled_decay),
    "sgd_ascends": ("optimizer_step", _sgd_ascends),
    "embed_backward_keeps_padding": ("embed_backward", _embed_bwd_keeps_padding),
    "embed_backward_overwrites_repeats": ("embed_backward", _embed_bwd_overwrites),
    "embed_forward_id_off_by_one": ("embed_forward", _embed_fwd_off_by_one),
    "shard_merge_without_rescale": ("merge_partials", _merge_without_rescale),
    "shard_label_not_offset": ("shard_partials", _shard_label_not_offset),
    "shard_backward_local_lse": ("shard_backward", _shard_backward_local_lse),
    "dlogits_without_onehot": ("dlogits", _no_onehot),
    "dlogits_wrong_sign": ("dlogits", _wrong_sign),
    "dlogits_missing_scale": ("dlogits", _unscaled),
    "dlogits_softmax_over_wrong_axis": ("dlogits", _softmax_wrong_axis),
    "target_label_off_by_one": ("target_logits", _label_off_by_one),
    "logits_dropped_feature": ("logits", _dropped_feature),
    "lse_without_max_shift": ("logsumexp_rows", _unshifted_lse),
    "lse_max_only": ("logsumexp_rows", _max_only_lse),
    "ignore_index_not_skipped": ("valid_mask", _keep_everything),
    "mean_over_wrong_count": ("_scale", _mean_over_all),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(name, monkeypatch):
    attr, fn = MUTATIONS[name]
    monkeypatch.setattr(O, attr, fn)
    failed = P.run_pins(O)
    assert failed, f"mutation {name} passed every pin"


def test_statistical_band_tiny_fp32():
    """Gaussian inputs: mean loss ~ ln V + sigma^2/2 with
    sigma^2 = d Var(H) Var(W) (sanity check of generator + oracle)."""
    from workloads import generate, CONFIGS
    wl = CONFIGS[1]
    H, W, y = generate(1)
    f = O.forward(H, W, y, -100)
    assert f.valid_count == 58
    s2 = wl.d * wl.h_std ** 2 * wl.w_std ** 2
    exp = math.log(wl.V) + s2 / 2
    sd = math.sqrt(s2) / math.sqrt(f.valid_count) + 1e-6
    assert abs(f.loss_mean - exp) < 5 * sd
