"""fp64 CPU oracle for fused linear + cross-entropy with ignored tokens.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
link this module: only ``tests/``, ``__graft_entry__.smoke()`` and the
benchmark's ``cpu_baseline`` leg use it.  It shares no code with the HIP
path.

What it computes is the plain definition of the result.  The pages describe
the method as reaching exactly this result with no approximation: the
projection and the loss are chunked into streaming steps that skip padding
tokens ("OjasX 0.6.1", section 核心技术 / "Core Technology": zero-byte
vocabulary logits table), the streaming max / normaliser recurrence gives
the same result as a full softmax (same page, paragraph on Online Softmax),
and the backward pass recomputes the logits chunk by chunk instead of saving
them ("6GB显卡预训练11亿参数模型", sections 内存实际花在哪里 and 关键参数说明,
--chunked-loss 512).  None of the pages writes the loss formula; the oracle
takes the textbook softmax cross-entropy that those passages name:

    z[n, v]   = sum_k H[n, k] * W[v, k]                 (output projection)
    lse[n]    = log sum_v exp(z[n, v])
    loss[n]   = lse[n] - z[n, y[n]]       for valid n, 0 for ignored n
    mean      = sum_n loss[n] / N_valid

and its exact gradient

    G[n, v]   = (exp(z[n, v] - lse[n]) - [v == y[n]]) * w,
                w = grad / N_valid ("mean") or grad ("sum"), 0 for ignored n
    dH        = G @ W,    dW = G^T @ H.

A row is valid when its label differs from ignore_index (the pages' "skip
padding tokens"; the valid-mask of the MaximusLLM page, section 2.3).  A
valid label outside [0, V) is an error (the out-of-range index failure in
"6GB显卡预训练11亿参数模型", section 可证伪测试抓到的8个静默bug, #155).

Everything is computed in float64 from the given (already rounded) inputs.
numpy's matrix product serves as the plain matrix product.  Each row block
materialises its full [rows, V] logits: that is the point of an oracle.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

DEFAULT_ROW_BLOCK = 256


# --------------------------------------------------------------------------
# named steps (kept small so that each can be checked and mutated alone)
# --------------------------------------------------------------------------

def valid_mask(labels: np.ndarray, ignore_index: int) -> np.ndarray:
    """Rows that take part in the loss: label != ignore_index."""
    return np.asarray(labels) != ignore_index


def logits(Hb: np.ndarray, W: np.ndarray) -> np.ndarray:
    """z = Hb W^T in float64 (the output projection)."""
    return np.asarray(Hb, dtype=np.float64) @ np.asarray(W, dtype=np.float64).T


def logsumexp_rows(Z: np.ndarray) -> np.ndarray:
    """log sum_v exp(Z[:, v]), shifted by the row max for range safety."""
    m = Z.max(axis=1)
    return m + np.log(np.exp(Z - m[:, None]).sum(axis=1))


def target_logits(Z: np.ndarray, y: np.ndarray) -> np.ndarray:
    """z[n, y[n]] for each row of the block."""
    return Z[np.arange(Z.shape[0]), y]


def dlogits(Z: np.ndarray, lse: np.ndarray, y: np.ndarray, w: float) -> np.ndarray:
    """G = (softmax(Z) - onehot(y)) * w for a block of valid rows."""
    P = np.exp(Z - lse[:, None])
    P[np.arange(Z.shape[0]), y] -= 1.0
    return P * w


# --------------------------------------------------------------------------
# compaction
# --------------------------------------------------------------------------

def compact_valid(labels: np.ndarray, ignore_index: int, V: int):
    """Ascending index of valid rows.

    Returns (valid_idx int32[N_valid], N_valid, bad_rows).  ``bad_rows`` lists
    rows whose label is neither ignore_index nor inside [0, V); they are not
    in valid_idx.
    """
    labels = np.asarray(labels, dtype=np.int64)
    keep = valid_mask(labels, ignore_index)
    in_range = (labels >= 0) & (labels < V)
    bad = np.flatnonzero(keep & ~in_range)
    idx = np.flatnonzero(keep & in_range).astype(np.int32)
    return idx, int(idx.size), bad


def _checked_index(labels, ignore_index, V, bad_labels):
    idx, n_valid, bad = compact_valid(labels, ignore_index, V)
    if bad.size and bad_labels == "raise":
        raise ValueError(
            f"{bad.size} label(s) outside [0, {V}) that are not ignore_index "
            f"(first at row {int(bad[0])}: {int(np.asarray(labels)[bad[0]])})")
    return idx, n_valid


def _scale(reduction: str, grad: float, n_valid: int) -> float:
    if reduction == "mean":
        return grad / n_valid if n_valid else 0.0
    if reduction == "sum":
        return grad
    raise ValueError(f"reduction must be 'mean' or 'sum', got {reduction!r}")


# --------------------------------------------------------------------------
# forward / backward
# --------------------------------------------------------------------------

@dataclasses.dataclass
class ForwardResult:
    loss: np.ndarray       # float64 [N], 0 on ignored rows
    lse: np.ndarray        # float64 [N], 0 on ignored rows
    valid_idx: np.ndarray  # int32 [N_valid], ascending
    valid_count: int
    loss_sum: float
    loss_mean: float       # NaN when no row is valid (PyTorch's convention)


def forward(H, W, labels, ignore_index: int = -100, *, bad_labels: str = "raise",
            row_block: int = DEFAULT_ROW_BLOCK) -> ForwardResult:
    H = np.asarray(H)
    W = np.asarray(W)
    labels = np.asarray(labels, dtype=np.int64)
    N, V = H.shape[0], W.shape[0]
    idx, n_valid = _checked_index(labels, ignore_index, V, bad_labels)
    loss = np.zeros(N, dtype=np.float64)
    lse = np.zeros(N, dtype=np.float64)
    W64 = np.asarray(W, dtype=np.float64)
    for s in range(0, n_valid, row_block):
        rows = idx[s:s + row_block]
        Z = logits(H[rows], W64)
        l = logsumexp_rows(Z)
        lse[rows] = l
        loss[rows] = l - target_logits(Z, labels[rows])
    loss_sum = float(loss[idx].sum()) if n_valid else 0.0
    mean = loss_sum / n_valid if n_valid else float("nan")
    return ForwardResult(loss, lse, idx, n_valid, loss_sum, mean)


def backward(H, W, labels, ignore_index: int = -100, *, grad: float = 1.0,
             reduction: str = "mean", bad_labels: str = "raise",
             row_block: int = DEFAULT_ROW_BLOCK):
    """(dH float64 [N, d], dW float64 [V, d]) of the reduced loss."""
    H = np.asarray(H)
    W = np.asarray(W)
    labels = np.asarray(labels, dtype=np.int64)
    N, d = H.shape
    V = W.shape[0]
    idx, n_valid = _checked_index(labels, ignore_index, V, bad_labels)
    w = _scale(reduction, grad, n_valid)
    W64 = np.asarray(W, dtype=np.float64)
    dH = np.zeros((N, d), dtype=np.float64)
    dW = np.zeros((V, d), dtype=np.float64)
    for s in range(0, n_valid, row_block):
        rows = idx[s:s + row_block]
        Hb = np.asarray(H[rows], dtype=np.float64)
        Z = logits(Hb, W64)
        G = dlogits(Z, logsumexp_rows(Z), labels[rows], w)
        dH[rows] = G @ W64
        dW += G.T @ Hb
    return dH, dW


# --------------------------------------------------------------------------
# per-row evaluation (for sampled checks at full size)
# --------------------------------------------------------------------------

def rows_forward(H, W, labels, rows):
    """(lse, loss, z_target) float64 for the given rows, assumed valid."""
    rows = np.asarray(rows)
    labels = np.asarray(labels, dtype=np.int64)
    Z = logits(np.asarray(H)[rows], W)
    l = logsumexp_rows(Z)
    zt = target_logits(Z, labels[rows])
    return l, l - zt, zt


def rows_dH(H, W, labels, rows, w: float):
    """dH rows for valid ``rows`` given the per-row scale w."""
    rows = np.asarray(rows)
    labels = np.asarray(labels, dtype=np.int64)
    W64 = np.asarray(W, dtype=np.float64)
    Z = logits(np.asarray(H)[rows], W64)
    G = dlogits(Z, logsumexp_rows(Z), labels[rows], w)
    return G @ W64


def rows_dW(H, W, labels, valid_idx, lse_valid, vocab_rows, w: float,
            row_block: int = 4096):
    """dW[vocab_rows] given lse of every valid row (ordered as valid_idx)."""
    vocab_rows = np.asarray(vocab_rows)
    labels = np.asarray(labels, dtype=np.int64)
    Wv = np.asarray(W, dtype=np.float64)[vocab_rows]
    out = np.zeros((vocab_rows.size, np.asarray(H).shape[1]), dtype=np.float64)
    for s in range(0, len(valid_idx), row_block):
        rows = valid_idx[s:s + row_block]
        Hb = np.asarray(np.asarray(H)[rows], dtype=np.float64)
        Z = Hb @ Wv.T                        # [rows, |vocab_rows|]
        P = np.exp(Z - np.asarray(lse_valid[s:s + row_block])[:, None])
        onehot = labels[rows][:, None] == vocab_rows[None, :]
        G = (P - onehot) * w
        out += G.T @ Hb
    return out


# --------------------------------------------------------------------------
# vocabulary shards
# --------------------------------------------------------------------------
#
# The vocabulary [0, V_total) cut into contiguous slices, each with its own
# rows of W (MaximusLLM page, section 2.1: the table split into contiguous
# sub-tables).  A shard's share of the online-softmax state (OjasX page, Online
# Softmax paragraph) is, per valid row,
#
#     m = max_{v in shard} z[n, v]
#     s = sum_{v in shard} exp(z[n, v] - m)
#     t = z[n, y[n]] if y[n] lies in the shard, else -inf
#
# and the shards combine with the same rescale step the recurrence uses:
#
#     M = max_k m_k,  S = sum_k s_k exp(m_k - M),  lse = M + log S,
#     loss = lse - (the one finite t_k).


@dataclasses.dataclass
class ShardPartials:
    part_max: np.ndarray     # float64 [N], 0 on ignored rows
    part_sum: np.ndarray     # float64 [N], 0 on ignored rows
    part_target: np.ndarray  # float64 [N], -inf off the shard and on ignored rows


def shard_partials(H, W_shard, labels, v_begin: int, V_total: int, ignore_index: int = -100,
                   *, bad_labels: str = "raise",
                   row_block: int = DEFAULT_ROW_BLOCK) -> ShardPartials:
    """(m, s, t) of the vocabulary slice [v_begin, v_begin + len(W_shard))."""
    H = np.asarray(H)
    labels = np.asarray(labels, dtype=np.int64)
    N = H.shape[0]
    Vs = np.asarray(W_shard).shape[0]
    idx, n_valid = _checked_index(labels, ignore_index, V_total, bad_labels)
    W64 = np.asarray(W_shard, dtype=np.float64)
    m = np.zeros(N)
    s = np.zeros(N)
    t = np.full(N, -np.inf)
    for b in range(0, n_valid, row_block):
        rows = idx[b:b + row_block]
        Z = logits(H[rows], W64)
        mb = Z.max(axis=1)
        m[rows] = mb
        s[rows] = np.exp(Z - mb[:, None]).sum(axis=1)
        yl = labels[rows] - v_begin
        inside = np.flatnonzero((yl >= 0) & (yl < Vs))
        t[rows[inside]] = Z[inside, yl[inside]]
    return ShardPartials(m, s, t)


def merge_partials(parts, valid_idx):
    """(loss, lse, loss_sum, loss_mean) from the partials of shards that
    cover the vocabulary exactly once."""
    valid_idx = np.asarray(valid_idx)
    N = parts[0].part_max.shape[0]
    loss = np.zeros(N)
    lse = np.zeros(N)
    if valid_idx.size:
        Mk = np.stack([p.part_max[valid_idx] for p in parts])
        Sk = np.stack([p.part_sum[valid_idx] for p in parts])
        Tk = np.stack([p.part_target[valid_idx] for p in parts])
        M = Mk.max(axis=0)
        S = (Sk * np.exp(Mk - M[None, :])).sum(axis=0)
        lse[valid_idx] = M + np.log(S)
        loss[valid_idx] = lse[valid_idx] - Tk.max(axis=0)
    loss_sum = float(loss[valid_idx].sum()) if valid_idx.size else 0.0
    mean = loss_sum / valid_idx.size if valid_idx.size else float("nan")
    return loss, lse, loss_sum, mean


def shard_backward(H, W_shard, labels, lse, v_begin: int, V_total: int,
                   ignore_index: int = -100, *, grad: float = 1.0, reduction: str = "mean",
                   bad_labels: str = "raise", row_block: int = DEFAULT_ROW_BLOCK):
    """(dH share float64 [N, d], dW_shard float64 [V_shard, d]) for the
    shard's columns of G, given the global lse of every row."""
    H = np.asarray(H)
    labels = np.asarray(labels, dtype=np.int64)
    N, d = H.shape
    Vs = np.asarray(W_shard).shape[0]
    idx, n_valid = _checked_index(labels, ignore_index, V_total, bad_labels)
    w = _scale(reduction, grad, n_valid)
    W64 = np.asarray(W_shard, dtype=np.float64)
    lse = np.asarray(lse, dtype=np.float64)
    dH = np.zeros((N, d))
    dW = np.zeros((Vs, d))
    for b in range(0, n_valid, row_block):
        rows = idx[b:b + row_block]
        Hb = np.asarray(H[rows], dtype=np.float64)
        Z = logits(Hb, W64)
        G = np.exp(Z - lse[rows][:, None])
        yl = labels[rows] - v_begin
        inside = np.flatnonzero((yl >= 0) & (yl < Vs))
        G[inside, yl[inside]] -= 1.0
        G *= w
        dH[rows] = G @ W64
        dW += G.T @ Hb
    return dH, dW


# --------------------------------------------------------------------------
# tied table: input side
# --------------------------------------------------------------------------
#
# The same table W read as the input embedding.  Positions whose id is the
# padding id are not looked up and get a zero vector (MaximusLLM page,
# section 2.3); the gradient of the lookup sends each valid row of dX back to
# the table row it came from.


def embed_forward(W, input_ids, pad_id: int):
    """(X float64 [N, d], valid_idx int32): X[n] = W[id[n]] for valid n, else 0."""
    W = np.asarray(W, dtype=np.float64)
    ids = np.asarray(input_ids, dtype=np.int64)
    idx, _, bad = compact_valid(ids, pad_id, W.shape[0])
    if bad.size:
        raise ValueError(f"{bad.size} input id(s) outside [0, {W.shape[0]})")
    X = np.zeros((ids.shape[0], W.shape[1]))
    X[idx] = W[ids[idx]]
    return X, idx


def embed_backward(dX, input_ids, pad_id: int, V: int):
    """dW float64 [V, d]: dW[v] = sum of dX[n] over valid n with id[n] = v."""
    dX = np.asarray(dX, dtype=np.float64)
    ids = np.asarray(input_ids, dtype=np.int64)
    idx, _, bad = compact_valid(ids, pad_id, V)
    if bad.size:
        raise ValueError(f"{bad.size} input id(s) outside [0, {V})")
    dW = np.zeros((V, dX.shape[1]))
    for n in idx:
        dW[ids[n]] += dX[n]
    return dW


# --------------------------------------------------------------------------
# optimizer step applied to the weight gradient
# --------------------------------------------------------------------------
#
# The update that consumes dW inside the backward pass instead of keeping a
# gradient buffer (OjasX page, core technology: no persistent .grad).  The
# formulas are PyTorch's: SGD without momentum, p -= lr (g + wd p); AdamW
# with decoupled weight decay and bias correction.


def optimizer_step(p, g, kind: str, lr: float, weight_decay: float = 0.0, beta1: float = 0.9,
                   beta2: float = 0.999, eps: float = 1e-8, step: int = 1, exp_avg=None,
                   exp_avg_sq=None):
    """(p_new, exp_avg_new, exp_avg_sq_new) in float64 (states None for SGD)."""
    p = np.asarray(p, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    if kind == "sgd":
        return p - lr * (g + weight_decay * p), None, None
    if kind != "adamw":
        raise ValueError(f"kind must be 'sgd' or 'adamw', got {kind!r}")
    m = np.asarray(exp_avg, dtype=np.float64)
    v = np.asarray(exp_avg_sq, dtype=np.float64)
    p = p * (1.0 - lr * weight_decay)
    m = beta1 * m + (1.0 - beta1) * g
    v = beta2 * v + (1.0 - beta2) * g * g
    bc1 = 1.0 - beta1 ** step
    bc2 = 1.0 - beta2 ** step
    p = p - (lr / bc1) * m / (np.sqrt(v) / np.sqrt(bc2) + eps)
    return p, m, v


# --------------------------------------------------------------------------
# output cast
# --------------------------------------------------------------------------
#
# The gradients come out of the backward pass in float32; a bfloat16
# parameter takes them rounded to the nearest bfloat16 value, a tie going to
# the neighbour whose last mantissa bit is 0 (IEEE round to nearest, ties to
# even).  A bfloat16 value is a float32 whose low 16 bits are zero (sign, 8
# exponent bits, 7 mantissa bits).  Below, the two bfloat16 neighbours of x
# are found from its bit pattern and the nearer one is picked by comparing
# the two distances exactly in float64.


def round_to_bf16(x) -> np.ndarray:
    """float32 array of x rounded to the nearest bfloat16 (ties to even).

    NaN stays NaN; values that are already bfloat16 (0, inf included) are
    unchanged; a magnitude at or past the midpoint between the largest
    bfloat16 and 2^128 becomes inf."""
    x = np.asarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    down = u & 0xFFFF0000                    # same sign, magnitude truncated
    up = down + 0x10000                      # next bfloat16 away from zero
    E = ((u >> 23) & 0xFF).astype(np.int64)  # exponent field of x
    spacing = np.ldexp(1.0, np.maximum(E, 1) - 134)   # bfloat16 step at x
    ax = np.abs(x.astype(np.float64))
    lo = np.abs(down.astype(np.uint32).view(np.float32).astype(np.float64))
    hi = lo + spacing
    with np.errstate(invalid="ignore"):
        d_lo = ax - lo
        d_hi = hi - ax
    odd = ((down >> 16) & 1) == 1
    take_up = (d_hi < d_lo) | ((d_hi == d_lo) & odd)
    out = np.where(take_up, up, down).astype(np.uint32)
    exact = (u & 0xFFFF) == 0
    out = np.where(exact, u.astype(np.uint32), out)
    res = out.view(np.float32).copy()
    res[np.isnan(x)] = np.nan
    return res.reshape(x.shape)


# --------------------------------------------------------------------------
# attention through an online softmax
# --------------------------------------------------------------------------
#
# "OjasX 0.6.1", section 核心技术 / "Core Technology": the [B, H, S, S] attention
# score matrix is never stored; score tiles stream through registers and
# on-chip memory, and the running max / normaliser recurrence (the page's
# Online Softmax paragraph) gives exactly the full-softmax result.  The
# operation itself is stated on the KV-cache page (KV Cache基础):
# Attention(Q, K, V) = softmax(Q K^T / sqrt(d_k)) V.  Reading taken here: the
# causal mask of a decoder (a query attends to keys at its own position and
# before) as an option, scale 1 / sqrt(d) by default.  The oracle is the
# definition: full scores, full softmax, one matrix product.


@dataclasses.dataclass
class AttentionResult:
    O: np.ndarray     # [B, H, S, D] float64
    lse: np.ndarray   # [B, H, S] natural-log sum of exp of the (masked, scaled) scores


def attention_scores(Q, K, scale: float) -> np.ndarray:
    """scale * Q K^T over the last two axes, float64."""
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    return (Q @ np.swapaxes(K, -1, -2)) * scale


def causal_allowed(S: int) -> np.ndarray:
    """[S, S] boolean: key k may be attended by query q iff k <= q."""
    q = np.arange(S)[:, None]
    k = np.arange(S)[None, :]
    return k <= q


def attention_forward(Q, K, V, causal: bool = False, scale: Optional[float] = None):
    """O = softmax(scale Q K^T [masked]) V and the per-row logsumexp."""
    Q = np.asarray(Q, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    S, D = Q.shape[-2], Q.shape[-1]
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    Z = attention_scores(Q, K, scale)
    if causal:
        Z = np.where(causal_allowed(S), Z, -np.inf)
    lead = Z.shape[:-1]
    lse = logsumexp_rows(Z.reshape(-1, Z.shape[-1])).reshape(lead)
    P = np.exp(Z - lse[..., None])
    return AttentionResult(O=P @ V, lse=lse)


@dataclasses.dataclass
class AttentionGrads:
    dQ: np.ndarray
    dK: np.ndarray
    dV: np.ndarray


def attention_row_dot(dO, O) -> np.ndarray:
    """D[q] = sum_d dO[q, d] O[q, d]: the softmax Jacobian's rank-one term,
    equal to sum_k P[q, k] dP[q, k]."""
    return (np.asarray(dO, dtype=np.float64) * np.asarray(O, dtype=np.float64)).sum(-1)


def attention_backward(Q, K, V, dO, causal: bool = False, scale: Optional[float] = None):
    """Exact gradient of O = softmax(scale Q K^T [masked]) V for an upstream dO:
    dV = P^T dO,  dP = dO V^T,  dS = P * (dP - D),  dQ = scale dS K,
    dK = scale dS^T Q, with P recomputed from the scores and the lse (the
    probabilities are never kept from the forward pass)."""
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    dO = np.asarray(dO, dtype=np.float64)
    S, D = Q.shape[-2], Q.shape[-1]
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    fwd = attention_forward(Q, K, V, causal, scale)
    Z = attention_scores(Q, K, scale)
    if causal:
        Z = np.where(causal_allowed(S), Z, -np.inf)
    P = np.exp(Z - fwd.lse[..., None])
    dV = np.swapaxes(P, -1, -2) @ dO
    dP = dO @ np.swapaxes(V, -1, -2)
    dS = P * (dP - attention_row_dot(dO, fwd.O)[..., None])
    return AttentionGrads(dQ=scale * (dS @ K), dK=scale * (np.swapaxes(dS, -1, -2) @ Q), dV=dV)
