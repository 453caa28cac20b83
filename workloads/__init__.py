"""Seeded synthetic inputs for the fused linear + cross-entropy path.

This module is shared by the GPU tests, the benchmark and the CPU oracle's
tests.  It draws random numbers and rounds them to the input precision; it
holds none of the method's arithmetic (no logits, no softmax, no gradients).

Workload shapes stand in for the pages' workloads:

* the tiny fp32 case is a unit-test shape;
* the 4K-context, d=2048 tied-embedding head follows the pretraining run
  configuration of "6GB显卡预训练11亿参数模型" (section 使用的预训练配置, 1.11B
  run: --d-model 2048, --seq-len 4096, --tie-embeddings, --chunked-loss 512);
* the 260K-vocab, batch 8 x 2048, mean valid length 850 case follows the
  MaximusLLM page, section 1 (26万词表, batch_size=8, seq_len=2048, longest
  sentence 2048, mean length 850, ~60% padding);
* the d=4096, V=128256 cases are a Llama-3-8B-shaped output head.

No dataset is read: labels are drawn from a truncated Zipf law (token
frequencies in text are Zipf-like) and hidden states / weights are Gaussian.

Generator conventions (fixed so that every consumer sees identical bytes):
``rng = numpy.random.default_rng(1000 + config_id)``; draw order W, H,
labels, ignore structure; normals drawn as float32 and rounded to bf16 with
round-to-nearest-even (kept in fp32 for the fp32 case); Zipf labels via
``searchsorted(cdf, u, side="right")`` with ``p_k ∝ k^-s`` for ranks
k = 1..V mapped to label k-1.
"""
from __future__ import annotations

import dataclasses
import hashlib
from typing import Optional, Tuple

import numpy as np

IGNORE_INDEX = -100


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic configuration.

    ``ignore`` is one of:
      ("count", k)      -- exactly k rows chosen uniformly without replacement
      ("seqlen", B, lo, hi) -- B sequences of N/B positions, valid length
                           drawn uniformly in [lo, hi], the rest padded
      ("lengths", (L0, L1, ...)) -- fixed valid lengths per sequence
      ("none",)         -- no ignored rows
    ``labels`` is ("uniform",) or ("zipf", s).
    """

    cid: int
    name: str
    N: int
    d: int
    V: int
    dtype: str  # "f32" or "bf16"
    w_std: float
    h_std: float
    labels: tuple
    ignore: tuple

    @property
    def seed(self) -> int:
        return 1000 + self.cid


CONFIGS = {
    1: Workload(1, "tiny_fp32", 64, 128, 1024, "f32", 0.02, 0.02,
                ("uniform",), ("count", 6)),
    2: Workload(2, "small_head_tied_4k", 4096, 2048, 32000, "bf16", 0.02, 1.0,
                ("zipf", 1.1), ("none",)),
    3: Workload(3, "llama3_8b_head_b4x2048", 8192, 4096, 128256, "bf16", 0.02, 1.0,
                ("zipf", 1.1), ("seqlen", 4, 512, 2048)),
    4: Workload(4, "vocab260k_b8x2048", 16384, 4096, 260000, "bf16", 0.02, 1.0,
                ("zipf", 1.05), ("lengths", (2048, 679, 679, 679, 679, 679, 679, 678))),
    5: Workload(5, "long_context_64k", 65536, 4096, 128256, "bf16", 0.02, 1.0,
                ("zipf", 1.1), ("count", 3277)),
}


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even).

    Returned as float32 whose low 16 mantissa bits are zero, so converting
    the result to bfloat16 anywhere is exact.  Inputs are finite.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    out = np.empty_like(u)
    # process in slabs to bound temporary memory on multi-GB arrays
    step = 1 << 26
    flat_u = u.reshape(-1)
    flat_o = out.reshape(-1)
    for s in range(0, flat_u.size, step):
        b = flat_u[s:s + step]
        lsb = (b >> np.uint32(16)) & np.uint32(1)
        r = (b + np.uint32(0x7FFF) + lsb) & np.uint32(0xFFFF0000)
        flat_o[s:s + step] = r
    return out.view(np.float32)


def _normals(rng: np.random.Generator, shape, std: float, dtype: str) -> np.ndarray:
    a = rng.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    if dtype == "bf16":
        a = bf16_round(a)
    return a


def zipf_labels(rng: np.random.Generator, N: int, V: int, s: float) -> np.ndarray:
    k = np.arange(1, V + 1, dtype=np.float64)
    p = np.power(k, -s)
    cdf = np.cumsum(p)
    cdf /= cdf[-1]
    u = rng.random(N)
    lab = np.searchsorted(cdf, u, side="right")
    return np.minimum(lab, V - 1).astype(np.int64)


def _apply_ignore(rng: np.random.Generator, labels: np.ndarray, spec: tuple) -> None:
    N = labels.shape[0]
    kind = spec[0]
    if kind == "none":
        return
    if kind == "count":
        k = spec[1]
        rows = rng.choice(N, k, replace=False)
        labels[rows] = IGNORE_INDEX
        return
    if kind == "seqlen":
        B, lo, hi = spec[1], spec[2], spec[3]
        S = N // B
        for b in range(B):
            L = int(rng.integers(lo, hi, endpoint=True))
            labels[b * S + L:(b + 1) * S] = IGNORE_INDEX
        return
    if kind == "lengths":
        lens = spec[1]
        S = N // len(lens)
        for b, L in enumerate(lens):
            labels[b * S + L:(b + 1) * S] = IGNORE_INDEX
        return
    raise ValueError(f"unknown ignore spec {spec!r}")


def generate(cfg, seed: Optional[int] = None):
    """Return (H, W, labels) for a configuration id or Workload.

    H is float32 [N, d] and W float32 [V, d]; for "bf16" workloads every
    value is exactly representable in bfloat16.  labels is int64 [N] with
    IGNORE_INDEX on ignored rows.
    """
    wl = CONFIGS[cfg] if isinstance(cfg, int) else cfg
    rng = np.random.default_rng(wl.seed if seed is None else seed)
    W = _normals(rng, (wl.V, wl.d), wl.w_std, wl.dtype)
    H = _normals(rng, (wl.N, wl.d), wl.h_std, wl.dtype)
    if wl.labels[0] == "uniform":
        labels = rng.integers(0, wl.V, wl.N).astype(np.int64)
    elif wl.labels[0] == "zipf":
        labels = zipf_labels(rng, wl.N, wl.V, wl.labels[1])
    else:
        raise ValueError(wl.labels)
    _apply_ignore(rng, labels, wl.ignore)
    return H, W, labels


def custom(N: int, d: int, V: int, dtype: str = "bf16", seed: int = 0,
           w_std: float = 0.02, h_std: float = 1.0, ignore_frac: float = 0.1,
           zipf_s: Optional[float] = 1.1) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Small seeded case for element-by-element parity tests."""
    k = int(round(ignore_frac * N))
    wl = Workload(0, "custom", N, d, V, dtype, w_std, h_std,
                  ("zipf", zipf_s) if zipf_s else ("uniform",),
                  ("count", k) if k > 0 else ("none",))
    return generate(wl, seed=seed)


def checksum(*arrays: np.ndarray) -> str:
    """sha256 over the raw bytes of the arrays (detects any generator drift)."""
    h = hashlib.sha256()
    for a in arrays:
        a = np.ascontiguousarray(a)
        h.update(str(a.dtype).encode())
        h.update(str(a.shape).encode())
        mv = memoryview(a.reshape(-1).view(np.uint8))
        step = 1 << 28
        for s in range(0, len(mv), step):
            h.update(mv[s:s + step])
    return h.hexdigest()


# --------------------------------------------------------------- attention
#
# Online-softmax attention inputs shaped like a Llama-3-8B attention layer
# at the MaximusLLM page's training batch (section 1 and its KV-cache
# figures: batch 8 x seq 2048, 32 heads, head_dim 128).  Q, K, V ~ N(0, 1)
# rounded to bf16, layout [B, H, S, D]; rng = default_rng(seed), draw order
# Q, K, V.  The decoder's causal mask is the default.


@dataclasses.dataclass(frozen=True)
class AttentionWorkload:
    name: str
    B: int
    H: int
    S: int
    D: int
    causal: bool
    seed: int


ATTENTION = AttentionWorkload("llama3_8b_attention_b8x2048", 8, 32, 2048, 128, True, 2001)


def attention_inputs(B: int, H: int, S: int, D: int, seed: int, std: float = 1.0):
    """(Q, K, V) as float32 arrays holding bf16-representable values."""
    rng = np.random.default_rng(seed)
    return tuple(_normals(rng, (B, H, S, D), std, "bf16") for _ in range(3))
