"""C-ABI checks that need no GPU: the library loads, exports every function
include/lce.h declares, and rejects bad arguments before launching anything."""
import ctypes
import os
import re

import pytest

from vocab_cross_entropy_valid_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lce.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(lce_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = _declared_functions()
    for n in ("lce_forward", "lce_backward", "lce_workspace_bytes", "lce_status_string",
              "lce_check_error"):
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = _lib.load()
    for name in _declared_functions():
        assert hasattr(lib, name), name
    assert set(_declared_functions()) == set(_lib.SIGNATURES)


def test_status_strings():
    assert _lib.lce_status_string(0) == "ok"
    assert "label" in _lib.lce_status_string(_lib.LCE_ERR_LABEL_RANGE)
    assert _lib.lce_status_string(99) == "unknown status"


def test_workspace_bounded_independent_of_n_times_v():
    bf = _lib.LCE_BF16
    # configs 3 and 5 differ only in N: the backward block dominates, same bytes
    w3 = _lib.lce_workspace_bytes(8192, 4096, 128256, bf)
    w5 = _lib.lce_workspace_bytes(65536, 4096, 128256, bf)
    assert w3 == w5
    # the backward block is bounded by constants (token chunk C <= 8192,
    # vocabulary block Vs <= 16384, padded strides) and d, never by N or V:
    # G [C, Vs] and H^T [d, C] in bf16 (dH reads W itself, dW reads G K-major)
    C, Vs, pad, d = 8192, 16384, 64, 4096
    exact = 2 * (C * (Vs + pad) + d * (C + pad))
    assert w5 == exact
    # fp32 adds G^T [Vs, C] and the W^T block [d, Vs]
    wf = _lib.lce_workspace_bytes(65536, d, 128256, _lib.LCE_F32)
    assert wf == 4 * (C * (Vs + pad) + Vs * (C + pad) + d * (C + pad)) + 4 * d * (Vs + pad)
    # far below the [N, V] fp32 logits table it replaces
    assert w5 < 65536 * 128256 * 4 / 40
    # growing V past the vocabulary block does not grow the workspace
    assert _lib.lce_workspace_bytes(8192, 4096, 260000, bf) == w3
    # growing N only adds O(N) per-token vectors
    big = _lib.lce_workspace_bytes(1 << 22, 4096, 128256, bf)
    assert big - w5 < (1 << 22) * 64 * 3 * 4 + (1 << 22) * 4 + (1 << 20)
    assert _lib.lce_workspace_bytes(64, 128, 1024, _lib.LCE_F32) > 0


@pytest.mark.parametrize("N,d,V,dt,status", [
    (-1, 64, 10, 1, _lib.LCE_ERR_INVALID_ARG),
    (10, 0, 10, 1, _lib.LCE_ERR_INVALID_ARG),
    (10, 64, 0, 1, _lib.LCE_ERR_INVALID_ARG),
    (10, 64, 10, 7, _lib.LCE_ERR_INVALID_ARG),
    (10, 100, 10, 1, _lib.LCE_ERR_UNSUPPORTED),
    (10, 64, 1 << 31, 1, _lib.LCE_ERR_UNSUPPORTED),
    (1, 1 << 22, 10, 1, _lib.LCE_ERR_UNSUPPORTED),     # fp32 block rows need 32-bit offsets
    (1 << 20, 4096, 10, 1, _lib.LCE_ERR_UNSUPPORTED),  # N * d * 2 bytes reach 4 GiB
])
def test_forward_rejects_bad_sizes_before_launch(N, d, V, dt, status):
    lib = _lib.load()
    fake = ctypes.c_void_p(0x1000)
    r = lib.lce_forward(fake, fake, fake, -100, N, d, V, dt, fake, fake, fake, fake, fake,
                        None, fake, fake, 1 << 40, None)
    assert r == status
    assert _lib.lce_last_error() != ""
    assert _lib.lce_workspace_bytes(N, d, V, dt) == 0


def test_forward_rejects_null_and_small_workspace():
    lib = _lib.load()
    fake = ctypes.c_void_p(0x1000)
    r = lib.lce_forward(None, fake, fake, -100, 10, 64, 10, 1, fake, fake, fake, fake, fake,
                        None, fake, fake, 1 << 40, None)
    assert r == _lib.LCE_ERR_INVALID_ARG
    need = _lib.lce_workspace_bytes(10, 64, 10, 1)
    r = lib.lce_forward(fake, fake, fake, -100, 10, 64, 10, 1, fake, fake, fake, fake, fake,
                        None, fake, fake, need - 1, None)
    assert r == _lib.LCE_ERR_WORKSPACE
    r = lib.lce_forward(fake, fake, fake, -100, 10, 64, 10, 1, fake, fake, fake, fake, fake,
                        None, fake, ctypes.c_void_p(0x1010), need, None)
    assert r == _lib.LCE_ERR_INVALID_ARG  # misaligned workspace


def test_backward_rejects_bad_reduction_and_nulls():
    lib = _lib.load()
    fake = ctypes.c_void_p(0x1000)
    args = [fake, fake, fake, -100, fake, fake, fake, 10, 64, 10, 1, fake, 5, fake, fake, 0,
            fake, 1 << 40, None]
    assert lib.lce_backward(*args) == _lib.LCE_ERR_INVALID_ARG
    args[12] = 0
    args[11] = None  # grad_out
    assert lib.lce_backward(*args) == _lib.LCE_ERR_INVALID_ARG
    args[11] = fake
    args[16] = fake
    args[17] = 16
    assert lib.lce_backward(*args) == _lib.LCE_ERR_WORKSPACE
    args[14] = ctypes.c_void_p(0x1004)  # dW is stored as 16-byte vectors
    assert lib.lce_backward(*args) == _lib.LCE_ERR_INVALID_ARG


def test_gemm_and_timing_argument_checks():
    lib = _lib.load()
    fake = ctypes.c_void_p(0x1000)
    assert lib.lce_gemm_nt(fake, fake, fake, 10, 10, 100, 1, None) == _lib.LCE_ERR_UNSUPPORTED
    assert lib.lce_gemm_nt(fake, fake, fake, 0, 10, 64, 1, None) == _lib.LCE_ERR_INVALID_ARG
    assert lib.lce_check_error(None, None) == _lib.LCE_ERR_INVALID_ARG
    ms = ctypes.c_double()
    n = ctypes.c_int64()
    assert lib.lce_timing_query(99, ctypes.byref(ms), ctypes.byref(n)) == _lib.LCE_ERR_INVALID_ARG
    assert lib.lce_timing_reset() == 0
    assert lib.lce_timing_query(0, ctypes.byref(ms), ctypes.byref(n)) == 0 and n.value == 0


def test_missing_library_fails_loudly(tmp_path):
    with pytest.raises(RuntimeError, match="not found"):
        _lib.load(str(tmp_path / "nope.so"))


@pytest.mark.parametrize("V_total,v_begin,V_shard", [
    (100, -1, 10), (100, 95, 10), (100, 0, 0), (0, 0, 10), (1 << 31, 0, 10),
])
def test_shard_entry_points_reject_bad_ranges_before_launch(V_total, v_begin, V_shard):
    lib = _lib.load()
    fake = ctypes.c_void_p(0x1000)
    r = lib.lce_forward_shard(fake, fake, fake, -100, 10, 64, V_total, v_begin, V_shard, 1,
                              fake, fake, fake, fake, fake, fake, fake, 1 << 40, None)
    assert r == _lib.LCE_ERR_INVALID_ARG, r
    r = lib.lce_backward_shard(fake, fake, fake, -100, fake, fake, fake, 10, 64, V_total,
                               v_begin, V_shard, 1, fake, 0, fake, 0, fake, 0, fake, 1 << 40,
                               None)
    assert r == _lib.LCE_ERR_INVALID_ARG, r


def test_shard_workspace_and_merge_argument_checks():
    lib = _lib.load()
    fake = ctypes.c_void_p(0x1000)
    need = _lib.lce_workspace_bytes(10, 64, 30, 1)
    r = lib.lce_forward_shard(fake, fake, fake, -100, 10, 64, 100, 40, 30, 1, fake, fake, fake,
                              fake, fake, fake, fake, need - 1, None)
    assert r == _lib.LCE_ERR_WORKSPACE
    r = lib.lce_backward_shard(fake, fake, fake, -100, fake, fake, fake, 10, 64, 100, 40, 30, 1,
                               fake, 0, fake, 0, ctypes.c_void_p(0x1008), 0, fake, 1 << 40, None)
    assert r == _lib.LCE_ERR_INVALID_ARG  # misaligned dW_shard
    # no shards, a stride shorter than N, missing outputs
    assert lib.lce_lse_merge(fake, fake, fake, 0, 10, 10, fake, fake, fake, fake, fake, None,
                             None) == _lib.LCE_ERR_INVALID_ARG
    assert lib.lce_lse_merge(fake, fake, fake, 2, 9, 10, fake, fake, fake, fake, fake, None,
                             None) == _lib.LCE_ERR_INVALID_ARG
    assert lib.lce_lse_merge(fake, fake, fake, 2, 10, 10, fake, fake, None, fake, fake, None,
                             None) == _lib.LCE_ERR_INVALID_ARG


def test_backward_step_argument_checks_before_launch():
    lib = _lib.load()
    fake = ctypes.c_void_p(0x1000)

    def call(N=10, dtype=1, master=fake, m=fake, v=fake, **kw):
        o = _lib.LceOptimizer(kind=kw.get("kind", _lib.LCE_OPT_ADAMW), lr=kw.get("lr", 1e-3),
                              weight_decay=0.0, beta1=kw.get("beta1", 0.9), beta2=0.999,
                              eps=kw.get("eps", 1e-8), step=kw.get("step", 1))
        return lib.lce_backward_step(fake, fake, fake, -100, fake, fake, fake, N, 64, 100, dtype,
                                     fake, 0, fake, master, m, v, ctypes.byref(o), fake, 1 << 40,
                                     None)
    assert call(master=None) == _lib.LCE_ERR_INVALID_ARG   # bf16 without master weights
    assert call(kind=7) == _lib.LCE_ERR_INVALID_ARG
    assert call(step=0) == _lib.LCE_ERR_INVALID_ARG
    assert call(beta1=1.0) == _lib.LCE_ERR_INVALID_ARG
    assert call(eps=0.0) == _lib.LCE_ERR_INVALID_ARG
    assert call(lr=-1.0) == _lib.LCE_ERR_INVALID_ARG
    assert call(m=None) == _lib.LCE_ERR_INVALID_ARG
    # any N: several token chunks need the larger step workspace
    need = _lib.lce_step_workspace_bytes(20000, 64, 100, 1)
    o = _lib.LceOptimizer(kind=_lib.LCE_OPT_SGD, lr=1e-3, weight_decay=0.0, beta1=0.9,
                          beta2=0.999, eps=1e-8, step=1)
    r = lib.lce_backward_step(fake, fake, fake, -100, fake, fake, fake, 20000, 64, 100, 1, fake,
                              0, fake, fake, None, None, ctypes.byref(o), fake, need - 1, None)
    assert r == _lib.LCE_ERR_WORKSPACE


def test_step_workspace_is_bounded():
    """The fused step adds the transposed W block and either G^T (one token
    chunk: the optimizer epilogue reads it) or the fp32 dW block accumulator
    (several chunks): bounded by constants and d, not by N or V."""
    bf = _lib.LCE_BF16
    d, Vs, C, pad = 4096, 16384, 8192, 64
    plain3 = _lib.lce_workspace_bytes(8192, d, 128256, bf)
    step3 = _lib.lce_step_workspace_bytes(8192, d, 128256, bf)
    assert step3 - plain3 == 2 * d * (Vs + pad) + 2 * Vs * (C + pad)   # W^T and G^T blocks
    step4 = _lib.lce_step_workspace_bytes(16384, d, 260000, bf)
    step5 = _lib.lce_step_workspace_bytes(65536, d, 128256, bf)
    assert step4 == step5 == plain3 + 2 * d * (Vs + pad) + 4 * Vs * d  # W^T + fp32 dW accumulator
    assert _lib.lce_step_workspace_bytes(1 << 20, d, 128256, bf) - step5 < (1 << 20) * 64 * 13
    assert _lib.lce_step_workspace_bytes(10, 100, 10, bf) == 0


def test_attention_argument_checks_before_launch():
    lib = _lib.load()
    fake = ctypes.c_void_p(0x1000)

    def call(B=1, H=2, S=100, D=128, causal=1, scale=0.0, q=fake, o=fake):
        return lib.lce_attention_forward(q, fake, fake, B, H, S, D, causal, scale, o, fake, None)

    assert call(D=96) == _lib.LCE_ERR_UNSUPPORTED
    assert call(D=256) == _lib.LCE_ERR_UNSUPPORTED
    assert call(S=-1) == _lib.LCE_ERR_INVALID_ARG
    assert call(B=-2) == _lib.LCE_ERR_INVALID_ARG
    assert call(causal=2) == _lib.LCE_ERR_INVALID_ARG
    assert call(scale=-0.5) == _lib.LCE_ERR_INVALID_ARG
    assert call(scale=float("nan")) == _lib.LCE_ERR_INVALID_ARG
    assert call(scale=float("inf")) == _lib.LCE_ERR_INVALID_ARG
    assert call(q=None) == _lib.LCE_ERR_INVALID_ARG
    assert call(o=None) == _lib.LCE_ERR_INVALID_ARG
    assert call(S=1 << 31) == _lib.LCE_ERR_UNSUPPORTED
    # empty problems launch nothing, so NULL pointers are fine
    assert lib.lce_attention_forward(None, None, None, 1, 2, 0, 128, 1, 0.0, None, None, None) == 0
    assert lib.lce_attention_forward(None, None, None, 0, 2, 64, 64, 0, 0.0, None, None, None) == 0


def test_attention_backward_argument_checks_before_launch():
    lib = _lib.load()
    f = ctypes.c_void_p(0x1000)

    def call(B=1, H=2, S=100, D=128, causal=1, scale=0.0, dq=f, delta=f):
        return lib.lce_attention_backward(f, f, f, f, f, f, B, H, S, D, causal, scale, dq, f, f,
                                          delta, None)

    assert call(D=80) == _lib.LCE_ERR_UNSUPPORTED
    assert call(S=-3) == _lib.LCE_ERR_INVALID_ARG
    assert call(causal=-1) == _lib.LCE_ERR_INVALID_ARG
    assert call(scale=-1.0) == _lib.LCE_ERR_INVALID_ARG
    assert call(dq=None) == _lib.LCE_ERR_INVALID_ARG
    assert call(delta=None) == _lib.LCE_ERR_INVALID_ARG
    assert call(S=0, dq=None, delta=None) == 0


def test_forward_noalloc_rejects_sizes_beyond_its_static_scratch():
    """lce_forward_noalloc keeps the forward's partials in a 16 MiB static
    device array: (3 J + 1) * round_up(N, 256) * 4 bytes with J <= 64
    vocabulary chunks, so every V fits up to N = 21504 and N = 21505 with 64
    chunks does not.  The check happens before anything is launched."""
    lib = _lib.load()
    fake = ctypes.c_void_p(0x1000)
    for N, V in ((21505, 260000), (65536, 128256)):
        r = lib.lce_forward_noalloc(fake, fake, fake, -100, N, 64, V, 1, fake, fake, fake, fake,
                                    fake, None, fake, None)
        assert r == _lib.LCE_ERR_UNSUPPORTED
        assert "static scratch" in _lib.lce_last_error()
    # the same argument checks as lce_forward
    assert lib.lce_forward_noalloc(fake, None, fake, -100, 10, 64, 10, 1, fake, fake, fake, fake,
                                   fake, None, fake, None) == _lib.LCE_ERR_INVALID_ARG
    assert lib.lce_forward_noalloc(fake, fake, fake, -100, 10, 100, 10, 1, fake, fake, fake, fake,
                                   fake, None, fake, None) == _lib.LCE_ERR_UNSUPPORTED


def test_mfma_peak_argument_checks():
    lib = _lib.load()
    fake = ctypes.c_void_p(0x1000)
    assert lib.lce_mfma_peak(None, 1 << 19, 10, None) == _lib.LCE_ERR_INVALID_ARG
    assert lib.lce_mfma_peak(fake, (1 << 19) - 1, 10, None) == _lib.LCE_ERR_INVALID_ARG
    assert lib.lce_mfma_peak(fake, 1 << 19, 0, None) == _lib.LCE_ERR_INVALID_ARG
    assert lib.lce_mfma_peak(fake, 1 << 19, (1 << 24) + 1, None) == _lib.LCE_ERR_INVALID_ARG


def test_embed_workspace_is_host_computable():
    """The input side's workspace is sized on the host (no device query): a
    positive size on a machine without a GPU, 0 only for unsupported sizes;
    O(N + N d / 32): keys, segment lists, sort histograms, chunk partials."""
    n3 = _lib.lce_embed_workspace_bytes(8192, 4096, 128256)
    n5 = _lib.lce_embed_workspace_bytes(65536, 4096, 128256)
    assert n3 > 0 and n5 > n3
    assert n5 < 65536 * 64 + 65536 * 4096 * 4 // 32 + (1 << 20)
    assert _lib.lce_embed_workspace_bytes(100, 100, 10) == 0      # d % 64 != 0
    assert _lib.lce_embed_workspace_bytes(-1, 64, 10) == 0
    assert _lib.lce_embed_workspace_bytes(0, 64, 300) > 0
