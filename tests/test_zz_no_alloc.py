"""lce_forward_noalloc (scratch in a static device array, no workspace
argument) against lce_forward (caller workspace): the same kernels on the
same inputs, so every output must agree bit for bit.  Two calls in a row, the
second smaller, so that the second runs on the scratch the first left
behind; then sizes beyond the static scratch are rejected before launch."""
import numpy as np
import pytest

import oracle
import workloads
from tests.gpu_helpers import announce, to_dev

pytestmark = pytest.mark.gpu


def _outs(N, dev):
    import torch
    return dict(loss=torch.full((N,), 7.0, device=dev), lse=torch.full((N,), 7.0, device=dev),
                valid_idx=torch.full((N,), -1, dtype=torch.int32, device=dev),
                valid_count=torch.full((1,), -1, dtype=torch.int32, device=dev),
                loss_sum=torch.full((1,), 7.0, dtype=torch.float64, device=dev),
                loss_mean=torch.full((1,), 7.0, device=dev),
                err_flag=torch.full((1,), 7, dtype=torch.int32, device=dev))


def _call(fn_name, Ht, Wt, yt, dt, o, ws=None):
    import torch
    from vocab_cross_entropy_valid_amd import _lib
    N, d = Ht.shape
    V = Wt.shape[0]
    s = torch.cuda.current_stream().cuda_stream
    args = [Ht.data_ptr(), Wt.data_ptr(), yt.data_ptr(), -100, N, d, V, dt, o["loss"].data_ptr(),
            o["lse"].data_ptr(), o["valid_idx"].data_ptr(), o["valid_count"].data_ptr(),
            o["loss_sum"].data_ptr(), o["loss_mean"].data_ptr(), o["err_flag"].data_ptr()]
    if fn_name == "lce_forward":
        args += [ws.data_ptr(), ws.numel()]
    getattr(_lib, fn_name)(*args, s)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_noalloc_forward_matches_workspace_forward(dtype):
    import torch
    from vocab_cross_entropy_valid_amd import _lib, torch_api
    dev = torch.device("cuda:0")
    dt = _lib.LCE_BF16 if dtype == "bf16" else _lib.LCE_F32
    # the second call is smaller and runs on the scratch the first left behind
    for N, d, V, seed in [(9000, 256, 40000, 61), (700, 128, 3001, 62)]:
        announce(f"noalloc forward {dtype} N={N} d={d} V={V}")
        H, W, y = workloads.custom(N, d, V, dtype=dtype, seed=seed, ignore_frac=0.2)
        Ht, Wt, yt = to_dev(H, W, y, dtype)
        ws = torch_api.alloc_workspace(N, d, V, Ht.dtype, dev)
        a, b = _outs(N, dev), _outs(N, dev)
        _call("lce_forward", Ht, Wt, yt, dt, a, ws)
        _call("lce_forward_noalloc", Ht, Wt, yt, dt, b)
        torch.cuda.synchronize()
        for k in a:
            assert torch.equal(a[k], b[k]), k
        # and both agree with the oracle (the forward's parity bar)
        ref = oracle.forward(H, W, y, -100)
        n = ref.valid_count
        assert int(b["valid_count"].item()) == n
        np.testing.assert_array_equal(b["valid_idx"][:n].cpu().numpy(), ref.valid_idx)
        tol = 1e-4 if dtype == "bf16" else 1e-5
        np.testing.assert_allclose(b["loss"].cpu().numpy(), ref.loss, rtol=0, atol=tol)


def test_noalloc_forward_rejects_sizes_beyond_the_scratch():
    import ctypes
    from vocab_cross_entropy_valid_amd import _lib
    lib = _lib.load()
    fake = ctypes.c_void_p(0x1000)
    # 65536 tokens x 64 vocabulary chunks of partials need ~50 MB > 16 MiB
    r = lib.lce_forward_noalloc(fake, fake, fake, -100, 65536, 4096, 128256, 1, fake, fake, fake,
                                fake, fake, None, fake, None)
    assert r == _lib.LCE_ERR_UNSUPPORTED
    assert "static scratch" in _lib.lce_last_error()
