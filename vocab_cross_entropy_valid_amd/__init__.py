"""Fused linear + cross-entropy over large vocabularies for MI355X (gfx950).

The compute path is liblce.so (hand-written HIP kernels behind a C ABI,
include/lce.h); ``_lib`` binds it with ctypes under the same names, and
``torch_api`` offers ``linear_cross_entropy`` as an autograd function.
"""
from . import _lib  # noqa: F401

__all__ = ["_lib", "torch_api", "linear_cross_entropy"]


def __getattr__(name):
    if name in ("torch_api", "linear_cross_entropy"):
        from . import torch_api
        return torch_api if name == "torch_api" else torch_api.linear_cross_entropy
    raise AttributeError(name)
