"""Fused linear + cross-entropy over large vocabularies for MI355X (gfx950).

The compute path is liblce.so (hand-written HIP kernels behind a C ABI,
include/lce.h); ``_lib`` binds it with ctypes under the same names, and
``torch_api`` offers ``linear_cross_entropy`` as an autograd function.
"""
import importlib

from . import _lib  # noqa: F401

__all__ = ["_lib", "torch_api", "linear_cross_entropy"]


def __getattr__(name):
    if name in ("torch_api", "linear_cross_entropy"):
        mod = importlib.import_module(__name__ + ".torch_api")
        return mod if name == "torch_api" else mod.linear_cross_entropy
    raise AttributeError(name)
