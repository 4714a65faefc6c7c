"""Batched multi-adapter layer in normal form on AMD MI355X (gfx950).

The compute path is libtpa.so (C ABI in include/tpa.h, HIP kernels in
csrc/).  ``binding`` exposes the C functions under their own names;
``layer.AdaptedLayer`` wraps one projection with torch-owned memory;
``bytemodel`` predicts the bytes and launches of each kernel.
"""
from . import bytemodel  # noqa: F401  (pure Python, no GPU)

__all__ = ["bytemodel", "binding", "layer"]


def __getattr__(name):
    # The binding loads libtpa.so on first use and fails loudly if it is
    # missing; the byte model stays importable without it.
    if name in ("binding", "layer"):
        import importlib
        return importlib.import_module("." + name, __name__)
    raise AttributeError(name)
