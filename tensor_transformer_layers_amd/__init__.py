"""tensor_transformer_layers_amd -- one tensor-parallel rank's Transformer-block shard on MI355X.

The compute lives in ``lib/libtpshard.so`` (hand-written HIP kernels for gfx950 behind the C ABI
of ``include/tp_shard.h``). This package holds its ctypes binding (``binding``), the shard
extraction helpers (``layout``) and the PyTorch-facing calls (``shard``). Importing the package
does not load the library; the first call does, and raises if it has not been built.
"""
import importlib

from . import binding, layout  # noqa: F401

__all__ = ["binding", "layout", "shard"]


def __getattr__(name):
    if name == "shard":   # imported lazily: it needs torch
        return importlib.import_module(__name__ + ".shard")
    raise AttributeError(name)
