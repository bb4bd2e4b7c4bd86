"""Sparse decode attention over an int8-scored KV cache, for MI355X (gfx950).

The compute path is the HIP library libsd.so (C ABI: include/sd.h); the
``binding`` module wraps it with ctypes.  ``inputs`` generates the seeded
synthetic workloads.  Submodules load lazily so that ``inputs`` works without
the built library.
"""
import importlib

__all__ = ["binding", "inputs", "build"]


def __getattr__(name):
    if name in __all__:
        return importlib.import_module(f".{name}", __name__)
    raise AttributeError(name)
