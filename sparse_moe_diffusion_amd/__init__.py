"""DiT-MoE sparse MoE feed-forward layer on MI355X (gfx950).

The compute lives in libmoe.so (hand-written HIP kernels behind the C ABI of
include/moe.h); this package is its ctypes binding.  There is no CPU
fallback: the first call fails with ImportError if the library is missing.
"""
from . import _lib  # noqa: F401

__all__ = ["_lib", "ops", "layer"]


def __getattr__(name):
    if name in ("ops", "layer"):
        import importlib
        return importlib.import_module(f"{__name__}.{name}")
    raise AttributeError(name)
