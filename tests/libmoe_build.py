"""Locate libmoe.so for the tests, building it in-tree if it is absent."""
import os

from sparse_moe_diffusion_amd import _lib


def ensure_built():
    if not os.path.exists(_lib.LIB_PATH):
        from sparse_moe_diffusion_amd import build
        build.build()
    return _lib.load()
