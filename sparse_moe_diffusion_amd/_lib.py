"""ctypes loader of libmoe.so, the gfx950 library behind include/moe.h.

Raw entry points with the C names and C argument order (pointers as ints).
There is no fallback: if the library is missing or fails to load, importing
anything that needs it raises.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
# MOE_LIB_PATH names another build of the same library (the tests' host
# sanitizer build); there is no fallback either way.
LIB_PATH = os.environ.get("MOE_LIB_PATH") or os.path.join(_PKG, "libmoe.so")

MOE_OK = 0
MOE_ERR_INVALID_ARGUMENT = 1
MOE_ERR_UNSUPPORTED = 2
MOE_ERR_WORKSPACE_TOO_SMALL = 3
MOE_ERR_HIP = 4

MOE_F32 = 0
MOE_BF16 = 1
MOE_ROUTE_TOPK = 0
MOE_ROUTE_EXPERT_RACE = 1
MOE_BAL_PER_SEQUENCE = 0
MOE_BAL_GLOBAL = 1
MOE_FFN_UP = 1
MOE_FFN_DOWN = 2
MOE_FFN_BOTH = 3

# name -> (restype, argtypes); the order and types of include/moe.h
_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_SZ = ctypes.c_size_t
_F = ctypes.c_float
_E = ctypes.c_int  # C enums

SIGNATURES = {
    "moe_status_string": (ctypes.c_char_p, [_E]),
    "moe_last_error": (ctypes.c_char_p, []),
    "moe_gate_workspace_size": (_SZ, [_I64, _I32, _I32, _E]),
    "moe_gate_topk": (_E, [_P, _E, _P, _P, _I64, _I32, _I32, _I32, _E, _P, _P,
                           _P, _P, _SZ, _P]),
    "moe_permute_workspace_size": (_SZ, [_I64, _I32, _I32]),
    "moe_permute": (_E, [_P, _E, _P, _I64, _I32, _I32, _I32, _I32, _P, _P, _P,
                         _P, _P, _P, _SZ, _P]),
    "moe_permute_noalloc": (_E, [_P, _E, _P, _I64, _I32, _I32, _I32, _I32, _P,
                                 _P, _P, _P, _P, _P]),
    "moe_grouped_ffn": (_E, [_P, _P, _I64, _E, _I64, _P, _I32, _I32, _I32, _P,
                             _P, _P, _P, _P, _P, _P, _E, _E, _P]),
    "moe_grouped_ffn_split_workspace_size": (_SZ, []),
    "moe_grouped_ffn_split": (_E, [_P, _P, _I64, _E, _I64, _P, _I32, _I32,
                                   _I32, _P, _P, _P, _P, _P, _P, _P, _E, _E,
                                   _P, _SZ, _P]),
    "moe_grouped_mlp_fused": (_E, [_P, _P, _I64, _E, _I64, _P, _I32, _I32,
                                   _I32, _P, _P, _P, _P, _P, _E, _P]),
    "moe_combine": (_E, [_P, _E, _P, _P, _I64, _I32, _I32, _P, _E, _P, _E, _P]),
    "moe_balance_stats": (_E, [_P, _P, _I32, _I32, _I32, _I32, _I32, _F, _E, _P,
                               _P, _P, _P]),
    "moe_gate_balance_workspace_size": (_SZ, [_I32, _I32, _I32]),
    "moe_gate_topk_balance": (_E, [_P, _E, _P, _P, _I32, _I32, _I32, _I32, _I32,
                                   _F, _E, _P, _P, _P, _P, _P, _P, _P, _SZ,
                                   _P]),
    "moe_gate_route_workspace_size": (_SZ, [_I32, _I32, _I32]),
    "moe_gate_route": (_E, [_P, _E, _P, _P, _I32, _I32, _I32, _I32, _I32, _F,
                            _E, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                            _SZ, _P]),
    "moe_ffn_down_combine": (_E, [_P, _E, _I64, _I32, _I32, _P, _P, _P, _P, _P,
                                  _I32, _P, _P]),
    "moe_combine_backward": (_E, [_P, _E, _P, _E, _P, _P, _I64, _I32, _I32, _P,
                                  _P, _P]),
    "moe_ffn_backward_workspace_size": (_SZ, [_I64, _I32, _I32, _I32]),
    "moe_grouped_ffn_backward": (_E, [_P, _P, _I64, _E, _I64, _P, _I32, _I32,
                                      _I32, _P, _P, _P, _P, _P, _P, _P, _SZ, _P,
                                      _E, _P, _P, _P]),
    "moe_gate_backward_workspace_size": (_SZ, [_I64, _I32, _I32]),
    "moe_gate_backward": (_E, [_P, _E, _P, _P, _P, _P, _P, _I32, _I32, _I32,
                               _I32, _I32, _I32, _F, _F, _E, _P, _P, _P, _E,
                               _P, _P, _P, _P, _SZ, _P]),
    "moe_routing_histogram": (_E, [_P, _I32, _I32, _I32, _I32, _P, _I32, _P, _P,
                                   _P]),
}

_lib = None


class MoEError(RuntimeError):
    def __init__(self, name: str, status: int, detail: str):
        super().__init__(f"{name} failed with {status_string(status)}: {detail}")
        self.status = status


def load() -> ctypes.CDLL:
    """Load libmoe.so once; raise if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m sparse_moe_diffusion_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def status_string(status: int) -> str:
    return load().moe_status_string(status).decode()


def last_error() -> str:
    return load().moe_last_error().decode()


def call(name: str, *args) -> int:
    """Call an entry point; raise MoEError on a non-zero status."""
    st = getattr(load(), name)(*args)
    if st != MOE_OK:
        raise MoEError(name, st, last_error())
    return st


def call_status(name: str, *args) -> int:
    """Call an entry point and return its status (no raise)."""
    return getattr(load(), name)(*args)
