"""Build libmoe.so (the gfx950 HIP kernels and the C ABI) in-tree.

Usage:  python -m sparse_moe_diffusion_amd.build [-v]
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libmoe.so")
BUILD_DIR = os.path.join(PKG, "_build")

SOURCES = ["gate.hip", "permute.hip", "ffn.hip", "combine.hip", "balance.hip",
           "analytics.hip", "backward.hip", "abi.cpp"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # no packed fp32 instructions anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    # a variable read before it is set is an error, not a warning
    "-Werror=uninitialized", "-Werror=sometimes-uninitialized",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


# Host-side AddressSanitizer and UndefinedBehaviorSanitizer for the C ABI's
# validation code (device code is built as usual): each flag applies to the
# host compilation only.
HOST_SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host",
                 "-fsanitize=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
                 "-Xarch_host", "-shared-libasan"]


def _compile(src: str, verbose: bool, build_dir: str = BUILD_DIR,
             extra=()) -> str:
    obj = os.path.join(build_dir, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, *extra, "-x", "hip", "-c", os.path.join(CSRC, src),
           "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{out}")
    if verbose and out.strip():
        print(out, flush=True)
    return obj


def build(verbose: bool = False, sanitize: bool = False) -> str:
    """Compile every source for gfx950 and link libmoe.so; returns its path.
    With sanitize, the host code is instrumented with ASan and UBSan and the
    library goes to _build/host_sanitize/libmoe.so (loaded with the clang
    ASan runtime preloaded; see tests/test_abi_host_sanitized.py)."""
    bdir = os.path.join(BUILD_DIR, "host_sanitize") if sanitize else BUILD_DIR
    lib = os.path.join(bdir, "libmoe.so") if sanitize else LIB
    extra = HOST_SANITIZE if sanitize else []
    os.makedirs(bdir, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 4)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose, bdir, extra), SOURCES))
    tmp = lib + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *extra, *objs,
           "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}{r.stderr}")
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
