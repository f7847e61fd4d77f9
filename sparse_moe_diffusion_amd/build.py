"""Build libmoe.so (the gfx950 HIP kernels and the C ABI) in-tree.

Usage:  python -m sparse_moe_diffusion_amd.build [-v]
"""
from __future__ import annotations

import json
import os
import re
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libmoe.so")
BUILD_DIR = os.path.join(PKG, "_build")
# The compiler's register, scratch and LDS figures of every kernel of the
# last build (written by build(); read by the host tests, which require that
# no GEMM kernel spills registers to scratch).
RESOURCES = os.path.join(BUILD_DIR, "kernel_resources.json")

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


RESOURCE_REMARKS = "-Rpass-analysis=kernel-resource-usage"
_REMARK = re.compile(r"remark:\s+(.+?): (\S+) \[" + re.escape(RESOURCE_REMARKS) + r"\]")


def parse_resource_usage(text: str) -> dict:
    """{kernel symbol: {figure: value}} from the compiler's resource-usage
    remarks (VGPRs, AGPRs, 'VGPRs Spill', 'ScratchSize [bytes/lane]', ...)."""
    out, cur = {}, None
    for line in text.splitlines():
        m = _REMARK.search(line)
        if not m:
            continue
        key, val = m.group(1), m.group(2)
        if key == "Function Name":
            cur = out.setdefault(val, {})
        elif cur is not None:
            cur[key] = int(val) if val.lstrip("-").isdigit() else val
    return out


def _compile(src: str, verbose: bool, build_dir: str = BUILD_DIR,
             extra=()) -> tuple:
    obj = os.path.join(build_dir, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, *extra, "-x", "hip", "-c", os.path.join(CSRC, src),
           "-o", obj]
    if src.endswith(".hip"):
        cmd.append(RESOURCE_REMARKS)
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    text = r.stdout + r.stderr
    out = "\n".join(l for l in text.splitlines()
                    if "packed-fp32-ops" not in l and RESOURCE_REMARKS[2:] not in l
                    and not l.lstrip().startswith(("|", "^")) and
                    not re.match(r"\s*\d+ \|", l))
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{out}")
    if verbose and out.strip():
        print(out, flush=True)
    return obj, parse_resource_usage(text)


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
        done = list(ex.map(lambda s: _compile(s, verbose, bdir, extra), SOURCES))
    objs = [o for o, _ in done]
    if not sanitize:
        usage = {}
        for src, (_, u) in zip(SOURCES, done):
            for k, v in u.items():
                usage[k] = dict(v, source=src)
        with open(RESOURCES, "w") as f:
            json.dump(usage, f, indent=1, sort_keys=True)
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
