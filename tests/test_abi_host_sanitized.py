"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer:
libmoe.so is built with its host side instrumented (device code as usual),
and the host tests (argument validation, workspace queries, exported
symbols, the gathered-row offset arithmetic) run against it in a child
process with clang's ASan runtime preloaded.  Any sanitizer report aborts
the child and fails this test."""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _asan_runtime():
    hits = sorted(glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/"
                            "libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


def test_host_tests_under_asan_ubsan(tmp_path):
    rt = _asan_runtime()
    if rt is None or not os.path.exists("/opt/rocm/bin/hipcc"):
        pytest.skip("no hipcc / clang ASan runtime")
    sys.path.insert(0, ROOT)
    from sparse_moe_diffusion_amd import build
    lib = build.build(sanitize=True)
    log = str(tmp_path / "sanitizer")
    env = dict(os.environ)
    env.update(
        LD_PRELOAD=rt,
        MOE_LIB_PATH=lib,
        ASAN_OPTIONS=f"detect_leaks=0:halt_on_error=1:log_path={log}",
        UBSAN_OPTIONS=f"halt_on_error=1:print_stacktrace=1:log_path={log}")
    r = subprocess.run(
        [sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
         os.path.join(ROOT, "tests", "test_abi_host.py"),
         os.path.join(ROOT, "tests", "test_gather_offsets.py")],
        cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    reports = ""
    for f in glob.glob(log + "*"):
        reports += open(f).read()
    assert r.returncode == 0 and not reports, (
        f"rc={r.returncode}\n{r.stdout[-3000:]}\n{r.stderr[-3000:]}\n"
        f"{reports[:4000]}")
