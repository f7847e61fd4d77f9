"""The byte-offset arithmetic of rows gathered through a row index
(csrc/gather.hpp), compiled as plain C++ on the host and checked against
exact integer arithmetic: valid entries address their own row, every other
entry (negative, past the matrix, the int32 extremes) lands at or past the
end of the buffer descriptor's range, and within the row-count limit the
largest offset a kernel forms never wraps around 32 bits."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "sparse_moe_diffusion_amd", "csrc")

PROGRAM = r"""
#include <stdio.h>
#include "gather.hpp"
int main() {
  long long src;
  unsigned long long rows, rb, col;
  while (scanf("%lld %llu %llu %llu", &src, &rows, &rb, &col) == 4)
    printf("%u %d %d\n",
           moe::gather_row_offset((int)src, (unsigned)rows, (unsigned)rb,
                                  (unsigned)col),
           (int)moe::gather_fits((long long)rows, (long long)rb),
           (int)moe::gather_row_valid(src, (long long)rows));
  return 0;
}
"""


@pytest.fixture(scope="module")
def prog(tmp_path_factory):
    cxx = shutil.which("g++")
    if cxx is None:
        pytest.skip("no host C++ compiler")
    d = tmp_path_factory.mktemp("gather")
    src = d / "gather_check.cpp"
    src.write_text(PROGRAM)
    exe = d / "gather_check"
    # the header's functions are host+device; on the host the qualifiers
    # are empty
    subprocess.run([cxx, "-std=c++17", "-O1", "-D__host__=", "-D__device__=",
                    f"-I{CSRC}", str(src), "-o", str(exe)], check=True)
    return str(exe)


def _run(exe, cases):
    text = "".join(f"{s} {r} {b} {c}\n" for s, r, b, c in cases)
    out = subprocess.run([exe], input=text, capture_output=True, text=True,
                         check=True).stdout.split("\n")
    return [tuple(int(v) for v in line.split()) for line in out if line]


def _fits(rows, rb):
    return rows >= 0 and rb > 0 and (rows + 1) * rb + 256 <= 1 << 32


def test_offsets_against_integer_arithmetic(prog):
    cases = []
    for rows, rb in [(1, 256), (7, 2304), (32768, 2304), (16384, 4096),
                     ((1 << 24) - 2, 256), (1864134, 2304)]:
        assert _fits(rows, rb)
        for src in (0, 1, rows - 1, rows, rows + 1, -1, -2, -(1 << 31),
                    (1 << 31) - 1, rows // 2):
            for col in (0, 16, rb - 16, rb + 112):
                cases.append((src, rows, rb, col))
    for (src, rows, rb, col), (off, fits, valid) in zip(cases, _run(prog, cases)):
        ok = 0 <= src < rows
        assert valid == ok
        assert fits == 1
        if ok:
            assert off == src * rb + col
        else:
            # past the descriptor's range [0, rows * rb): reads zero
            assert off == rows * rb + col
            assert off >= rows * rb
        # no 32-bit wrap for any column offset a kernel adds (< rb + 256)
        assert rows * rb + col < 1 << 32


def test_fits_boundary(prog):
    # (rows + 1) * rb + 256 == 2^32 fits, one more row does not
    rb = 256
    edge = ((1 << 32) - 256) // rb - 1
    res = _run(prog, [(0, edge, rb, 0), (0, edge + 1, rb, 0)])
    assert [r[1] for r in res] == [1, 0]
    assert _fits(edge, rb) and not _fits(edge + 1, rb)
