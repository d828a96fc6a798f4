"""The kernels' multiply-shift division, checked on the CPU.

Every kernel splits its flat work-item index into (unit, list, tile, ...)
with `fast_div`, whose multiplier and shift the host derives with
`make_fastdiv` (Granlund and Montgomery, "Division by invariant integers
using multiplication", 1994).  A wrong multiplier would silently send a
workgroup to another unit's data, so the exact quotient is pinned here
against plain integer division: exhaustively for small divisors and
dividends, at the edges of the dividend range (up to 2^31 - 1), and on
random pairs.  The test compiles the header's host path with hipcc; it
needs no GPU.
"""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "sparse_weight_memory_amd", "csrc")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"

PROGRAM = r"""
#include "fwpkm_device.h"
#include <cstdio>
#include <cstdint>
#include <random>

static int check(int x, int d, fwpkm::FastDiv f) {
  if (fwpkm::fast_div(x, f) != x / d) {
    std::printf("mismatch x=%d d=%d got=%d want=%d\n", x, d, fwpkm::fast_div(x, f), x / d);
    return 1;
  }
  return 0;
}

int main() {
  long long checked = 0;
  // every divisor up to 4096, every dividend below 70000
  for (int d = 1; d <= 4096; ++d) {
    const fwpkm::FastDiv f = fwpkm::make_fastdiv(d);
    for (int x = 0; x < 70000; ++x, ++checked)
      if (check(x, d, f)) return 1;
    // the top of the dividend range and the multiples of d around it
    const int top = 0x7fffffff;
    for (int x = top; x > top - 3 * d - 3; --x, ++checked)
      if (check(x, d, f)) return 1;
  }
  // powers of two, their neighbours and large divisors, against every edge
  std::mt19937_64 rng(20260101);
  for (int e = 0; e < 31; ++e)
    for (int delta = -1; delta <= 1; ++delta) {
      const long long dd = (1ll << e) + delta;
      if (dd < 1 || dd > 0x7fffffff) continue;
      const int d = (int)dd;
      const fwpkm::FastDiv f = fwpkm::make_fastdiv(d);
      for (int i = 0; i < 20000; ++i, ++checked) {
        const int x = (int)(rng() & 0x7fffffff);
        if (check(x, d, f)) return 1;
      }
      for (long long m = 0; m <= 4; ++m)
        for (long long off = -1; off <= 1; ++off) {
          const long long x = m * (long long)d + off;
          if (x < 0 || x > 0x7fffffff) continue;
          ++checked;
          if (check((int)x, d, f)) return 1;
        }
    }
  // random divisors and dividends over the whole range
  for (int i = 0; i < 2000000; ++i, ++checked) {
    const int d = 1 + (int)(rng() % 0x7fffffff);
    const int x = (int)(rng() & 0x7fffffff);
    if (check(x, d, fwpkm::make_fastdiv(d))) return 1;
  }
  std::printf("ok %lld\n", checked);
  return 0;
}
"""


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not found")
def test_fast_div_equals_integer_division(tmp_path):
    src = tmp_path / "fastdiv.cpp"
    exe = tmp_path / "fastdiv"
    src.write_text(PROGRAM)
    # host-only build of the header (its device functions are never called)
    subprocess.run([HIPCC, "-x", "hip", "--cuda-host-only", "-std=c++17", "-O2",
                    "-I", CSRC, str(src), "-o", str(exe)],
                   check=True, capture_output=True, text=True, timeout=300)
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300)
    assert out.returncode == 0, out.stdout + out.stderr
    assert out.stdout.startswith("ok ")
