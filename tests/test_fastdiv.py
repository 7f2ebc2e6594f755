"""The kernels' magic-number division (block_sparse_draft_amd/csrc/fastdiv.h),
compiled for the host and checked against exact integer division on edge and
random dividends for every divisor below 5000 and random divisors up to 2^31."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PROGRAM = r'''
#include <hip/hip_runtime.h>
#include <cstdio>
#include "fastdiv.h"
int main() {
  unsigned long long bad = 0, checks = 0;
  unsigned seed = 12345;
  auto rnd = [&]() { seed = seed * 1103515245u + 12345u; return seed >> 1; };
  for (int d = 1; d < 5000; ++d) {
    skv::FastDiv f = skv::FastDiv::make(d);
    int ns[] = {0, 1, d - 1, d, d + 1, 2 * d - 1, 2 * d, 0x7fffffff, 0x7fffffff - d};
    for (int n : ns) { ++checks; if (f.div(n) != n / d || f.mod(n) != n % d) ++bad; }
    for (int k = 0; k < 200; ++k) {
      int n = (int)(rnd() & 0x7fffffff); ++checks;
      if (f.div(n) != n / d || f.mod(n) != n % d) ++bad;
    }
  }
  for (int k = 0; k < 20000; ++k) {
    int d = (int)(rnd() & 0x7fffffff); if (d == 0) d = 1;
    skv::FastDiv f = skv::FastDiv::make(d);
    int n = (int)(rnd() & 0x7fffffff); ++checks;
    if (f.div(n) != n / d) ++bad;
  }
  printf("%llu %llu\n", bad, checks);
  return bad != 0;
}
'''


def test_fast_division_matches_exact_division(tmp_path):
    hipcc = "/opt/rocm/bin/hipcc" if os.path.exists("/opt/rocm/bin/hipcc") else shutil.which("hipcc")
    if hipcc is None:
        pytest.skip("hipcc not available")
    src = tmp_path / "fd.cpp"
    src.write_text(PROGRAM)
    exe = tmp_path / "fd"
    subprocess.run([hipcc, "-x", "hip", "--offload-host-only", "-O2", "-I",
                    os.path.join(ROOT, "block_sparse_draft_amd", "csrc"), str(src), "-o", str(exe)],
                   check=True, capture_output=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True)
    bad, checks = map(int, out.stdout.split())
    assert out.returncode == 0 and bad == 0 and checks > 1_000_000
