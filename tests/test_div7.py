"""The IF4 kernels divide k * 6 s g by 7 in fp64 without a division
instruction: q0 = RN(x y) with y = RN(1/7), r = fma(-q0, 7, x) (exact), then
q = fma(r, y, q0), Markstein's correction.  The numerator is an integer of at
most 33 significant bits times a power of two (k <= 7, 6, the 4-bit E4M3
significand and the 24-bit fp32 g), and rounding of x / 7 does not depend on
the power of two, so checking every integer in [2^32, 2^33) against the
correctly rounded division shows that the kernels' quotient is the division's
for every input they see.  Host C, compiled with gcc (OpenMP over the host's
cores, a few seconds)."""
import os
import shutil
import subprocess

import pytest

SRC = r"""
#include <math.h>
#include <stdint.h>
#include <stdio.h>
int main(void) {
  const double y = 1.0 / 7.0;
  unsigned long long bad = 0;
#pragma omp parallel for reduction(+ : bad) schedule(static)
  for (long hi = 0; hi < (1L << 16); ++hi) {
    for (unsigned long lo = 0; lo < (1UL << 16); ++lo) {
      const double x = (double)((1ULL << 32) + ((unsigned long long)hi << 16) + lo);
      const double q0 = x * y;
      const double q = fma(fma(-q0, 7.0, x), y, q0);
      const volatile double ref = x / 7.0;
      if (q != ref) ++bad;
    }
  }
  printf("%llu\n", bad);
  return 0;
}
"""


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_markstein_div7_matches_division(tmp_path):
    c = tmp_path / "div7.c"
    c.write_text(SRC)
    exe = tmp_path / "div7"
    subprocess.run(["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-o", str(exe), str(c), "-lm"], check=True)
    env = dict(os.environ, OMP_NUM_THREADS=str(min(16, os.cpu_count() or 1)))
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True, env=env, timeout=600)
    assert int(out.stdout.strip()) == 0
