"""The fp8 append's fast quotient, checked exhaustively on the CPU.

For plain scales (s = absmax / 448, fp32) the append kernel does not divide
each element: with r = 1/s (correctly rounded, once per row) it forms
q = x * r and refines it with the residual x - q * s (Markstein's correction,
two fused multiply-adds). The codes are only right if that quotient equals
the correctly rounded x / s wherever it can decide an e4m3 code. This test
runs the same IEEE binary32 sequence in C over every pair of bf16 values
x and absmax >= |x| with absmax >= 2^-82 (the range where the kernel uses
it; smaller rows divide) and requires: the two quotients agree bit for bit
whenever |x / s| >= 2^-11, and below that the fast one stays <= 2^-10, which
encodes to zero like the exact one (the code's sign is taken from x).
"""
import os
import shutil
import subprocess
import tempfile

import pytest

C_SOURCE = r"""
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>
static float bf16(uint32_t h) { uint32_t u = h << 16; float f; memcpy(&f, &u, 4); return f; }
static uint32_t bits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }
int main(void) {
  long long pairs = 0, bad = 0;
  #pragma omp parallel for reduction(+ : pairs, bad) schedule(dynamic)
  for (uint32_t ha = 1; ha < 0x7F80; ++ha) {
    const float amax = bf16(ha);
    if (!(amax >= 0x1p-82f)) continue;
    const float s = amax / 448.0f, r = 1.0f / s;
    for (uint32_t hx = 0; hx < 0x10000; ++hx) {
      const float x = bf16(hx);
      if (!(fabsf(x) <= amax)) continue;
      const float q = x * r;
      const float y = fmaf(fmaf(-q, s, x), r, q);
      const float ref = x / s;
      ++pairs;
      const int ok = fabsf(ref) >= 0x1p-11f ? bits(fabsf(y)) == bits(fabsf(ref)) : fabsf(y) <= 0x1p-10f;
      if (!ok) ++bad;
    }
  }
  printf("%lld %lld\n", pairs, bad);
  return 0;
}
"""


def test_fast_quotient_matches_correctly_rounded_division_exhaustively():
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    with tempfile.TemporaryDirectory() as d:
        src, exe = os.path.join(d, "q.c"), os.path.join(d, "q")
        with open(src, "w") as f:
            f.write(C_SOURCE)
        subprocess.run([gcc, "-O2", "-march=native", "-fopenmp", "-ffp-contract=off", src, "-o", exe, "-lm"],
                       check=True)
        env = dict(os.environ, OMP_NUM_THREADS=str(min(8, os.cpu_count() or 1)))
        out = subprocess.run([exe], check=True, capture_output=True, text=True, env=env, timeout=600).stdout
    pairs, bad = map(int, out.split())
    assert pairs > 10 ** 9        # every bf16 pair in range
    assert bad == 0
