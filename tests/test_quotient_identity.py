"""The quantiser's division-free quotient equals IEEE division (no GPU needed).

The activation kernel computes r / s for a whole row with one divide per row:
y = RN(1/s), q0 = RN(r*y), e = fma(-q0, s, r), q1 = fma(e, y, q0). Markstein's
division theorem says q1 = RN(r/s); this test checks that claim against the
IEEE divide for every fp32 numerator mantissa and a sample of divisor
mantissas (the result is invariant under power-of-two scaling of r and s as
long as nothing overflows or underflows, which the kernel guarantees by using
the IEEE divide when s is outside [2^-120, 2^120]). It also checks the
1.5 * 2^23 rounding trick against rintf over the quantiser's code range.
"""
import os
import subprocess

import pytest

SRC = r"""
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>
static float fb(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t bf(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }
int main(int argc, char **argv) {
  int ns = atoi(argv[1]);
  long long bad = 0, total = 0;
  #pragma omp parallel for reduction(+:bad,total) schedule(dynamic)
  for (int t = 0; t < ns; ++t) {
    uint64_t x = 0x243F6A8885A308D3ull + (uint64_t)t * 0x9E3779B97F4A7C15ull;
    x ^= x >> 31; x *= 0xBF58476D1CE4E5B9ull; x ^= x >> 29;
    static const uint32_t special[8] = {0, 1, 0x7FFFFF, 0x400000, 0x3504F3, 0x12345, 0x7FFFFE, 0x555555};
    uint32_t sm = t < 8 ? special[t] : (uint32_t)(x & 0x7FFFFF);
    float s = fb(0x3F800000u | sm);
    float y = 1.0f / s;
    for (uint32_t rm = 0; rm < (1u << 23); ++rm) {
      float r = fb(0x3F800000u | rm);
      float q0 = r * y;
      float e = fmaf(-q0, s, r);
      float q1 = fmaf(e, y, q0);
      total++;
      if (bf(q1) != bf(r / s)) bad++;
    }
  }
  /* rounding by adding 1.5 * 2^23: low byte = rintf(q) as int8 for |q| <= 127.25 (codes stay in [-127, 127]) */
  long long bad2 = 0;
  for (float q = -128.0f; q <= 128.0f; q = nextafterf(q, 200.0f)) {
    uint32_t bits = bf(q + 12582912.0f);
    int code = (int8_t)(bits & 0xFF);
    if (fabsf(q) <= 127.25f && code != (int)rintf(q)) bad2++;
  }
  printf("%lld %lld %lld\n", total, bad, bad2);
  return 0;
}
"""


@pytest.fixture(scope="module")
def prog(tmp_path_factory):
    d = tmp_path_factory.mktemp("quot")
    src = d / "q.c"
    src.write_text(SRC)
    exe = d / "q"
    subprocess.check_call(["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-mfma", str(src), "-o", str(exe), "-lm"])
    return str(exe)


def test_markstein_quotient_matches_ieee_division(prog):
    out = subprocess.check_output([prog, "256"], env=dict(os.environ, OMP_NUM_THREADS="8"), text=True)
    total, bad, bad2 = map(int, out.split())
    assert total == 256 * (1 << 23)
    assert bad == 0
    assert bad2 == 0
