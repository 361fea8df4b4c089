"""The FP8 cast kernels divide x by the group scale s as
    q = RN(x * y), r = fma(-s, q, x), x/s ~ fma(r, y, q),   y = RN(1/s),
with the sign of x copied onto the result. By Markstein's theorem (y the
correctly rounded reciprocal, q within one ulp of x/s) this is the correctly
rounded quotient RN(x/s) whenever the quotient is a normal float; below that
every E4M3 code is a signed zero either way. This test checks the identity
exhaustively on the CPU -- every bf16 significand of x against every float
significand of s, in both orders of magnitude -- so the kernels' codes can
match the oracle's plain division bit for bit. The quotient's significand
depends only on the two significands, so one exponent of s covers all."""
import os
import subprocess

SRC = r"""
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>
static float u2f(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static float div_fma(float x, float s, float y) {
  float q = x * y;
  float r = fmaf(-s, q, x);
  return copysignf(fmaf(r, y, q), x);
}
int main(void) {
  long bad = 0, n = 0;
  for (uint32_t sign = 0; sign < 2; ++sign)
    for (uint32_t xm = 0; xm < 128; ++xm)
      for (uint32_t xe = 0; xe < 2; ++xe) {
        float x = u2f(sign << 31 | (126u + xe) << 23 | xm << 16);
        for (uint32_t sm = 0; sm < (1u << 23); sm += 1) {
          float s = u2f(120u << 23 | sm);
          float y = 1.0f / s;
          float got = div_fma(x, s, y), want = x / s;
          ++n;
          if (memcmp(&got, &want, 4) != 0) {
            if (bad < 4) printf("x=%a s=%a got %a want %a\n", x, s, got, want);
            ++bad;
          }
        }
      }
  /* signed zeros */
  float z[2] = {0.0f, -0.0f};
  for (int i = 0; i < 2; ++i) {
    float got = div_fma(z[i], 0.3f, 1.0f / 0.3f), want = z[i] / 0.3f;
    if (memcmp(&got, &want, 4) != 0) { printf("zero sign\n"); ++bad; }
  }
  printf("%ld %ld\n", n, bad);
  return bad != 0;
}
"""


def test_fma_corrected_division_is_correctly_rounded(tmp_path):
    c = os.path.join(str(tmp_path), "div.c")
    exe = os.path.join(str(tmp_path), "div")
    with open(c, "w") as f:
        f.write(SRC)
    subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-o", exe, c, "-lm"], check=True)
    out = subprocess.run([exe], capture_output=True, text=True, timeout=600)
    assert out.returncode == 0, out.stdout
    n, bad = map(int, out.stdout.split()[-2:])
    assert n == 2 * 128 * 2 * (1 << 23) and bad == 0
