"""Exhaustive host-side checks that the division shortcuts the HIP kernels
use give the IEEE binary32 quotient.

The kernels replace some correctly rounded divisions with Markstein's
correction step (P. Markstein, IBM J. Res. Dev. 34(1), 1990): with rs =
RN(1/s), q0 = RN(x*rs), e = fma(-q0, s, x) (exact), q1 = RN(q0 + e*rs).  The
result scales exactly by powers of two while no step leaves the normal
range, so checking every significand pair covers every exponent the kernels
let through.  Two uses are checked here, each over its whole domain:
  * the fp8 store: x a bf16 value (128 significands), s = RN(amax/448) for
    any binary32 significand (2^23), i.e. 2^30 pairs;
  * the NVFP4 block scale: t/6 for every binary32 significand t (2^23);
  * fp16 sources: every fp16 significand x (1024) against the scale of
    every fp16 amax significand (1024).
The program is plain C compiled with gcc (hardware fma when the host has
it, glibc's correctly rounded fmaf otherwise)."""
import os
import subprocess
import tempfile


SRC = r"""
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>
static float f_of(uint32_t b) { float f; memcpy(&f, &b, 4); return f; }
static uint32_t b_of(float f) { uint32_t b; memcpy(&b, &f, 4); return b; }
static float markstein(float x, float s, float rs) {
  float q0 = x * rs;
  float e = fmaf(-q0, s, x);
  return fmaf(e, rs, q0);
}
int main(void) {
  long bad6 = 0, bad8 = 0;
  volatile float six = 6.0f;
  float r6 = 1.0f / six;
  for (uint32_t m = 0; m < (1u << 23); ++m) {
    float t = f_of(0x3F800000u | m);                  /* t in [1, 2) */
    if (b_of(markstein(t, six, r6)) != b_of(t / six)) ++bad6;
  }
  for (uint32_t ms = 0; ms < (1u << 23); ++ms) {
    float s = f_of(0x3F800000u | ms);                 /* s in [1, 2) */
    float rs = 1.0f / s;
    for (uint32_t mx = 0; mx < 128; ++mx) {
      float x = f_of(0x3F800000u | (mx << 16));       /* bf16 significand */
      if (b_of(markstein(x, s, rs)) != b_of(x / s)) ++bad8;
      float x2 = x * 2.0f;                            /* quotient in [1, 4) */
      if (b_of(markstein(x2, s, rs)) != b_of(x2 / s)) ++bad8;
    }
  }
  /* fp16 sources: x any fp16 significand (1024), s = RN(m/448) for every fp16
     amax significand m (the only scales an fp16 token can produce) */
  long bad16 = 0;
  for (uint32_t ma = 0; ma < 1024; ++ma) {
    float s = f_of(0x3F800000u | (ma << 13)) / 448.0f;
    float rs = 1.0f / s;
    for (uint32_t mx = 0; mx < 1024; ++mx) {
      float x = f_of(0x3F800000u | (mx << 13));
      for (int sh = 0; sh < 2; ++sh) {
        float xx = sh ? x * 2.0f : x;
        if (b_of(markstein(xx, s, rs)) != b_of(xx / s)) ++bad16;
      }
    }
  }
  printf("%ld %ld %ld\n", bad6, bad8, bad16);
  return 0;
}
"""


def test_markstein_quotients_equal_ieee_division():
    with tempfile.TemporaryDirectory() as d:
        c = os.path.join(d, "m.c")
        exe = os.path.join(d, "m")
        open(c, "w").write(SRC)
        flags = ["-O2", "-std=c11", "-fno-fast-math", "-ffp-contract=off"]
        if "fma" in open("/proc/cpuinfo").read().split():
            flags.append("-mfma")
        subprocess.run(["gcc", *flags, c, "-o", exe, "-lm"], check=True)
        out = subprocess.run([exe], capture_output=True, text=True, check=True, timeout=600)
    bad6, bad8, bad16 = map(int, out.stdout.split())
    assert bad6 == 0, f"{bad6} significands where the corrected t/6 differs"
    assert bad8 == 0, f"{bad8} significand pairs where the corrected x/s differs"
    assert bad16 == 0, f"{bad16} fp16 significand pairs where the corrected x/s differs"


def test_invariant_integer_division_by_multiplication():
    """The kernels divide unit indices n < 2^31 by a launch-constant d with
    q = (n * m) >> (31 + l), l = ceil(log2 d), m = ceil(2^(31+l) / d)
    (Granlund and Montgomery, PLDI 1994, Theorem 4.2).  Checked here against
    integer division at the edges of every residue pattern that matters: all
    n near multiples of d and near 2^31, for every divisor up to 4096 and a
    spread of larger ones."""
    import numpy as np

    def magic(d):
        l = (d - 1).bit_length()
        return (2 ** (31 + l) + d - 1) // d, 31 + l

    rng = np.random.default_rng(0)
    divisors = list(range(1, 4097)) + [int(x) for x in rng.integers(4097, 2 ** 31, 2000)]
    for d in divisors:
        m, sh = magic(d)
        assert m < 2 ** 32
        k = np.unique(np.concatenate([np.arange(0, 64), rng.integers(0, (2 ** 31 - 1) // d + 1, 64),
                                      [(2 ** 31 - 1) // d]])).astype(np.int64)
        n = np.concatenate([k * d, k * d + d - 1, k * d - 1, [2 ** 31 - 1]])
        n = n[(n >= 0) & (n < 2 ** 31)].astype(object)
        q = [(int(v) * m) >> sh for v in n]
        assert q == [int(v) // d for v in n], d
