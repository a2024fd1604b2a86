"""The numerical claim the fp8 dispatch kernel relies on, checked on the CPU.

The kernel does not divide every element by the block scale.  It computes
y = RN(1/s) once per block and corrects q0 = |x|*y with Markstein's step
(r = fma(-q0, s, |x|), q = fma(r, y, q0)), then applies the sign of x after
encoding.  The claim: for every bf16 amax >= 2^-80 and every bf16 x with
|x| <= amax, the 8-bit code of that q, with x's sign, equals the code of the
correctly rounded quotient x / s, for both formats the kernel casts to:
OCP E4M3 with s = RN(amax / 448) and OCP E5M2 with s = RN(amax / 57344).

This test restates the claim in C, independently of both the kernel and the
oracle, and checks it on a sweep over amax significands and exponents and
over x, with the same RNE-saturating rounding of each format written from
its definition here.  The amax exponents are sampled (every 7th) so the suite
stays fast; the full sweep (every bf16 amax >= 2^-80, every |x| <= amax)
was run the same way with no mismatch.  The GPU parity tests then check the kernel itself against the
oracle bit for bit.
"""

import os
import subprocess

import pytest

SRC = r"""
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>
static float bf(uint32_t hi) { uint32_t u = hi << 16; float f; memcpy(&f, &u, 4); return f; }
/* the finite non-negative values of the format, ascending with their
   codes: E4M3 codes 0..0x7E (bias 7, 3 mantissa bits, largest 448), E5M2
   codes 0..0x7B (bias 15, 2 mantissa bits, largest 57344) */
static double VAL[127];
static int TOP;
static float FMAX;
static void table(int e5m2) {
    TOP = e5m2 ? 0x7B : 0x7E;
    FMAX = e5m2 ? 57344.0f : 448.0f;
    for (int c = 0; c <= TOP; ++c) {
        int mb = e5m2 ? 2 : 3, bias = e5m2 ? 15 : 7;
        int e = c >> mb, m = c & ((1 << mb) - 1);
        double f = (double)m / (1 << mb);
        VAL[c] = e ? ldexp(1.0 + f, e - bias) : ldexp(f, 1 - bias);
    }
}
/* nearest code by binary search in the table, ties to the even code,
   saturating at the largest finite value; sign kept */
static unsigned enc(float v) {
    unsigned s = signbit(v) ? 0x80u : 0u;
    double a = fabs((double)v);
    if (a >= VAL[TOP]) return s | (unsigned)TOP;
    int lo = 0, hi = TOP;                 /* VAL[lo] <= a < VAL[hi] */
    while (hi - lo > 1) { int mid = (lo + hi) / 2; if (VAL[mid] <= a) lo = mid; else hi = mid; }
    double dl = a - VAL[lo], dh = VAL[hi] - a;
    unsigned c = dl < dh ? (unsigned)lo : dh < dl ? (unsigned)hi : ((lo & 1) ? (unsigned)hi : (unsigned)lo);
    return s | c;
}
int main(int argc, char** argv) {
    int step = atoi(argv[1]);
    long n = 0, bad = 0;
    table(atoi(argv[2]));
    for (int ae = 127 - 80; ae <= 254; ae += step)
        for (int am = 0; am < 128; ++am) {
            float amax = bf((uint32_t)(ae << 7 | am));
            float s = amax / FMAX, y = 1.0f / s;
            for (int xe = 0; xe <= ae; ++xe) {
                if (ae - xe > 24 && xe % 11) continue;   /* far below 2^-10 * s: sample */
                for (int xm = 0; xm < 128; ++xm)
                    for (int sg = 0; sg < 2; ++sg) {
                        float x = bf((uint32_t)(sg << 15 | xe << 7 | xm));
                        if (fabsf(x) > amax) continue;
                        float ax = fabsf(x), q0 = ax * y, r = fmaf(-q0, s, ax), q = fmaf(r, y, q0);
                        unsigned got = enc(q) | (signbit(x) ? 0x80u : 0u);
                        ++n;
                        if (got != enc(x / s)) { if (bad < 5) printf("amax=%a x=%a\n", amax, x); ++bad; }
                    }
            }
        }
    printf("%ld %ld\n", n, bad);
    return 0;
}
"""


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_markstein_quotient_gives_the_division_code(tmp_path, fmt):
    src = tmp_path / "claim.c"
    exe = tmp_path / "claim"
    src.write_text(SRC.replace("#include <string.h>", "#include <string.h>\n#include <stdlib.h>"))
    subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-o", str(exe), str(src), "-lm"], check=True)
    out = subprocess.run([str(exe), "7", "1" if fmt == "e5m2" else "0"], capture_output=True,
                         text=True, check=True).stdout
    n, bad = map(int, out.split()[-2:])
    assert n > 2_000_000
    assert bad == 0, out
