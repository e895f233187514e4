"""The AdamW kernels (device and host) divide m and v by the bias corrections
1 - beta^t through the correctly rounded reciprocal of the divisor and one
fused correction step.  By Markstein's theorem (P. Markstein, "Computation of
elementary functions on the IBM RISC System/6000 processor", IBM J. Res.
Dev. 34(1), 1990) that gives the correctly rounded quotient for finite
operands without underflow.  This checks it in C on the host, bit for bit
against IEEE division, for every bias correction the steps use (beta in a
grid of common values, t up to 10^4) and random dividends, plus random
divisors in (0, 1]; a zero dividend keeps its sign by a separate select."""
import os
import shutil
import subprocess

import pytest

SRC = r"""
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>
static uint64_t s = 0x9E3779B97F4A7C15ull;
static uint64_t xr(void) { s ^= s << 13; s ^= s >> 7; s ^= s << 17; return s; }
static double dividend(void) {
    uint64_t u = xr();
    double x = ldexp(1.0 + (double)(u >> 11) * 0x1p-53, (int)(xr() % 300) - 160);
    if (xr() & 1) {  /* fp32-representable values too (finite, non-zero ones) */
        float f = (float)x;
        if (isfinite(f) && f != 0.0f) x = f;
    }
    return (u & 1) ? -x : x;
}
static int same(double q, double a, double b) { double r = a / b; return memcmp(&q, &r, 8) == 0; }
static double div_by(double a, double b, double rb) {
    double q0 = a * rb;
    double q = fma(fma(-b, q0, a), rb, q0);
    return a == 0.0 ? a : q;
}
int main(void) {
    const double betas[] = {0.0, 0.5, 0.8, 0.9, 0.95, 0.98, 0.99, 0.995, 0.999, 0.9999};
    long bad = 0, n = 0;
    for (int i = 0; i < 10; ++i)
        for (long t = 1; t <= 10000; t += t < 100 ? 1 : 97) {
            volatile double p = pow(betas[i], (double)t);
            double b = 1.0 - p;
            if (b == 0.0) continue;
            double rb = 1.0 / b;
            for (int k = 0; k < 2000; ++k, ++n) {
                double a = dividend();
                bad += !same(div_by(a, b, rb), a, b);
            }
            bad += !same(div_by(0.0, b, rb), 0.0, b) + !same(div_by(-0.0, b, rb), -0.0, b);
        }
    for (long k = 0; k < 4000000; ++k, ++n) {
        double b = (double)((xr() >> 11) | 1) * 0x1p-53, a = dividend();
        bad += !same(div_by(a, b, 1.0 / b), a, b);
    }
    printf("%ld %ld\n", n, bad);
    return 0;
}
"""


def test_reciprocal_division_is_correctly_rounded(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc is not installed")
    src, exe = tmp_path / "div.c", tmp_path / "div"
    src.write_text(SRC)
    subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", str(src), "-o",
                    str(exe), "-lm"], check=True)
    n, bad = (int(x) for x in subprocess.run([str(exe)], check=True, capture_output=True,
                                               text=True, timeout=120).stdout.split())
    assert n > 5_000_000 and bad == 0, (n, bad)
