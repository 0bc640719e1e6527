"""The quantization kernels divide every element of a block by the block's
scale s through its reciprocal: q0 = x * (1/s), then one fma correction with
the residual x - s*q0 (Markstein's method). This CPU test checks, in C with the
C library's correctly rounded fmaf and IEEE division, that the corrected
quotient rounds to the same int8 byte as x / s for every bf16 x within the
block's range, over scales s = amax / 127 spread across the exponent range
(s >= 2^-90, the kernels' condition for using it), and that it equals the IEEE
quotient bit for bit whenever |x| >= s/4 (below that the residual may
underflow, and the byte is 0 either way). Near-tie values x = s*(k + 1/2)
+- a few ulps are included. The formula is restated here from the method; no
GPU code is compiled or run.
"""
from __future__ import annotations

import shutil
import subprocess

import pytest

SRC = r"""
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>
static float from_bits(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t to_bits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }
static int byte_of(float q) { return (int)fminf(fmaxf(rintf(q), -127.f), 127.f); }
static long long n, bad_q, bad_b;
static void check(float x, float s, float rs) {
    const float q = x / s;
    const float q0 = x * rs;
    const float q1 = fmaf(fmaf(-s, q0, x), rs, q0);
    ++n;
    if (fabsf(x) >= 0.25f * s && to_bits(q1) != to_bits(q)) ++bad_q;
    if (byte_of(q1) != byte_of(q)) ++bad_b;
}
int main(void) {
    uint32_t seed = 12345u;
    for (int t = 0; t < 400; ++t) {
        seed = seed * 1664525u + 1013904223u;
        /* amax: a random fp32 with exponent in [-80, 100] */
        const uint32_t e = 47u + (seed >> 8) % 181u;
        const float amax = from_bits((e << 23) | (seed & 0x7fffffu));
        const float s = amax / 127.0f;
        if (!(s >= 0x1p-90f)) continue;
        const float rs = 1.0f / s;
        for (uint32_t p = 0; p < 65536u; ++p) {
            const float x = from_bits(p << 16);
            if (isfinite(x) && fabsf(x) <= amax) check(x, s, rs);
        }
        for (int k = 0; k <= 127; ++k)
            for (int d = -4; d <= 4; ++d) {
                const float x = from_bits(to_bits(s * ((float)k + 0.5f)) + d);
                if (isfinite(x) && fabsf(x) <= amax) { check(x, s, rs); check(-x, s, rs); }
            }
    }
    printf("%lld %lld %lld\n", n, bad_q, bad_b);
    return 0;
}
"""


def test_reciprocal_division_gives_the_ieee_bytes(tmp_path):
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    src = tmp_path / "div.c"
    exe = tmp_path / "div"
    src.write_text(SRC)
    subprocess.run([cc, "-O2", "-ffp-contract=off", str(src), "-o", str(exe), "-lm"], check=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.split()
    n, bad_q, bad_b = (int(v) for v in out)
    assert n > 10_000_000
    assert bad_q == 0, f"{bad_q} quotients with |x| >= s/4 differ from x / s"
    assert bad_b == 0, f"{bad_b} bytes differ"
