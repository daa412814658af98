"""The quantizer's reciprocal-and-correct division, checked on the host.

The block encoder divides each element by the block divisor d without a
divide instruction: y = RN(1/d), q0 = RN(x*y), then twice q <- fma(-(fma(q, d,
-x)), y, q).  Under the encoder's conditions (d in [2^-100, 2^125), |x| <= 8d,
x a bf16 value) the result must equal the IEEE quotient bit for bit, signed
zeros included, except where both are below 2^-11 in magnitude with the same
sign (such quotients give E2M1 code 0 or 8 either way).  The same fp32
operations run on the host's FMA unit here: IEEE fma is defined bit for bit,
so the check carries over to the GPU.  Every finite bf16 numerator is tried
against a spread of divisors (random normals, all-ones mantissas, short
mantissas, the range limits).
"""
import os
import shutil
import subprocess

import pytest

SRC = r"""
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>
static float f_of(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t u_of(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }
static float div_rn(float a, float d, float y) {
    float q0 = a * y;
    float n0 = fmaf(q0, d, -a);
    __asm__("" : "+x"(n0));   /* keep the negations where they are written */
    float q1 = fmaf(-n0, y, q0);
    float n1 = fmaf(q1, d, -a);
    __asm__("" : "+x"(n1));
    return fmaf(-n1, y, q1);
}
int main(int argc, char** argv) {
    long nd = atol(argv[1]);
    long bad = 0, total = 0;
    #pragma omp parallel for reduction(+:bad,total) schedule(dynamic, 16)
    for (long i = 0; i < nd + 4; i++) {
        uint64_t z = 0x9E3779B97F4A7C15ull * (uint64_t)(i + 1);
        z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull; z = (z ^ (z >> 27)) * 0x94D049BB133111EBull; z ^= z >> 31;
        uint32_t e = 27 + (uint32_t)((z >> 23) % 225);          /* exponents of [2^-100, 2^125) */
        uint32_t ub;
        switch (i % 3) {
            case 0: ub = (uint32_t)(z & 0x7FFFFFu) | (e << 23); break;
            case 1: ub = 0x7FFFFFu | (e << 23); break;
            default: ub = (uint32_t)((z & 0xFu) << 19) | (e << 23); break;
        }
        if (i == nd) ub = u_of(0x1p-100f);
        if (i == nd + 1) ub = u_of(0x1.fffffep124f);
        if (i == nd + 2) ub = u_of(1.0f);
        if (i == nd + 3) ub = u_of(0x1.8p-9f / 6.0f);
        float d = f_of(ub);
        if (!(d >= 0x1p-100f && d < 0x1p125f)) continue;
        float y = 1.0f / d, cap = 8.0f * d;
        for (uint32_t h = 0; h < 0x10000; h++) {
            if ((h & 0x7F80) == 0x7F80) continue;          /* inf / nan */
            float a = f_of(h << 16);
            if (fabsf(a) > cap) continue;
            float ref = a / d, got = div_rn(a, d, y);
            total++;
            if (u_of(got) == u_of(ref)) continue;
            if (fabsf(ref) < 0x1p-11f && fabsf(got) < 0x1p-11f && signbit(ref) == signbit(got)) continue;
            bad++;
        }
    }
    printf("%ld %ld\n", total, bad);
    return 0;
}
"""


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_reciprocal_division_is_exact(tmp_path):
    src = tmp_path / "div.c"
    exe = tmp_path / "div"
    src.write_text(SRC)
    flags = ["-O2", "-ffp-contract=off", "-mfma", "-fopenmp"]
    r = subprocess.run(["gcc", *flags, "-o", str(exe), str(src), "-lm"], capture_output=True, text=True)
    if r.returncode != 0:
        pytest.skip("host compiler without FMA/OpenMP support: " + r.stderr[-200:])
    env = dict(os.environ, OMP_NUM_THREADS=str(min(8, os.cpu_count() or 1)))
    out = subprocess.run([str(exe), "3000"], capture_output=True, text=True, env=env, timeout=600)
    total, bad = (int(v) for v in out.stdout.split())
    assert total > 10**8
    assert bad == 0
