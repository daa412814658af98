"""The quantizer's reciprocal-and-correct division, checked on the host.

The block encoder divides each element by the block divisor d without a
divide instruction: y = RN(1/d), q0 = RN(x*y), q = fma(-(fma(q0, d, -x)), y,
q0), and only feeds q to the E2M1 rounding (nearest grid value, ties to the
even code, saturating at 6, sign kept).  Under the encoder's conditions (d in
[2^-100, 2^125), |x| <= 8d, x a bf16 value) two facts make its codes those of
the IEEE quotient:

* q is faithful: it equals RN(x/d) or a neighbour one ulp away, with the same
  sign (random and structured divisors against every finite bf16 numerator);
* next to every E2M1 midpoint, where a one-ulp difference could change the
  code, q equals RN(x/d): for every finite bf16 numerator x and every midpoint
  m, all divisors within 64 ulps of |x|/m are tried.

Both sweeps also compare the E2M1 codes directly.  The same fp32 operations
run on the host's FMA unit here: IEEE fma is defined bit for bit, so the
check carries over to the GPU.
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
static float div_q(float a, float d, float y) {
    float q0 = a * y;
    float n0 = fmaf(q0, d, -a);
    __asm__("" : "+x"(n0));   /* keep the negation where it is written */
    return fmaf(-n0, y, q0);
}
/* E2M1 rounding written as midpoint comparisons (ties to the even code) */
static unsigned e2m1(float v) {
    unsigned s = signbit(v) ? 8u : 0u;
    float a = fabsf(v);
    return s | ((a > 0.25f) + (a >= 0.75f) + (a > 1.25f) + (a >= 1.75f) + (a > 2.5f) + (a >= 3.5f) + (a > 5.0f));
}
/* returns 1 if q is not faithful to the IEEE quotient or the codes differ */
static int check(float a, float d, long* not_rn) {
    float y = 1.0f / d, ref = a / d, got = div_q(a, d, y);
    if (u_of(got) != u_of(ref)) {
        long du = (long)u_of(got) - (long)u_of(ref);
        ++*not_rn;
        if (signbit(got) != signbit(ref) || du > 1 || du < -1) return 1;
    }
    return e2m1(got) != e2m1(ref);
}
static int in_range(float a, float d) { return d >= 0x1p-100f && d < 0x1p125f && fabsf(a) <= 8.0f * d; }
int main(int argc, char** argv) {
    long nd = atol(argv[1]);
    long bad = 0, total = 0, not_rn = 0, tie_total = 0, tie_bad = 0, tie_not_rn = 0;
    /* sweep 1: divisors (random normals, all-ones mantissas, short mantissas, range limits) x every bf16 */
    #pragma omp parallel for reduction(+:bad,total,not_rn) schedule(dynamic, 16)
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
        for (uint32_t h = 0; h < 0x10000; h++) {
            if ((h & 0x7F80) == 0x7F80) continue;          /* inf / nan */
            float a = f_of(h << 16);
            if (!in_range(a, d)) continue;
            total++;
            bad += check(a, d, &not_rn);
        }
    }
    /* sweep 2: every bf16 numerator, every E2M1 midpoint, divisors within 64 ulps of |x| / m */
    const float mids[7] = {0.25f, 0.75f, 1.25f, 1.75f, 2.5f, 3.5f, 5.0f};
    #pragma omp parallel for reduction(+:tie_total,tie_bad,tie_not_rn) schedule(dynamic, 64)
    for (long h = 0; h < 0x10000; h++) {
        if ((h & 0x7F80) == 0x7F80) continue;
        float a = f_of((uint32_t)h << 16);
        if (a == 0.0f) continue;
        for (int k = 0; k < 7; k++) {
            float d0 = fabsf(a) / mids[k];
            for (int off = -64; off <= 64; off++) {
                float d = f_of(u_of(d0) + off);
                if (!in_range(a, d)) continue;
                tie_total++;
                tie_bad += check(a, d, &tie_not_rn);
            }
        }
    }
    printf("%ld %ld %ld %ld %ld %ld\n", total, bad, not_rn, tie_total, tie_bad, tie_not_rn);
    return 0;
}
"""


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_reciprocal_division_gives_ieee_codes(tmp_path):
    src = tmp_path / "div.c"
    exe = tmp_path / "div"
    src.write_text(SRC)
    flags = ["-O2", "-ffp-contract=off", "-mfma", "-fopenmp"]
    r = subprocess.run(["gcc", *flags, "-o", str(exe), str(src), "-lm"], capture_output=True, text=True)
    if r.returncode != 0:
        pytest.skip("host compiler without FMA/OpenMP support: " + r.stderr[-200:])
    env = dict(os.environ, OMP_NUM_THREADS=str(min(8, os.cpu_count() or 1)))
    out = subprocess.run([str(exe), "3000"], capture_output=True, text=True, env=env, timeout=600)
    total, bad, not_rn, tie_total, tie_bad, tie_not_rn = (int(v) for v in out.stdout.split())
    assert total > 10**8 and tie_total > 10**7
    # faithful everywhere, and the E2M1 codes always those of the IEEE quotient
    assert bad == 0 and tie_bad == 0
    # next to the E2M1 midpoints the quotient is the IEEE one
    assert tie_not_rn == 0
