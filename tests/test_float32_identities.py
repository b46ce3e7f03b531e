"""The float32 identities the quantizer kernels rely on, checked on the host
with the same IEEE single-precision operations (C, fused multiply-add from
libm), against correctly rounded references.

* d / L in three operations: q0 = RN(d / L's reciprocal product), the exact
  residual e = fma(-q0, L, d), q1 = fma(e, 1/L, q0). The kernels take it for
  the scale (max - min) / L with L = 15 or 255 and d the float32 difference
  of two fp16 numbers (0 <= d <= 131008). Reference: (float)((double)d / L),
  which is the correctly rounded quotient (d / L never lies within 2^-53 of
  a float32 midpoint for these L). The full range (every float32 d in
  [0, 2^17]) was checked once, 1.2e9 values per L; this test walks it with a
  stride plus the edges.
* rint(x / s) for fp16 x and s from the reciprocal product with one
  correction step (inv within one ulp of 1/s: both the correctly rounded
  reciprocal and its neighbours are tried), against the exact quotient's
  rint in float64, over every fp16 x for a set of fp16 scales.
"""
import os
import shutil
import subprocess
import tempfile

import numpy as np
import pytest

SRC = r"""
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>
static float f32(uint32_t u) { float x; memcpy(&x, &u, 4); return x; }
static uint32_t bits(float x) { uint32_t u; memcpy(&u, &x, 4); return u; }
int main(int argc, char **argv) {
    long bad = 0, n = 0;
    const int Ls[2] = {15, 255};
    for (int li = 0; li < 2; ++li) {
        const float L = (float)Ls[li], rL = 1.0f / L;
        for (uint64_t u = 0; u <= 0x48000000u; u += (u < 4096 || u > 0x47FFF000u) ? 1 : 97) {
            const float d = f32((uint32_t)u);
            const float q0 = d * rL;
            const float e = fmaf(-q0, L, d);
            const float q1 = fmaf(e, rL, q0);
            const float ref = (float)((double)d / (double)Ls[li]);
            ++n;
            if (bits(q1) != bits(ref)) ++bad;
        }
    }
    printf("%ld %ld\n", n, bad);
    return 0;
}
"""

SRC_Q = r"""
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>
/* stdin: count, then count lines "x s" (float32 values of fp16 numbers) and
   the expected rint; prints the number of mismatches over three reciprocals */
int main(void) {
    long n, bad = 0;
    if (scanf("%ld", &n) != 1) return 1;
    for (long i = 0; i < n; ++i) {
        float x, s; double want;
        if (scanf("%a %a %lf", &x, &s, &want) != 3) return 1;
        const float r0 = 1.0f / s;
        const float rs[3] = {nextafterf(r0, 0.0f), r0, nextafterf(r0, INFINITY)};
        for (int k = 0; k < 3; ++k) {
            const float inv = rs[k];
            const float p = x * inv;
            const float r = fmaf(-p, s, x);
            const float q = fmaf(r, inv, p);
            const float y = q + 12582912.0f;
            if ((double)y - 12582912.0 != want) ++bad;
        }
    }
    printf("%ld\n", bad);
    return 0;
}
"""


def _build(src, tmp, name):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    c = os.path.join(tmp, name + ".c")
    exe = os.path.join(tmp, name)
    with open(c, "w") as fh:
        fh.write(src)
    subprocess.run(["gcc", "-O2", "-ffp-contract=off", c, "-o", exe, "-lm"], check=True)
    return exe


def test_division_by_the_step_count_in_three_operations():
    with tempfile.TemporaryDirectory() as tmp:
        exe = _build(SRC, tmp, "divsteps")
        n, bad = map(int, subprocess.run([exe], check=True, capture_output=True, text=True).stdout.split())
    assert n > 20_000_000 and bad == 0


def test_rint_of_fp16_quotients_from_the_corrected_reciprocal_product():
    # every finite fp16 x against 24 fp16 scales (normal, small to large),
    # |x / s| kept below 2^12 as the kernels' clamps need
    xs = np.arange(0, 0x10000, dtype=np.uint32).astype(np.uint16).view(np.float16)
    xs = xs[np.isfinite(xs)].astype(np.float64)
    rng = np.random.default_rng(3)
    scales = np.concatenate([np.float16([2.0 ** -14, 1e-3, 0.0135, 0.125, 1.0, 3.0, 7.0, 4368.0]),
                             np.float16(np.exp2(rng.uniform(-14, 12, size=16)))]).astype(np.float64)
    lines = []
    for s in scales:
        q = xs / s
        keep = np.abs(q) < 4096
        for x, want in zip(xs[keep], np.rint(q[keep])):
            lines.append(f"{float(np.float32(x)).hex()} {float(np.float32(s)).hex()} {want:.1f}")
    with tempfile.TemporaryDirectory() as tmp:
        exe = _build(SRC_Q, tmp, "rintq")
        out = subprocess.run([exe], input=f"{len(lines)}\n" + "\n".join(lines) + "\n", check=True,
                             capture_output=True, text=True).stdout
    assert len(lines) > 500_000 and int(out) == 0
