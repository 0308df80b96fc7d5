"""Host build of the HIP path's quantizer division (``wire_quotient`` in
csrc/codec.hpp): for every pair of bf16 values (x, amax) with |x| <= amax and
scale s = fl32(amax / 448) > 0, the fp64-reciprocal quotient the kernels use
must equal IEEE fp32 division x / s bit for bit.  This is the whole domain the
per-row quantizer can meet (about 1.07e9 pairs), so the e4m3 decision the
device takes is the one the definition takes."""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "block_scaled_fp8_bsgemm_amd", "csrc")

PROGRAM = r"""
#include <cstdio>
#include <cstdint>
#include <cstring>
#include "codec.hpp"
static float bf(uint32_t b) { uint32_t u = b << 16; float f; std::memcpy(&f, &u, 4); return f; }
int main() {
    unsigned long long pairs = 0, bad = 0;
#pragma omp parallel for schedule(dynamic, 16) reduction(+ : pairs, bad)
    for (int ab = 1; ab < 0x7F80; ab++) {
        const float s = bf(ab) / 448.0f;
        if (s == 0.0f) continue;
        const double R = 1.0 / (double)s;
        for (int xb = 0; xb <= ab; xb++)
            for (int sg = 0; sg < 2; sg++) {
                const float x = bf(xb | (sg << 15));
                const float a = x / s, b = wire_quotient(x, R);
                uint32_t ua, ub;
                std::memcpy(&ua, &a, 4);
                std::memcpy(&ub, &b, 4);
                pairs++;
                if (ua != ub) bad++;
            }
    }
    std::printf("%llu %llu\n", pairs, bad);
    return 0;
}
"""


def test_wire_quotient_equals_ieee_division(tmp_path):
    src = tmp_path / "q.cpp"
    exe = tmp_path / "q"
    src.write_text(PROGRAM)
    subprocess.run(["g++", "-O2", "-std=c++17", "-fopenmp", "-ffp-contract=off", "-I", CSRC,
                    str(src), "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True, timeout=600).stdout
    pairs, bad = map(int, out.split())
    assert pairs > 1_000_000_000
    assert bad == 0


def test_bf16_quotients_stay_below_the_e4m3_overflow_midpoint():
    """The quantizers of bf16 data convert quotients without clamping them:
    for every finite nonzero bf16 amax and s = fl32(amax / 448), the largest
    quotient the kernels form, wire_quotient(amax, 1 / s), stays below 464
    (the midpoint between 448 and the next e4m3 step).  It exceeds 448 only by
    the rounding of s: one fp32 step (448 + 2^-15) while s is normal, up to
    448.88 where s is subnormal.  Those amax values are the ones the device
    test feeds the row quantizer (test_gpu_stream.py)."""
    import numpy as np
    b = np.arange(1, 0x7F80, dtype=np.uint32)
    amax = (b << 16).view(np.float32)
    s = amax / np.float32(448.0)
    assert np.all(s > 0)
    q = (amax.astype(np.float64) * (1.0 / s.astype(np.float64))).astype(np.float32)
    assert q.max() < 464.0 and q.max() < 449.0, q.max()
    normal = s >= np.float32(2.0 ** -126)
    assert q[normal].max() == np.float32(448.0 + 2.0 ** -15)
    assert np.count_nonzero(q > 448.0) > 1000
