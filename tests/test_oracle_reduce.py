"""Pins for the oracle's band reduce (O6): the exact (float64) sum of the P
bf16 parts, rounded once to bf16, must agree with the fp32 index-ordered sum
except where fp32 rounding of a partial sum can move the value across a bf16
rounding midpoint; plus exact special cases."""
import numpy as np

import oracle
import synth


def test_band_reduce_vs_exact_sum():
    parts = synth.partial_bands(256, 7168, P=8, seed0=100)
    out = oracle.band_reduce(parts)
    X = np.stack([oracle.bf16_to_f64(p) for p in parts])
    exact = X.sum(axis=0)  # exact: 8 bf16 values of similar magnitude fit in 53 bits
    ref = oracle.bf16_rne_array(exact.astype(np.float32))
    diff = out != ref
    # allowed only within the fp32 partial-sum error of a bf16 midpoint
    absum = np.abs(X).sum(axis=0)
    a = np.abs(exact)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    ulp = 2.0 ** (np.maximum(e, -126) - 7)
    f = a / ulp
    mid_dist = np.abs(f - np.floor(f) - 0.5) * ulp
    assert np.all(mid_dist[diff] <= 8 * 2.0 ** -24 * absum[diff])
    assert diff.mean() < 1e-3
    # differing outputs are one bf16 step apart
    assert np.all(np.abs(out[diff].astype(np.int32) - ref[diff].astype(np.int32)) <= 1)


def test_band_reduce_identical_parts_scale_exactly():
    x = synth.wire_rows(64, 1024, seed=1)
    out = oracle.band_reduce([x] * 8)
    assert np.array_equal(oracle.bf16_to_f64(out), 8 * oracle.bf16_to_f64(x))


def test_band_reduce_single_part_identity_and_zero_sign():
    x = synth.wire_rows(16, 512, seed=2)
    assert np.array_equal(oracle.band_reduce([x]), x)
    negz = np.full((4, 64), 0x8000, np.uint16)
    # the sum starts from +0.0, so a sum of -0 parts is +0
    assert np.all(oracle.band_reduce([negz, negz]) == 0x0000)


def test_band_reduce_cancellation_order():
    """Index order matters in fp32: (big + 1) - big = 0 at bf16/fp32 widths
    where big = 2^25, while the exact sum is 1."""
    big = oracle.bf16_rne(2.0 ** 25)
    nbig = big | 0x8000
    one = oracle.bf16_rne(1.0)
    p0 = np.full((1, 8), big, np.uint16)
    p1 = np.full((1, 8), one, np.uint16)
    p2 = np.full((1, 8), nbig, np.uint16)
    assert np.all(oracle.band_reduce([p0, p1, p2]) == 0)
    assert np.all(oracle.band_reduce([p0, p2, p1]) == one)
