"""Pins for the oracle's e4m3 codec, bf16 narrowing and per-row fp8 wire.

These check the oracle against things other than itself: the OCP E4M3 code
points, torch's independent float8_e4m3fn and bfloat16 casts, the exact
round trip on representable rows, and the relL2-by-granularity table that
"MORI GEMM + All-Reduce Benchmark" prints in "What fp8 costs, numerically".
"""
import math
import os

import numpy as np
import pytest
import torch

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_golden(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                rows.append(line.split())
    return rows


def _all_finite_bf16():
    b = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    return b[(b & 0x7F80) != 0x7F80]


def test_e4m3_code_points():
    for code, val in _read_golden("e4m3_points.txt"):
        v = oracle.e4m3_value(int(code, 16))
        if val == "nan":
            assert math.isnan(v), code
        else:
            assert v == float(val), (code, v, val)
            assert math.copysign(1.0, v) == math.copysign(1.0, float(val)), code


def test_e4m3_table_structure():
    t = oracle.e4m3_table()
    pos = t[:0x7F]
    assert np.all(np.diff(pos) > 0), "codes 0x00..0x7E must increase strictly"
    assert pos[-1] == 448.0
    neg = t[0x80:0xFF]
    assert np.array_equal(neg, -pos)
    finite = t[np.isfinite(t)]
    assert finite.size == 254
    assert np.unique(finite).size == 253  # +0 and -0 compare equal
    assert np.isnan(t[0x7F]) and np.isnan(t[0xFF])
    # 3 mantissa bits: within each binade the step is 1/8 of the binade's base
    for e in range(1, 16):
        for m in range(8):
            c = (e << 3) | m
            if c == 0x7F:
                continue
            assert t[c] == (1 + m / 8) * 2.0 ** (e - 7)


def test_encode_exhaustive_bf16_vs_torch():
    """O2 against torch's float8_e4m3fn cast (its own RNE encoder) on all finite
    bf16 inputs, at several scales, after clamping to +-448 (torch's cast
    does not saturate)."""
    b = _all_finite_bf16()
    x = oracle.bf16_to_f64(b).astype(np.float32)
    for s in [1.0, 2.0 ** -7, 0.0091, 3.3e-4, 1.0 / 448.0, 37.5]:
        with np.errstate(over="ignore"):
            v = x / np.float32(s)
        v = v[np.isfinite(v)]
        got = oracle.e4m3_codes(v)
        clamped = np.clip(v, -448.0, 448.0).astype(np.float32)
        ref = torch.from_numpy(clamped).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        bad = np.nonzero(got != ref)[0]
        assert bad.size == 0, (s, v[bad[:5]], got[bad[:5]], ref[bad[:5]])


def test_encode_ties_and_edges():
    c = oracle.e4m3_code
    assert c(1.0625) == 0x38          # midway 1 and 1.125 -> even (1.0)
    assert c(1.1875) == 0x3A          # midway 1.125 and 1.25 -> even (1.25)
    assert c(2.0 ** -10) == 0x00      # midway 0 and 2^-9 -> 0
    assert c(3 * 2.0 ** -10) == 0x02  # midway 2^-9 and 2^-8 -> 2^-8
    assert c(-2.0 ** -11) == 0x80     # negative, rounds to zero: sign kept
    assert c(-0.0) == 0x80 and c(0.0) == 0x00
    assert c(448.0) == 0x7E and c(-448.0) == 0xFE
    assert c(464.0) == 0x7E and c(1e30) == 0x7E and c(-3e38) == 0xFE  # saturate
    assert c(232.0) == 0x76           # midway 224 and 240 -> even (224)
    assert c(244.0) == 0x77 and c(248.0) == 0x78 and c(250.0) == 0x78
    assert c(float("nan")) == -1 and c(float("inf")) == -1


def test_bf16_rne_vs_torch():
    rng = np.random.default_rng(3)
    u = rng.integers(0, 2 ** 32, size=2_000_000, dtype=np.uint64).astype(np.uint32)
    # add exact ties (low half 0x8000) with odd and even kept halves
    ties = (rng.integers(0, 2 ** 16, size=200_000, dtype=np.uint64).astype(np.uint32) << 16) | 0x8000
    u = np.concatenate([u, ties, np.array([0x7F7FFFFF, 0x7F7F8000, 0xFF7F8000, 0x00008000,
                                           0x80018000, 0x3F808000, 0x3F818000], np.uint32)])
    x = u.view(np.float32)
    x = x[np.isfinite(x)]
    got = oracle.bf16_rne_array(x)
    ref = torch.from_numpy(x.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, (x.view(np.uint32)[bad[:5]], got[bad[:5]], ref[bad[:5]])
    assert oracle.bf16_rne(float("nan")) == 0x7FC0


def _representable_rows(rows, N, seed):
    """bf16 rows whose values are e4m3 codes times 2^e_row with a +-448 entry:
    then amax/448 = 2^e_row exactly and every quotient is a grid value."""
    rng = np.random.default_rng(seed)
    t = oracle.e4m3_table()
    finite_codes = np.array([c for c in range(256) if np.isfinite(t[c])])
    codes = rng.choice(finite_codes, size=(rows, N))
    pos = rng.integers(0, N, size=rows)
    codes[np.arange(rows), pos] = rng.choice([0x7E, 0xFE], size=rows)
    e = rng.integers(-20, 20, size=rows)
    vals = t[codes] * (2.0 ** e)[:, None]
    b = oracle.bf16_rne_array(vals.astype(np.float32))
    assert np.array_equal(oracle.bf16_to_f64(b), vals)  # exact in bf16 by construction
    return b, codes.astype(np.uint8), (2.0 ** e).astype(np.float32)


def test_rowq_rowdq_exact_on_representable_rows():
    b, codes, scales = _representable_rows(64, 512, 11)
    q, s = oracle.rowq(b)
    assert np.array_equal(s, scales)
    assert np.array_equal(q, codes)
    y = oracle.rowdq(q, s)
    assert np.array_equal(y, b)


def test_rowq_amax_code_and_zero_rows():
    x = synth.wire_rows(32, 1024, seed=5)
    x[3] = 0
    x[7] = 0x8000  # all -0
    q, s = oracle.rowq(x)
    for r in range(32):
        if r in (3, 7):
            assert s[r] == 0 and np.all(q[r] == 0)
        else:
            assert np.any((q[r] == 0x7E) | (q[r] == 0xFE)), r
            amax = np.max(np.abs(oracle.bf16_to_f64(x[r])))
            assert s[r] == np.float32(np.float32(amax) / np.float32(448.0))


def test_rowq_scale_invariance_power_of_two():
    x = synth.wire_rows(16, 896, seed=9)
    q, s = oracle.rowq(x)
    x2 = oracle.bf16_rne_array((oracle.bf16_to_f64(x) * 8.0).astype(np.float32))
    q2, s2 = oracle.rowq(x2)
    assert np.array_equal(q, q2) and np.array_equal(s2, s * np.float32(8.0))


def test_fp8_wire_granularity_table():
    """relL2 of the round trip on a [2048,7168] N(0,1) payload, per row and per
    group of 512/256/128/32, against the pages' table (statistical pin: the
    pages' draw is not ours; this draw lands within 0.25% of every entry, and
    the bound is 0.5%)."""
    table = {int(w): float(v) for w, v in _read_golden("fp8_wire_granularity.txt")}
    x = synth.wire_rows(2048, 7168, seed=200)
    xf = oracle.bf16_to_f64(x)
    t = oracle.e4m3_table()
    for w, ref in table.items():
        if w == 7168:
            q, s = oracle.rowq(x)
            y = oracle.bf16_to_f64(oracle.rowdq(q, s))
        else:
            q, s = oracle.quant_blocks(xf.astype(np.float32), 1, w)
            y = t[q] * np.repeat(s.astype(np.float64), w, axis=1)
        r = oracle.rel_l2(y, xf)
        assert abs(r / ref - 1) < 0.005, (w, r, ref)


@pytest.mark.parametrize("heavy_rows", [False, True])
def test_rowq_vs_torch_quotient_cast(heavy_rows):
    """O7 on full [2048, 7168] rows against an independent formulation in
    torch: amax per row in fp32, s = amax / 448 (fp32 division), codes =
    float8_e4m3fn cast of the fp32 quotient x / s clamped to +-448 (torch's
    cast rounds to nearest even but does not saturate).  A quotient taken as
    x * (448 / amax), or a scale of 448 / amax, would differ on many codes."""
    rows, N = 2048, 7168
    x = synth.wire_rows(rows, N, seed=300)
    if heavy_rows:
        # rows spread over many binades, some with tiny or huge amax
        xf = (x.astype(np.uint32) << 16).view(np.float32)
        mult = np.exp2(np.random.default_rng(5).integers(-60, 60, rows)).astype(np.float32)
        x = oracle.bf16_rne_array(xf * mult[:, None])
    q, s = oracle.rowq(x)
    xt = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).float()
    amax = xt.abs().amax(dim=1)
    st = amax / 448.0
    qt = (xt / st[:, None]).clamp(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(s.view(np.uint32), st.numpy().view(np.uint32))
    assert np.array_equal(q, qt)
    # the multiply-by-reciprocal formulation is not the same function
    qm = (xt * (448.0 / amax)[:, None]).clamp(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.count_nonzero(qm != q) > 0
