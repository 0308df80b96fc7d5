"""GPU parity of band_reduce, rowq_e4m3, rowdq_e4m3, blockq_e4m3 and
actq_e4m3 against the oracle (O6, O7, O8, O3; actq is O3 with 1x128 blocks on
the fp32 values of bf16 inputs).  All of these are bit-exact: the device takes
the same fp32 decisions in the same order as the definition."""
import numpy as np
import pytest
import torch

import block_scaled_fp8_bsgemm_amd as bs
import oracle
import synth
from gpuutil import bf16_dev, bits16, device, poison_bf16, poison_u8, say, to_dev

pytestmark = pytest.mark.gpu


# ------------------------------------------------------------------ reduce --

@pytest.mark.parametrize("rows,N,P", [(2048, 7168, 8), (37, 104, 3), (5, 8, 1), (64, 1024, 16), (130, 7168, 8)])
def test_band_reduce_bitexact(rows, N, P):
    say(f"band_reduce rows={rows} N={N} P={P}")
    parts = synth.partial_bands(rows, N, P=P, seed0=100)
    ref = oracle.band_reduce(parts)
    out = poison_bf16(torch.empty((rows, N), dtype=torch.bfloat16, device=device()))
    bs.band_reduce([bf16_dev(p) for p in parts], out)
    torch.cuda.synchronize()
    assert np.array_equal(bits16(out), ref)


def test_band_reduce_order_and_zero_sign():
    one = oracle.bf16_rne(1.0)
    big = oracle.bf16_rne(2.0 ** 25)
    parts = [np.full((4, 64), v, np.uint16) for v in (big, one, big | 0x8000)]
    negz = [np.full((4, 64), 0x8000, np.uint16)] * 2
    say("band_reduce order / -0")
    out = bs.band_reduce([bf16_dev(p) for p in parts])
    out2 = bs.band_reduce([bf16_dev(p) for p in negz])
    torch.cuda.synchronize()
    assert np.array_equal(bits16(out), oracle.band_reduce(parts))
    assert np.all(bits16(out) == 0)
    assert np.all(bits16(out2) == 0)


# ---------------------------------------------------------------- row codec --

def rowq_dev(x_bits):
    rows, N = x_bits.shape
    q = poison_u8(torch.empty((rows, N), dtype=torch.uint8, device=device()))
    s = torch.full((rows,), float("nan"), dtype=torch.float32, device=device())
    bs.rowq_e4m3(bf16_dev(x_bits), q, s)
    torch.cuda.synchronize()
    return q.cpu().numpy(), s.cpu().numpy()


@pytest.mark.parametrize("rows,N", [(2048, 7168), (3, 8), (17, 2056), (2, 40960),
                                    (5, 2048), (9, 4096), (6, 8192), (3, 16384), (4, 7160)])
def test_rowq_bitexact(rows, N):
    say(f"rowq_e4m3 rows={rows} N={N}")
    x = synth.wire_rows(rows, N, seed=200)
    qr, sr = oracle.rowq(x)
    q, s = rowq_dev(x)
    assert np.array_equal(s.view(np.uint32), sr.view(np.uint32))
    assert np.array_equal(q, qr)


@pytest.mark.parametrize("N", [8, 2048, 2056, 4096, 7168, 8192, 16384, 16392])
def test_rowq_zero_and_negative_zero_rows(N):
    """All-zero and all -0 rows get scale 0 and +0 codes on every kernel shape
    (full rows of 64 * CPL packs, guarded rows, long rows)."""
    say(f"rowq_e4m3 zero rows N={N}")
    x = synth.wire_rows(6, N, seed=201)
    x[1] = 0
    x[3] = 0x8000
    x[4, ::2] = 0x8000
    x[4, 1::2] = 0
    qr, sr = oracle.rowq(x)
    assert sr[1] == 0 and sr[3] == 0 and sr[4] == 0 and not np.any(qr[[1, 3, 4]])
    q, s = rowq_dev(x)
    assert np.array_equal(s.view(np.uint32), sr.view(np.uint32))
    assert np.array_equal(q, qr)


def exhaustive_rows():
    """Rows holding every finite bf16 value up to a chosen amax, for amax over
    many binades (including amax whose scale amax/448 is an fp32 subnormal or
    underflows to zero), plus zero, -0 and single-entry rows."""
    b = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    b = b[(b & 0x7F80) != 0x7F80]
    mag = b & 0x7FFF
    amaxes = [0x0001, 0x0005, 0x0080, 0x0100, 0x2F55, 0x3F80, 0x3FC1, 0x4480, 0x43E0, 0x6000, 0x7F7F]
    rows = []
    width = b.size + 8
    for a in amaxes:
        sel = b[mag <= a]
        row = np.zeros(width, np.uint16)
        row[: sel.size] = sel
        row[-1] = a
        rows.append(row)
    rows.append(np.zeros(width, np.uint16))
    rows.append(np.full(width, 0x8000, np.uint16))
    single = np.zeros(width, np.uint16)
    single[123] = 0xC2F7
    rows.append(single)
    return np.stack(rows)


def test_rowq_exhaustive_bf16():
    x = exhaustive_rows()
    say(f"rowq_e4m3 exhaustive {x.shape}")
    qr, sr = oracle.rowq(x)
    q, s = rowq_dev(x)
    assert np.array_equal(s.view(np.uint32), sr.view(np.uint32))
    bad = np.argwhere(q != qr)
    assert bad.size == 0, [(int(r), int(c), hex(x[r, c]), hex(q[r, c]), hex(qr[r, c])) for r, c in bad[:8]]


def overflow_edge_rows(cols=128):
    """One row per bf16 amax whose largest quotient x / s lands above 448
    (3217 of them: s = fl32(amax / 448) rounded down; up to 448.88 where s is
    subnormal): +-amax at both ends of the row, random smaller values between.
    The quantizers convert these quotients without a clamp."""
    b = np.arange(1, 0x7F80, dtype=np.uint32)
    amax = (b << 16).view(np.float32)
    q = (amax.astype(np.float64) * (1.0 / (amax / np.float32(448.0)).astype(np.float64))).astype(np.float32)
    over = b[q > 448.0].astype(np.uint16)
    rng = np.random.default_rng(17)
    frac = rng.random((over.size, cols)).astype(np.float32)
    mag = (over.astype(np.uint32) << 16).view(np.float32)
    rows = oracle.bf16_rne_array(frac * mag[:, None])
    rows = np.minimum(rows & 0x7FFF, over[:, None]) | (rows & 0x8000)
    rows[:, 0] = over
    rows[:, -1] = over | 0x8000
    return rows.astype(np.uint16)


@pytest.mark.parametrize("cols", [128, 2048])
def test_quantizers_at_the_e4m3_edge(cols):
    """Rows whose largest quotient exceeds 448 by the rounding of the scale:
    the row, activation (1x128) and fused reduce + row quantizers give the
    oracle's (saturating) codes, +-448 at the extremes, with no NaN code."""
    x = overflow_edge_rows(cols)
    say(f"quantizers at the e4m3 edge {x.shape}")
    qr, sr = oracle.rowq(x)
    assert np.all(qr[:, 0] == 0x7E) and np.all(qr[:, -1] == 0xFE)
    q, s = rowq_dev(x)
    assert np.array_equal(s.view(np.uint32), sr.view(np.uint32))
    assert np.array_equal(q, qr)
    x32 = (x.astype(np.uint32) << 16).view(np.float32)
    qa_r, sa_r = oracle.quant_blocks(x32, 1, 128)
    qa, sa = bs.actq_e4m3(bf16_dev(x))
    qf = poison_u8(torch.empty(x.shape, dtype=torch.uint8, device=device()))
    sf = torch.full((x.shape[0],), float("nan"), dtype=torch.float32, device=device())
    bs.band_rowq_e4m3([bf16_dev(x)], qf, sf)
    torch.cuda.synchronize()
    assert np.array_equal(qa.cpu().numpy(), qa_r)
    assert np.array_equal(sa.cpu().numpy().view(np.uint32), sa_r.view(np.uint32))
    assert np.array_equal(qf.cpu().numpy(), qr)
    assert np.array_equal(sf.cpu().numpy().view(np.uint32), sr.view(np.uint32))


@pytest.mark.parametrize("rows,N", [(16384, 7168), (7, 24), (3, 33000)])
def test_rowdq_bitexact(rows, N):
    say(f"rowdq_e4m3 rows={rows} N={N}")
    x = synth.wire_rows(rows, N, seed=200)
    q, s = oracle.rowq(x)
    ref = oracle.rowdq(q, s)
    y = poison_bf16(torch.empty((rows, N), dtype=torch.bfloat16, device=device()))
    bs.rowdq_e4m3(to_dev(q), to_dev(s), y)
    torch.cuda.synchronize()
    assert np.array_equal(bits16(y), ref)


def test_rowdq_every_code_and_scale():
    t = oracle.e4m3_table()
    codes = np.array([c for c in range(256) if np.isfinite(t[c])], np.uint8)
    scales = np.array([1.0, 2.0 ** -9, 0.0091, 3.3e-4, 7.5e35, 1e-40, 0.0, 1.1754944e-38, 123.456], np.float32)
    q = np.tile(np.resize(codes, 256), (scales.size, 1))
    say("rowdq_e4m3 all codes x scales")
    ref = oracle.rowdq(q, scales)
    y = bs.rowdq_e4m3(to_dev(q), to_dev(scales))
    torch.cuda.synchronize()
    assert np.array_equal(bits16(y), ref)


def test_rowq_rowdq_roundtrip_exact_on_grid_rows():
    """rows of e4m3 grid values times 2^e with a +-448 entry survive the round
    trip bit for bit"""
    rng = np.random.default_rng(11)
    t = oracle.e4m3_table()
    finite = np.array([c for c in range(256) if np.isfinite(t[c])])
    codes = rng.choice(finite, size=(64, 512))
    codes[np.arange(64), rng.integers(0, 512, 64)] = rng.choice([0x7E, 0xFE], size=64)
    vals = t[codes] * (2.0 ** rng.integers(-20, 20, size=64))[:, None]
    x = oracle.bf16_rne_array(vals.astype(np.float32))
    say("rowq/rowdq grid round trip")
    q, s = rowq_dev(x)
    assert np.array_equal(q, codes.astype(np.uint8))
    y = bs.rowdq_e4m3(to_dev(q), to_dev(s))
    torch.cuda.synchronize()
    assert np.array_equal(bits16(y), x)


# ---------------------------------------------------------- block quantizer --

@pytest.mark.parametrize("rows,cols,br", [(256, 256, 1), (300, 640, 1), (4096, 2048, 1),
                                          (256, 512, 128), (300, 384, 128), (7168, 2048, 128)])
def test_blockq_bitexact(rows, cols, br):
    say(f"blockq_e4m3 rows={rows} cols={cols} block_rows={br}")
    x = synth.operand_fp32(rows, 128, cols, seed=5, heavy=True)[0]   # [rows, cols]
    x[min(3, rows - 1), :128] = 0.0            # a zero block (1x128 case)
    qr, sr = oracle.quant_blocks(x, br, 128)
    q, s = bs.blockq_e4m3(to_dev(x), br)
    torch.cuda.synchronize()
    assert np.array_equal(s.cpu().numpy().view(np.uint32), sr.view(np.uint32))
    assert np.array_equal(q.cpu().numpy(), qr)


# ------------------------------------------------------ activation quantizer --

@pytest.mark.parametrize("rows,cols", [(256, 256), (300, 640), (1, 128), (4096, 2048), (16384, 2048)])
def test_actq_bitexact(rows, cols):
    say(f"actq_e4m3 rows={rows} cols={cols}")
    a = synth.operand_fp32(rows, 128, cols, seed=11, heavy=True)[0]   # [rows, cols]
    bits = oracle.bf16_rne_array(a)
    bits[min(3, rows - 1), :128] = 0                      # a zero block
    bits[min(5, rows - 1), 128 * (cols // 128 - 1):] = 0x8000   # a block of -0
    x32 = (bits.astype(np.uint32) << 16).view(np.float32)
    qr, sr = oracle.quant_blocks(x32, 1, 128)
    q = poison_u8(torch.empty((rows, cols), dtype=torch.uint8, device=device()))
    q, s = bs.actq_e4m3(bf16_dev(bits), q)
    torch.cuda.synchronize()
    assert np.array_equal(s.cpu().numpy().view(np.uint32), sr.view(np.uint32))
    assert np.array_equal(q.cpu().numpy(), qr)


def test_actq_matches_blockq():
    """The same values through the bf16 and the fp32 quantizer give the same codes."""
    rows, cols = 512, 1024
    a = synth.operand_fp32(rows, 128, cols, seed=12, heavy=True)[0]
    bits = oracle.bf16_rne_array(a)
    x32 = (bits.astype(np.uint32) << 16).view(np.float32)
    say("actq vs blockq")
    q1, s1 = bs.actq_e4m3(bf16_dev(bits))
    q2, s2 = bs.blockq_e4m3(to_dev(x32), 1)
    torch.cuda.synchronize()
    assert torch.equal(q1, q2) and torch.equal(s1.view(torch.int32), s2.view(torch.int32))


@pytest.mark.parametrize("rows,N,P", [(2048, 7168, 8), (37, 104, 3), (5, 8, 1), (130, 8192, 16), (64, 2048, 8),
                                      (300, 7168, 5), (17, 1024, 13), (2048, 7168, 7), (9, 2056, 6)])
def test_band_rowq_bitexact(rows, N, P):
    """The fused reduce + row quantize equals the oracle's row quantize of its
    band reduce, and the device's two separate kernels, bit for bit.  The
    kernel reads the parts four at a time, so P = 5, 6, 7, 13 end on a partial
    group; N = 2056 gives one lane a pack past the first 256."""
    say(f"band_rowq_e4m3 rows={rows} N={N} P={P}")
    parts = synth.partial_bands(rows, N, P=P, seed0=300)
    parts[0][min(2, rows - 1)] = 0                    # a zero row in one part only
    if P > 1:
        for p in parts:
            p[rows - 1] = 0                           # a row that sums to +0
    red_ref = oracle.band_reduce(parts)
    q_ref, s_ref = oracle.rowq(red_ref)
    dparts = [bf16_dev(p) for p in parts]
    q = poison_u8(torch.empty((rows, N), dtype=torch.uint8, device=device()))
    s = torch.full((rows,), float("nan"), dtype=torch.float32, device=device())
    bs.band_rowq_e4m3(dparts, q, s)
    q2, s2 = bs.rowq_e4m3(bs.band_reduce(dparts))
    torch.cuda.synchronize()
    assert np.array_equal(q.cpu().numpy(), q_ref)
    assert np.array_equal(s.cpu().numpy().view(np.uint32), s_ref.view(np.uint32))
    assert torch.equal(q, q2) and torch.equal(s.view(torch.int32), s2.view(torch.int32))
