"""GPU parity of the mxfp8 variant against the oracle: mxq_e4m3 (O10, the
32-wide E8M0 operand quantizer) bit for bit, and mxgemm_fp8 against the
exact mxfp8 product O11, every element inside the interval the scaled
MFMA's truncation and rounding allow (gpuutil.mx_accept); band layout
bitwise.

Inputs are the seeded synthetic operands; the GEMM tests quantize them with
the oracle's O10 so that both sides consume the same bytes, and one test runs
the device quantizer into the device GEMM."""
import numpy as np
import pytest
import torch

import block_scaled_fp8_bsgemm_amd as bs
import oracle
import synth
from gpuutil import bf16_dev, bits16, device, mx_accept, poison_bf16, poison_u8, say, to_dev

pytestmark = pytest.mark.gpu


def operands(M, N, K, seed=0, heavy=False):
    A, B = synth.operand_fp32(M, N, K, seed=seed, heavy=heavy)
    qa, ea = oracle.mx_quant(A)
    qb, eb = oracle.mx_quant(B)
    return qa, ea, qb, eb


def run(qa, ea, qb, eb, bands=1, band_stride=0, C=None):
    M, N = qa.shape[0], qb.shape[0]
    if C is None:
        band_rows = M // bands
        stride = band_stride or band_rows * N
        C = poison_bf16(torch.empty((bands - 1) * stride + band_rows * N, dtype=torch.bfloat16, device=device()))
    bs.mxgemm_fp8(to_dev(qa), to_dev(ea), to_dev(qb), to_dev(eb), C, bands=bands, band_stride=band_stride)
    torch.cuda.synchronize()
    return C


# ---------------------------------------------------------------- mxq_e4m3 --

@pytest.mark.parametrize("rows,cols", [(1, 32), (3, 96), (257, 2048), (64, 7168), (16384, 2048)])
def test_mxq_bitexact(rows, cols):
    say(f"mxq_e4m3 rows={rows} cols={cols}")
    a = synth.operand_fp32(rows, 128, cols, seed=21, heavy=True)[0]
    bits = oracle.bf16_rne_array(a)
    bits[min(2, rows - 1), :32] = 0                              # a zero block
    bits[min(1, rows - 1), cols - 32:] = 0x8000                  # a block of -0
    if cols >= 96:
        r = min(4, rows - 1)
        bits[r, 32:64] = 0x0001                                  # bf16 subnormals: scale clamps at 2^-127
        bits[r, 64] = 0x43E0                                     # 448: exactly a power of two of 448
    x32 = (bits.astype(np.uint32) << 16).view(np.float32)
    qr, er = oracle.mx_quant(x32)
    q = poison_u8(torch.empty((rows, cols), dtype=torch.uint8, device=device()))
    e = torch.full((rows, cols // 32), 0xAA, dtype=torch.uint8, device=device())
    bs.mxq_e4m3(bf16_dev(bits), q, e)
    torch.cuda.synchronize()
    assert np.array_equal(e.cpu().numpy(), er)
    assert np.array_equal(q.cpu().numpy(), qr)


# -------------------------------------------------------------- mxgemm_fp8 --

@pytest.mark.parametrize("M,N,K,heavy", [
    (256, 512, 256, False),
    (640, 640, 512, True),       # ragged M tile, 128-wide N tail
    (300, 384, 384, False),      # M not a multiple of 128, odd K-block count
    (16, 128, 128, False),       # one K block, one partial tile
    (513, 1024, 1152, True),     # 9 K blocks, ragged by one row
])
def test_mxgemm_full_vs_oracle(M, N, K, heavy):
    say(f"mxgemm_fp8 M={M} N={N} K={K} heavy={heavy}")
    qa, ea, qb, eb = operands(M, N, K, seed=1, heavy=heavy)
    C = run(qa, ea, qb, eb)
    mx_accept(bits16(C).reshape(M, N), qa, ea, qb, eb, f"mx M={M} N={N} K={K}")


def test_mxgemm_many_tiles_vs_oracle():
    """289 tiles, more than the chip has CUs: workgroups of the persistent
    kernel (K / 128 even) run two tiles each; ragged last M tile and 1063-row
    bands that begin inside tiles.  Element by element against the oracle."""
    M, N, K, bands = 4252, 4352, 256, 4
    say(f"mxgemm_fp8 many tiles M={M} N={N} K={K} bands={bands}")
    qa, ea, qb, eb = operands(M, N, K, seed=8, heavy=True)
    C = run(qa, ea, qb, eb, bands=bands)
    mx_accept(bits16(C).reshape(M, N), qa, ea, qb, eb, f"mx many tiles M={M}")


@pytest.mark.parametrize("M,bands,pad", [(8292, 1, 0), (8192, 4, 64)])
def test_mxgemm_persistent_tile_transitions(M, bands, pad):
    """The persistent kernel stores a plain tile behind the next tile's DMA
    and lets those stores drain under its first K block; other tiles store
    at once.  M = 8292: 33 x 17 tiles, about 2.2 per workgroup, the last
    M-tile ragged, so workgroups pass between plain and ragged tiles in both
    orders; M = 8192 with padded bands: no tile is plain.  Every element
    against the exact product, and the band gaps untouched."""
    N, K = 4352, 256
    qa, ea, qb, eb = operands(M, N, K, seed=12, heavy=True)
    say(f"mxgemm_fp8 tile transitions M={M} bands={bands} pad={pad}")
    band_rows = M // bands
    stride = band_rows * N + pad
    C = torch.empty((bands - 1) * stride + band_rows * N + pad, dtype=torch.bfloat16, device=device())
    C.view(torch.int16).fill_(0x5A5A)
    run(qa, ea, qb, eb, bands=bands, band_stride=stride if pad else 0, C=C)
    raw = bits16(C)
    got = np.concatenate([raw[d * stride: d * stride + band_rows * N] for d in range(bands)]).reshape(M, N)
    mx_accept(got, qa, ea, qb, eb, f"mx tile transitions M={M} bands={bands} pad={pad}", model=False)
    if pad:
        for d in range(bands):
            assert np.all(raw[d * stride + band_rows * N: (d + 1) * stride] == 0x5A5A)


def test_mxgemm_unit_scales_exact():
    """Small codes, every scale byte 127: all sums are exact in fp32, so the
    device result equals the oracle bit for bit."""
    rng = np.random.default_rng(2)
    t = oracle.e4m3_table()
    small = np.array([c for c in range(256) if np.isfinite(t[c]) and abs(t[c]) <= 4 and (t[c] * 2) % 1 == 0])
    M, N, K = 256, 256, 512
    qa = rng.choice(small, size=(M, K)).astype(np.uint8)
    qb = rng.choice(small, size=(N, K)).astype(np.uint8)
    ea = np.full((M, K // 32), 127, np.uint8)
    eb = np.full((N, K // 32), 127, np.uint8)
    say("mxgemm_fp8 unit scales exact")
    _, ref = oracle.mxgemm(qa, ea, qb, eb)
    assert np.array_equal(bits16(run(qa, ea, qb, eb)).reshape(M, N), ref)


def test_mxgemm_scale_indexing():
    """Scale bytes that differ per 32-block and per row on both sides, with
    codes whose products are exact: a swapped or shifted scale index changes
    the result by a power of two somewhere."""
    rng = np.random.default_rng(3)
    M, N, K = 128, 256, 384
    qa = rng.choice([0x38, 0xB8, 0x30, 0x40, 0x00], size=(M, K)).astype(np.uint8)   # +-1, 0.5, 2, 0
    qb = rng.choice([0x38, 0xB8, 0x40], size=(N, K)).astype(np.uint8)
    ea = rng.integers(124, 131, size=(M, K // 32)).astype(np.uint8)
    eb = rng.integers(124, 131, size=(N, K // 32)).astype(np.uint8)
    say("mxgemm_fp8 scale indexing")
    acc, ref = oracle.mxgemm(qa, ea, qb, eb)
    _, ref_m = oracle.mxgemm(qa, ea, qb, eb, mfma=True)
    assert np.array_equal(ref, ref_m)      # no truncation with these codes
    got = bits16(run(qa, ea, qb, eb)).reshape(M, N)
    assert np.array_equal(got, ref)


def test_mxgemm_band_layout():
    M, N, K, bands, pad = 1024, 512, 256, 4, 72
    qa, ea, qb, eb = operands(M, N, K, seed=4)
    say("mxgemm_fp8 bands")
    ref = bits16(run(qa, ea, qb, eb))
    assert np.array_equal(bits16(run(qa, ea, qb, eb, bands=bands)), ref)
    stride = (M // bands) * N + pad
    C = torch.empty(bands * stride, dtype=torch.bfloat16, device=device())
    C.view(torch.int16).fill_(0x5A5A)
    run(qa, ea, qb, eb, bands=bands, band_stride=stride, C=C)
    expect = np.full(bands * stride, 0x5A5A, np.uint16)
    oracle.band_store(ref.reshape(M, N), bands, stride, expect)
    assert np.array_equal(bits16(C), expect)


def test_mxq_into_mxgemm():
    """bf16 operands quantized on the device, then multiplied: codes and scales
    equal O10's, the product lies within the bound of O11 on them."""
    M, N, K = 512, 640, 1024
    A, B = synth.operand_fp32(M, N, K, seed=5, heavy=True)
    ab, bb = oracle.bf16_rne_array(A), oracle.bf16_rne_array(B)
    qa, ea = oracle.mx_quant((ab.astype(np.uint32) << 16).view(np.float32))
    qb, eb = oracle.mx_quant((bb.astype(np.uint32) << 16).view(np.float32))
    say("mxq -> mxgemm")
    dqa, dea = bs.mxq_e4m3(bf16_dev(ab))
    dqb, deb = bs.mxq_e4m3(bf16_dev(bb))
    C = poison_bf16(torch.empty(M * N, dtype=torch.bfloat16, device=device()))
    bs.mxgemm_fp8(dqa, dea, dqb, deb, C)
    torch.cuda.synchronize()
    assert np.array_equal(dqa.cpu().numpy(), qa) and np.array_equal(dea.cpu().numpy(), ea)
    assert np.array_equal(dqb.cpu().numpy(), qb) and np.array_equal(deb.cpu().numpy(), eb)
    mx_accept(bits16(C).reshape(M, N), qa, ea, qb, eb, "mxq -> mxgemm")


@pytest.mark.parametrize("M,N,K,bands", [(16384, 5120, 2048, 1), (4096, 5120, 4096, 8)])
def test_mxgemm_full_size(M, N, K, bands):
    """The mxfp8 wo_b shapes (N = 5120, K = 2048 and 4096), every output
    element against O11."""
    qa, ea, qb, eb = operands(M, N, K, seed=6, heavy=True)
    say(f"mxgemm_fp8 full size M={M} N={N} K={K} bands={bands}")
    out = bits16(run(qa, ea, qb, eb, bands=bands)).reshape(M, N)
    mx_accept(out, qa, ea, qb, eb, f"mx M={M} N={N} K={K} all elements", model=False)


def test_mxgemm_rejects_without_writing():
    qa, ea, qb, eb = operands(256, 512, 256)
    C = poison_bf16(torch.empty(256 * 512, dtype=torch.bfloat16, device=device()))
    with pytest.raises(bs.BSError) as e:
        bs.mxgemm_fp8(to_dev(qa), to_dev(ea), to_dev(qb), to_dev(eb), C, bands=3)
    assert e.value.status == bs.BS_ERR_UNSUPPORTED
    torch.cuda.synchronize()
    assert np.all(bits16(C) == 0x7FC0)


@pytest.mark.parametrize("M,N,K", [(1, 256, 256), (3, 128, 8192), (200, 384, 8192)])
def test_mxgemm_edge_shapes(M, N, K):
    say(f"mxgemm_fp8 edge M={M} N={N} K={K}")
    qa, ea, qb, eb = operands(M, N, K, seed=7, heavy=True)
    mx_accept(bits16(run(qa, ea, qb, eb)).reshape(M, N), qa, ea, qb, eb, f"mx edge M={M} N={N} K={K}")
