"""GPU parity of bsgemm_fp8 against the oracle (O4 product, O5 band layout).

Inputs are the seeded synthetic operands quantized by the oracle's block
quantizer; both sides consume the same bytes.  Acceptance: every bf16 output
element inside the interval the fp8 MFMA's truncation and rounding allow
around the exact product O4 (gpuutil.gemm_accept, oracle/bounds.py), at
every shape including the benchmark's full sizes; bit for bit where all sums
are exact; bitwise for the band layout and for repeated runs."""
import numpy as np
import pytest
import torch

import block_scaled_fp8_bsgemm_amd as bs
import oracle
import synth
from gpuutil import bits16, device, gemm_accept, poison_bf16, say, to_dev, workload_operands

pytestmark = pytest.mark.gpu


def operands(M, N, K, seed=0, heavy=False, pad_to=None):
    A, B = synth.operand_fp32(M, N, K, seed=seed, heavy=heavy)
    if pad_to:
        A = synth.pad_rows(A, pad_to)
    qa, sa = oracle.quant_blocks(A, 1, 128)
    qb, sb = oracle.quant_blocks(B, 128, 128)
    return qa, sa, qb, sb


def run(qa, sa, qb, sb, bands=1, band_stride=0, C=None):
    dA, dsa, dB, dsb = to_dev(qa), to_dev(sa), to_dev(qb), to_dev(sb)
    M, N = qa.shape[0], qb.shape[0]
    if C is None:
        band_rows = M // bands
        stride = band_stride or band_rows * N
        C = torch.empty((bands - 1) * stride + band_rows * N, dtype=torch.bfloat16, device=device())
        poison_bf16(C)
    bs.bsgemm_fp8(dA, dsa, dB, dsb, C, bands=bands, band_stride=band_stride)
    torch.cuda.synchronize()
    return C


@pytest.mark.parametrize("M,N,K,heavy", [
    (256, 512, 256, False),     # the tiny workload (one M tile, two N tiles)
    (640, 640, 512, True),      # 2.5 x 2.5 tiles: ragged M tile and a 128-wide N tail
    (300, 384, 384, False),     # M not a multiple of 128
    (16, 128, 128, False),      # a single partial tile
    (513, 1024, 1152, True),    # 9 K blocks (odd count), ragged by one row
    (1500, 2304, 512, True),    # 6 x 9 tiles: a full group of 4 M-tiles and a partial one
])
def test_gemm_full_vs_oracle(M, N, K, heavy):
    say(f"bsgemm_fp8 M={M} N={N} K={K} heavy={heavy}")
    qa, sa, qb, sb = operands(M, N, K, seed=0, heavy=heavy)
    C = run(qa, sa, qb, sb)
    gemm_accept(bits16(C).reshape(M, N), qa, sa, qb, sb, f"M={M} N={N} K={K}")


def test_gemm_unit_scale_exact():
    """Small-integer codes with unit scales: every sum is exact in fp32, so the
    device result must equal the oracle bit for bit."""
    rng = np.random.default_rng(1)
    t = oracle.e4m3_table()
    small = np.array([c for c in range(256) if np.isfinite(t[c]) and abs(t[c]) <= 4 and (t[c] * 2) % 1 == 0])
    M, N, K = 256, 256, 512
    qa = rng.choice(small, size=(M, K)).astype(np.uint8)
    qb = rng.choice(small, size=(N, K)).astype(np.uint8)
    sa = np.ones((M, K // 128), np.float32)
    sb = np.ones((N // 128, K // 128), np.float32)
    say("bsgemm_fp8 unit scales exact")
    _, ref = oracle.bsgemm(qa, sa, qb, sb)
    C = run(qa, sa, qb, sb)
    assert np.array_equal(bits16(C).reshape(M, N), ref)


def test_gemm_zero_rows_and_determinism():
    M, N, K = 512, 512, 512
    qa, sa, qb, sb = operands(M, N, K, seed=2)
    qa[17] = 0
    sa[300] = 0
    say("bsgemm_fp8 zero rows + repeat")
    C1 = run(qa, sa, qb, sb)
    C2 = run(qa, sa, qb, sb)
    b1 = bits16(C1).reshape(M, N)
    assert np.array_equal(b1, bits16(C2).reshape(M, N))
    assert np.all(b1[17] == 0) and np.all(b1[300] == 0)


@pytest.mark.parametrize("M,bands", [(4252, 4), (4224, 33)])
def test_gemm_many_tiles_vs_oracle(M, bands):
    """More tiles than the chip has CUs (17 x 17 = 289), so that workgroups of
    the persistent kernel (K / 128 even) run two tiles each; element by
    element against the oracle.  M = 4252: a ragged last M tile and 1063-row
    bands that begin inside tiles; M = 4224: 33 bands of 128 rows, shorter
    than a tile."""
    N, K = 4352, 256
    qa, sa, qb, sb = operands(M, N, K, seed=7, heavy=True)
    say(f"bsgemm_fp8 many tiles M={M} N={N} K={K} bands={bands}")
    C = run(qa, sa, qb, sb, bands=bands)
    gemm_accept(bits16(C).reshape(M, N), qa, sa, qb, sb, f"many tiles M={M} bands={bands}")


@pytest.mark.parametrize("M,bands,pad", [(2048, 8, 0), (1024, 4, 136), (20096 // 8, 2, 8)])
def test_gemm_band_layout(M, bands, pad):
    """Band epilogue: contiguous bands are byte-identical to the row-major
    output; padded bands hold the same rows and leave the gaps untouched."""
    N, K = 512, 256
    qa, sa, qb, sb = operands(M, N, K, seed=3)
    say(f"bsgemm_fp8 bands={bands} pad={pad} M={M}")
    ref = bits16(run(qa, sa, qb, sb, bands=1))
    got = bits16(run(qa, sa, qb, sb, bands=bands))
    assert np.array_equal(got, ref)
    band_rows = M // bands
    stride = band_rows * N + pad
    C = torch.empty(bands * stride, dtype=torch.bfloat16, device=device())
    C.view(torch.int16).fill_(0x5A5A)
    run(qa, sa, qb, sb, bands=bands, band_stride=stride, C=C)
    out = bits16(C)
    expect = np.full(bands * stride, 0x5A5A, np.uint16)
    oracle.band_store(ref.reshape(M, N), bands, stride, expect)
    assert np.array_equal(out, expect)


@pytest.mark.parametrize("M,bands,pad", [(8292, 1, 0), (8192, 4, 64)])
def test_gemm_persistent_tile_transitions(M, bands, pad):
    """The persistent kernel carries a plain tile's stores over into the next
    tile (half at the tile's end, half inside the next tile's first K block)
    and stores other tiles at once.  M = 8292: 33 x 17 tiles, about 2.2 per
    workgroup, the last M-tile ragged, so workgroups pass between plain and
    ragged tiles in both orders; M = 8192 with padded bands: no tile is
    plain.  Every element against the exact product, and the band gaps
    untouched."""
    N, K = 4352, 256
    qa, sa, qb, sb = operands(M, N, K, seed=11, heavy=True)
    say(f"bsgemm_fp8 tile transitions M={M} bands={bands} pad={pad}")
    band_rows = M // bands
    stride = band_rows * N + pad
    C = torch.empty((bands - 1) * stride + band_rows * N + pad, dtype=torch.bfloat16, device=device())
    C.view(torch.int16).fill_(0x5A5A)
    run(qa, sa, qb, sb, bands=bands, band_stride=stride if pad else 0, C=C)
    raw = bits16(C)
    got = np.concatenate([raw[d * stride: d * stride + band_rows * N] for d in range(bands)]).reshape(M, N)
    gemm_accept(got, qa, sa, qb, sb, f"tile transitions M={M} bands={bands} pad={pad}")
    if pad:
        for d in range(bands):
            assert np.all(raw[d * stride + band_rows * N: (d + 1) * stride] == 0x5A5A)


@pytest.mark.parametrize("M,bands,pad_to", [(4096, 1, None), (16384, 8, None), (20000, 8, 20096)])
def test_gemm_full_size(M, bands, pad_to):
    """The benchmark shapes (N=7168, K=2048, heavy rows), in the launch
    configuration the benchmark times, every output element against the
    exact product; padded rows must be exactly zero."""
    N, K = synth.HIDDEN, synth.K_SHARD
    qa, sa, qb, sb = workload_operands(M, N, K, seed=0, heavy=True, pad_to=pad_to)
    Mp = qa.shape[0]
    say(f"bsgemm_fp8 full size M={Mp} bands={bands}")
    C = run(qa, sa, qb, sb, bands=bands)
    out = bits16(C).reshape(Mp, N)  # contiguous bands == row-major
    del C
    gemm_accept(out, qa, sa, qb, sb, f"M={Mp} all elements", key=("wo_b", M, pad_to), model=False)
    if pad_to:
        assert np.all(out[M:] == 0)


def test_gemm_rejects_without_writing():
    qa, sa, qb, sb = operands(256, 512, 256)
    dA, dsa, dB, dsb = to_dev(qa), to_dev(sa), to_dev(qb), to_dev(sb)
    C = poison_bf16(torch.empty(256 * 512, dtype=torch.bfloat16, device=device()))
    with pytest.raises(bs.BSError) as e:
        bs.bsgemm_fp8(dA, dsa, dB, dsb, C, bands=3)   # 256 % 3 != 0
    assert e.value.status == bs.BS_ERR_UNSUPPORTED
    torch.cuda.synchronize()
    assert np.all(bits16(C) == 0x7FC0)


@pytest.mark.parametrize("M,N,K", [(1, 256, 256), (3, 128, 8192), (200, 384, 8192)])
def test_gemm_edge_shapes(M, N, K):
    """One row; a single 128-column block; K = 8192 (64 K blocks, four times the
    benchmark's depth, even and odd block counts are covered elsewhere)."""
    say(f"bsgemm_fp8 edge M={M} N={N} K={K}")
    qa, sa, qb, sb = operands(M, N, K, seed=5, heavy=True)
    C = run(qa, sa, qb, sb)
    gemm_accept(bits16(C).reshape(M, N), qa, sa, qb, sb, f"edge M={M} N={N} K={K}")
    Bp = torch.empty(N * K, dtype=torch.uint8, device=device())
    bs.bprepack_e4m3(to_dev(qb), Bp)
    C2 = poison_bf16(torch.empty(M * N, dtype=torch.bfloat16, device=device()))
    bs.bsgemm_fp8_pb(to_dev(qa), to_dev(sa), Bp, to_dev(sb), C2)
    torch.cuda.synchronize()
    assert np.array_equal(bits16(C2), bits16(C))
