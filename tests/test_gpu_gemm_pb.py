"""GPU parity of the prepacked-weight GEMM: bprepack_e4m3 against the
oracle's layout O12 byte for byte, and bsgemm_fp8_pb on the prepacked weight
against bsgemm_fp8 on the plain one bit for bit (they feed the MFMA the same
bytes in the same order) and against the exact product O4 under the GEMM's
element-wise bound."""
import numpy as np
import pytest
import torch

import block_scaled_fp8_bsgemm_amd as bs
import oracle
import synth
from gpuutil import bits16, device, gemm_accept, poison_bf16, poison_u8, say, to_dev, workload_operands

pytestmark = pytest.mark.gpu


def operands(M, N, K, seed=0, heavy=False, pad_to=None):
    A, B = synth.operand_fp32(M, N, K, seed=seed, heavy=heavy)
    if pad_to:
        A = synth.pad_rows(A, pad_to)
    qa, sa = oracle.quant_blocks(A, 1, 128)
    qb, sb = oracle.quant_blocks(B, 128, 128)
    return qa, sa, qb, sb


def prepack(qb):
    N, K = qb.shape
    Bp = poison_u8(torch.empty(N * K, dtype=torch.uint8, device=device()))
    bs.bprepack_e4m3(to_dev(qb), Bp)
    return Bp


def run_both(qa, sa, qb, sb, bands=1):
    M, N = qa.shape[0], qb.shape[0]
    dA, dsa, dB, dsb = to_dev(qa), to_dev(sa), to_dev(qb), to_dev(sb)
    Bp = prepack(qb)
    C1 = poison_bf16(torch.empty(M * N, dtype=torch.bfloat16, device=device()))
    C2 = poison_bf16(torch.empty(M * N, dtype=torch.bfloat16, device=device()))
    bs.bsgemm_fp8(dA, dsa, dB, dsb, C1, bands=bands)
    bs.bsgemm_fp8_pb(dA, dsa, Bp, dsb, C2, bands=bands)
    torch.cuda.synchronize()
    return bits16(C1).reshape(M, N), bits16(C2).reshape(M, N)


@pytest.mark.parametrize("N,K", [(128, 128), (512, 256), (384, 1152), (7168, 2048)])
def test_bprepack_bitexact(N, K):
    say(f"bprepack_e4m3 N={N} K={K}")
    rng = np.random.default_rng(N + K)
    qb = rng.integers(0, 256, size=(N, K), dtype=np.uint8)
    Bp = prepack(qb)
    torch.cuda.synchronize()
    assert np.array_equal(Bp.cpu().numpy(), oracle.bprepack(qb))


@pytest.mark.parametrize("M,N,K,heavy", [
    (256, 512, 256, False),
    (640, 640, 512, True),      # ragged M tile; N = 2.5 tiles (the last tile's second half is past N)
    (300, 384, 384, False),     # odd K-block count
    (16, 128, 128, False),      # one K block, one partial tile
    (513, 1024, 1152, True),
])
def test_gemm_pb_equals_plain_and_oracle(M, N, K, heavy):
    say(f"bsgemm_fp8_pb M={M} N={N} K={K}")
    qa, sa, qb, sb = operands(M, N, K, seed=0, heavy=heavy)
    c_plain, c_pb = run_both(qa, sa, qb, sb)
    assert np.array_equal(c_pb, c_plain)
    gemm_accept(c_pb, qa, sa, qb, sb, f"pb M={M} N={N} K={K}")


@pytest.mark.parametrize("M,bands,pad_to", [(16384, 8, None), (20000, 8, 20096)])
def test_gemm_pb_full_size(M, bands, pad_to):
    """The benchmark shapes in the benchmark's launch configuration: bit for
    bit equal to the plain-B GEMM everywhere, and every element against the
    exact product."""
    N, K = synth.HIDDEN, synth.K_SHARD
    qa, sa, qb, sb = workload_operands(M, N, K, seed=0, heavy=True, pad_to=pad_to)
    Mp = qa.shape[0]
    say(f"bsgemm_fp8_pb full size M={Mp} bands={bands}")
    c_plain, c_pb = run_both(qa, sa, qb, sb, bands=bands)
    assert np.array_equal(c_pb, c_plain)
    del c_plain
    gemm_accept(c_pb, qa, sa, qb, sb, f"pb M={Mp} all elements", key=("wo_b", M, pad_to), model=False)
    if pad_to:
        assert np.all(c_pb[M:] == 0)


def test_gemm_pb_bands_with_stride():
    M, N, K, bands, pad = 1024, 512, 256, 4, 136
    qa, sa, qb, sb = operands(M, N, K, seed=3)
    say("bsgemm_fp8_pb padded bands")
    c_plain, _ = run_both(qa, sa, qb, sb)
    Bp = prepack(qb)
    stride = (M // bands) * N + pad
    C = torch.empty(bands * stride, dtype=torch.bfloat16, device=device())
    C.view(torch.int16).fill_(0x5A5A)
    bs.bsgemm_fp8_pb(to_dev(qa), to_dev(sa), Bp, to_dev(sb), C, bands=bands, band_stride=stride)
    torch.cuda.synchronize()
    expect = np.full(bands * stride, 0x5A5A, np.uint16)
    oracle.band_store(c_plain, bands, stride, expect)
    assert np.array_equal(bits16(C), expect)
