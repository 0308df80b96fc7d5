"""Maximum-size cases on the device (an MI355X holds 288 GB): the dequantizer
past 2^31 packs, where it switches to 64-bit indices, the GEMM with a
14 GiB output written as 8 bands, where row offsets pass 2^32 bytes, and the
GEMMs (blockscale and mxfp8) with an operand of more than 2^31 bytes.  Inputs
are drawn on the device; sampled outputs (whole rows for the GEMM) are
checked against the oracle, so nothing large crosses to the host."""
import numpy as np
import pytest
import torch

import block_scaled_fp8_bsgemm_amd as bs
import oracle
import synth
from gpuutil import bits16, device, gemm_accept_rows, mx_accept, say

pytestmark = pytest.mark.gpu


def test_rowdq_64bit_index():
    rows, N = 1 << 21, 8192                     # 2^34 codes = 2^31 packs of 8
    dev = device()
    say(f"rowdq_e4m3 rows={rows} N={N} (64-bit index path)")
    g = torch.Generator(device=dev)
    g.manual_seed(21)
    q = torch.randint(0, 0x7F, (rows, N), dtype=torch.uint8, device=dev, generator=g)   # no NaN codes
    q |= torch.randint(0, 2, (rows, N), dtype=torch.uint8, device=dev, generator=g) << 7
    s = torch.rand(rows, device=dev, generator=g) * 4.0
    y = bs.rowdq_e4m3(q, s)
    torch.cuda.synchronize()
    mi, ni = synth.sample_indices(rows, N, 65536, seed=3)
    mi = np.concatenate([mi, np.full(64, rows - 1), np.arange(rows - 64, rows)])
    ni = np.concatenate([ni, np.arange(N - 64, N), np.full(64, N - 1)])
    tm, tn = torch.from_numpy(mi).to(dev), torch.from_numpy(ni).to(dev)
    qs = q[tm, tn].cpu().numpy()
    ss = s[tm].cpu().numpy()
    ys = y[tm, tn].view(torch.int16).cpu().numpy().view(np.uint16)
    ref = oracle.rowdq(qs[:, None], ss)[:, 0]
    del q, y
    torch.cuda.empty_cache()
    assert np.array_equal(ys, ref)


def test_gemm_output_past_4gib():
    M, N, K, bands = 1 << 20, 7168, 256, 8     # C: 14 GiB in 8 bands of 1.75 GiB
    dev = device()
    say(f"bsgemm_fp8 M={M} N={N} K={K} bands={bands} (C past 2^32 bytes)")
    g = torch.Generator(device=dev)
    g.manual_seed(22)
    qa, sa = bs.blockq_e4m3(torch.randn(M, K, device=dev, generator=g), 1)
    qb, sb = bs.blockq_e4m3(0.02 * torch.randn(N, K, device=dev, generator=g), 128)
    C = torch.empty(M * N, dtype=torch.bfloat16, device=dev)
    C.view(torch.int16).fill_(0x7FC0)
    bs.bsgemm_fp8(qa, sa, qb, sb, C, bands=bands)
    torch.cuda.synchronize()
    # whole rows: random ones, the first and last row of every band, the last row
    rng = np.random.default_rng(4)
    edge = [M // bands * d + o for d in range(bands) for o in (0, M // bands - 1)]
    rows = np.unique(np.concatenate([rng.integers(0, M, 48), edge, [M - 1]])).astype(np.int64)
    tm = torch.from_numpy(rows).to(dev)
    got = C.view(M, N)[tm].view(torch.int16).cpu().numpy().view(np.uint16)
    qa_h, sa_h = qa.cpu().numpy(), sa.cpu().numpy()
    qb_h, sb_h = qb.cpu().numpy(), sb.cpu().numpy()
    del C, qa, sa
    torch.cuda.empty_cache()
    gemm_accept_rows(got, rows, qa_h, sa_h, qb_h, sb_h, f"M={M} {rows.size} whole rows")


def test_gemm_persistent_offsets_near_2gib():
    """The largest A the persistent kernel takes at K = 2048: (M + 256) * K
    just under 2^31, so its lanes' byte offsets, ragged tile rows included,
    come within one tile of 2^31.  Whole rows at both ends against the
    oracle (both GEMMs)."""
    M, N, K = (1 << 20) - 384, 512, 2048
    assert (M + 256) * K <= 0x7FFFFFFF < (M + 384) * K   # the largest M (a multiple of 128) it takes
    KB = K // 128
    dev = device()
    say(f"bsgemm_fp8 / mxgemm_fp8 M={M} N={N} K={K} (A of {M * K} bytes, persistent)")
    g = torch.Generator(device=dev)
    g.manual_seed(25)
    qa = torch.randint(0, 0x7F, (M, K), dtype=torch.uint8, device=dev, generator=g)   # no NaN codes
    qa |= torch.randint(0, 2, (M, K), dtype=torch.uint8, device=dev, generator=g) << 7
    sa = torch.rand((M, KB), device=dev, generator=g) * 2.0 ** -8
    ea = torch.randint(117, 128, (M, K // 32), dtype=torch.uint8, device=dev, generator=g)
    qb, sb = bs.blockq_e4m3(0.02 * torch.randn(N, K, device=dev, generator=g), 128)
    eb = torch.randint(117, 128, (N, K // 32), dtype=torch.uint8, device=dev, generator=g)
    C = torch.empty(M * N, dtype=torch.bfloat16, device=dev)
    C2 = torch.empty(M * N, dtype=torch.bfloat16, device=dev)
    C.view(torch.int16).fill_(0x7FC0)
    C2.view(torch.int16).fill_(0x7FC0)
    bs.bsgemm_fp8(qa, sa, qb, sb, C)
    bs.mxgemm_fp8(qa, ea, qb, eb, C2)
    torch.cuda.synchronize()
    rng = np.random.default_rng(7)
    rows = np.unique(np.concatenate([rng.integers(0, M, 24), [0, 1, M - 257, M - 256, M - 2, M - 1]])).astype(np.int64)
    tm = torch.from_numpy(rows).to(dev)
    got = C.view(M, N)[tm].view(torch.int16).cpu().numpy().view(np.uint16)
    got2 = C2.view(M, N)[tm].view(torch.int16).cpu().numpy().view(np.uint16)
    qa_r, sa_r, ea_r = qa[tm].cpu().numpy(), sa[tm].cpu().numpy(), ea[tm].cpu().numpy()
    qb_h, sb_h, eb_h = qb.cpu().numpy(), sb.cpu().numpy(), eb.cpu().numpy()
    del C, C2, qa, sa, ea
    torch.cuda.empty_cache()
    gemm_accept_rows(got, np.arange(rows.size), qa_r, sa_r, qb_h, sb_h, f"M={M} {rows.size} whole rows")
    mx_accept(got2, qa_r, ea_r, qb_h, eb_h, f"mx M={M} {rows.size} whole rows", model=False)


def test_gemm_operand_past_2gib():
    """A of 2^31 bytes and more (M = 2^20 + 128, K = 2048): past what one
    31-bit descriptor offset reaches, so the host takes the tile kernel,
    whose descriptors start at each tile.  Whole rows on both sides of byte
    2^31 of A against the oracle."""
    M, N, K = (1 << 20) + 128, 256, 2048
    KB = K // 128
    dev = device()
    say(f"bsgemm_fp8 M={M} N={N} K={K} (A of {M * K} bytes)")
    g = torch.Generator(device=dev)
    g.manual_seed(23)
    qa = torch.randint(0, 0x7F, (M, K), dtype=torch.uint8, device=dev, generator=g)   # no NaN codes
    qa |= torch.randint(0, 2, (M, K), dtype=torch.uint8, device=dev, generator=g) << 7
    sa = torch.rand((M, KB), device=dev, generator=g) * 2.0 ** -8
    qb, sb = bs.blockq_e4m3(0.02 * torch.randn(N, K, device=dev, generator=g), 128)
    C = torch.empty(M * N, dtype=torch.bfloat16, device=dev)
    C.view(torch.int16).fill_(0x7FC0)
    bs.bsgemm_fp8(qa, sa, qb, sb, C)
    torch.cuda.synchronize()
    rng = np.random.default_rng(5)
    split = (1 << 31) // K                     # the first row at or past byte 2^31 of A
    edge = [0, split - 1, split, split + 1, M - 129, M - 128, M - 1]
    rows = np.unique(np.concatenate([rng.integers(0, M, 40), edge])).astype(np.int64)
    tm = torch.from_numpy(rows).to(dev)
    got = C.view(M, N)[tm].view(torch.int16).cpu().numpy().view(np.uint16)
    qa_r, sa_r = qa[tm].cpu().numpy(), sa[tm].cpu().numpy()
    qb_h, sb_h = qb.cpu().numpy(), sb.cpu().numpy()
    del C, qa, sa
    torch.cuda.empty_cache()
    gemm_accept_rows(got, np.arange(rows.size), qa_r, sa_r, qb_h, sb_h, f"M={M} {rows.size} whole rows")


def test_mxgemm_operand_past_2gib():
    """The mxfp8 GEMM with an A of more than 2^31 bytes (M = 2^20 + 128,
    K = 2048), which the host also sends to the tile kernel.  Whole rows on
    both sides of byte 2^31 of A against O11."""
    M, N, K = (1 << 20) + 128, 256, 2048
    dev = device()
    say(f"mxgemm_fp8 M={M} N={N} K={K} (A of {M * K} bytes)")
    g = torch.Generator(device=dev)
    g.manual_seed(24)
    qa = torch.randint(0, 0x7F, (M, K), dtype=torch.uint8, device=dev, generator=g)   # no NaN codes
    qa |= torch.randint(0, 2, (M, K), dtype=torch.uint8, device=dev, generator=g) << 7
    ea = torch.randint(117, 128, (M, K // 32), dtype=torch.uint8, device=dev, generator=g)
    qb = torch.randint(0, 0x7F, (N, K), dtype=torch.uint8, device=dev, generator=g)
    qb |= torch.randint(0, 2, (N, K), dtype=torch.uint8, device=dev, generator=g) << 7
    eb = torch.randint(117, 128, (N, K // 32), dtype=torch.uint8, device=dev, generator=g)
    C = torch.empty(M * N, dtype=torch.bfloat16, device=dev)
    C.view(torch.int16).fill_(0x7FC0)
    bs.mxgemm_fp8(qa, ea, qb, eb, C)
    torch.cuda.synchronize()
    rng = np.random.default_rng(6)
    split = (1 << 31) // K
    edge = [0, split - 1, split, split + 1, M - 129, M - 128, M - 1]
    rows = np.unique(np.concatenate([rng.integers(0, M, 40), edge])).astype(np.int64)
    tm = torch.from_numpy(rows).to(dev)
    got = C.view(M, N)[tm].view(torch.int16).cpu().numpy().view(np.uint16)
    qa_r, ea_r = qa[tm].cpu().numpy(), ea[tm].cpu().numpy()
    qb_h, eb_h = qb.cpu().numpy(), eb.cpu().numpy()
    del C, qa, ea
    torch.cuda.empty_cache()
    mx_accept(got, qa_r, ea_r, qb_h, eb_h, f"mx M={M} {rows.size} whole rows", model=False)
