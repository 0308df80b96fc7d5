"""The composed per-GPU step (GEMM with band epilogue -> band reduce -> row
quantize -> row dequantize) against the same chain run entirely in the oracle
(GEMM as O4m, the definition that forms block dot products as the fp8 MFMA
does).

The GEMM's bf16 output is fixed up to accumulation order (relL2 <= 3e-5), so
later stages are compared where their inputs agree exactly: every row of the
reduced band that matches the oracle's bit for bit must give the oracle's
codes and scale bit for bit, and the stand-in rows of the wire buffer, which
do not depend on the GEMM, must dequantize bit for bit."""
import numpy as np
import pytest
import torch

import oracle
import synth
from block_scaled_fp8_bsgemm_amd.pipeline import WoBStep
from gpuutil import bf16_dev, bits16, gemm_compare, say, to_dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("M,N,K,bands", [(512, 1024, 512, 8), (1000, 512, 256, 8)])
def test_pipeline_vs_oracle_chain(M, N, K, bands):
    say(f"pipeline M={M} N={N} K={K} bands={bands}")
    band_rows = M // bands
    A, B = synth.operand_fp32(M, N, K, seed=0, heavy=True)
    qa, sa = oracle.quant_blocks(A, 1, 128)
    qb, sb = oracle.quant_blocks(B, 128, 128)
    parts = synth.partial_bands(band_rows, N, P=bands, seed0=100)[1:]
    wire_x = synth.wire_rows(M, N, seed=200)
    wq, ws = oracle.rowq(wire_x)          # stand-in gathered wire (rows 0..band_rows overwritten)

    # oracle chain
    _, c_exact = oracle.bsgemm(qa, sa, qb, sb)
    _, c_ref = oracle.bsgemm(qa, sa, qb, sb, mfma=True)
    red_ref = oracle.band_reduce([c_ref[:band_rows]] + parts)
    q_own_ref, s_own_ref = oracle.rowq(red_ref)
    wq_ref, ws_ref = wq.copy(), ws.copy()
    wq_ref[:band_rows], ws_ref[:band_rows] = q_own_ref, s_own_ref
    y_ref = oracle.rowdq(wq_ref, ws_ref)

    # device chain
    step = WoBStep(to_dev(qa), to_dev(sa), to_dev(qb), to_dev(sb), [bf16_dev(p) for p in parts],
                   to_dev(wq), to_dev(ws), bands)
    step.step()
    torch.cuda.synchronize()

    gemm_compare(bits16(step.C), c_ref, c_exact, "pipeline gemm")
    red = bits16(step.reduced)
    red_exact = oracle.band_reduce([c_exact[:band_rows]] + parts)
    gemm_compare(red, red_ref, red_exact, "pipeline reduce")
    q_own = step.own_q.cpu().numpy()
    s_own = step.own_s.cpu().numpy()
    same = np.all(red == red_ref, axis=1)
    assert same.mean() > 0.5, same.mean()
    assert np.array_equal(q_own[same], q_own_ref[same])
    assert np.array_equal(s_own[same].view(np.uint32), s_own_ref[same].view(np.uint32))
    y = bits16(step.out)
    assert np.array_equal(y[band_rows:], y_ref[band_rows:])
    rows_same = np.nonzero(same)[0]
    assert np.array_equal(y[rows_same], y_ref[rows_same])


@pytest.mark.parametrize("M,fused", [(8192, False), (8192, True), (16384, False), (16384, True),
                                     (20000, True)])
def test_pipeline_full_size(M, fused):
    """The pipeline sweep at its real shapes (N=7168, K=2048, 8 bands; M=20000
    zero-padded to 20096 = 157 * 128), with reduce and quantize as two calls
    or fused into one (the benchmark's step).  The GEMM is checked at sampled
    elements (a quarter of them in band 0, the reduce's input); every later
    stage is checked bit for bit against the oracle applied to the device's
    own input to that stage: the reduce of the device's band 0 and the 7
    stand-in bands, the row quantize of that reduced band, and the dequantize
    of the wire buffer holding the device's codes."""
    _full_chain_check(M, synth.HIDDEN, synth.K_SHARD, synth.P_RANKS, fused, full_gemm=False)


@pytest.mark.parametrize("M,N,K,bands", [(512, 1024, 512, 8), (1000, 512, 256, 8), (96, 384, 128, 3)])
def test_pipeline_fused_small(M, N, K, bands):
    """The fused step at small and ragged shapes (a ragged last GEMM tile, N
    not a multiple of 256, three bands), checked as the full-size test does
    but with the whole GEMM output compared."""
    _full_chain_check(M, N, K, bands, True, full_gemm=True)


def _full_chain_check(M, N, K, bands, fused, full_gemm):
    Mp = -(-M // 128) * 128 if not full_gemm else M
    band_rows = Mp // bands
    say(f"pipeline M={M} (padded {Mp}) N={N} K={K} bands={bands} fused={fused}")
    A, B = synth.operand_fp32(M, N, K, seed=0, heavy=True)
    A = synth.pad_rows(A, Mp)
    qa, sa = oracle.quant_blocks(A, 1, 128)
    qb, sb = oracle.quant_blocks(B, 128, 128)
    del A, B
    parts = synth.partial_bands(band_rows, N, P=bands, seed0=100)[1:]
    wq, ws = oracle.rowq(synth.wire_rows(Mp, N, seed=200))

    step = WoBStep(to_dev(qa), to_dev(sa), to_dev(qb), to_dev(sb), [bf16_dev(p) for p in parts],
                   to_dev(wq), to_dev(ws), bands, fused=fused)
    step.step()
    torch.cuda.synchronize()
    c = bits16(step.C).reshape(Mp, N)

    if full_gemm:
        _, c_exact = oracle.bsgemm(qa, sa, qb, sb)
        _, c_ref = oracle.bsgemm(qa, sa, qb, sb, mfma=True)
        gemm_compare(c, c_ref, c_exact, f"pipeline M={M} N={N} K={K}")
    else:
        mi, ni = synth.sample_indices(Mp, N, 24576, seed=M)
        m0, n0 = synth.sample_indices(band_rows, N, 8192, seed=M + 1)
        mi, ni = np.concatenate([mi, m0]), np.concatenate([ni, n0])
        _, e_ref = oracle.bsgemm_elems(qa, sa, qb, sb, mi, ni)
        _, e_ref_m = oracle.bsgemm_elems(qa, sa, qb, sb, mi, ni, mfma=True)
        gemm_compare(c[mi, ni], e_ref_m, e_ref, f"pipeline M={Mp} sampled")
        assert np.all(c[M:] == 0)

    red = oracle.band_reduce([c[:band_rows]] + parts)
    if not fused:
        assert np.array_equal(bits16(step.reduced), red)
    q_dev = step.own_q.cpu().numpy()
    s_dev = step.own_s.cpu().numpy()
    q_ref, s_ref = oracle.rowq(red)
    assert np.array_equal(q_dev, q_ref)
    assert np.array_equal(s_dev.view(np.uint32), s_ref.view(np.uint32))
    wq_ref, ws_ref = wq.copy(), ws.copy()
    wq_ref[:band_rows], ws_ref[:band_rows] = q_ref, s_ref
    assert np.array_equal(bits16(step.out), oracle.rowdq(wq_ref, ws_ref))
