"""Pins for the element-wise GEMM acceptance bounds (oracle/bounds.py).

A bound is only worth something if (1) the arithmetic it claims to cover
stays inside it and (2) the mistakes it is meant to catch fall outside it.
(1): the instruction model O4m (and O11m for mxfp8) lies inside the bound of
the exact definition O4 (O11) on the workload's distributions and on
adversarial codes and scales.  (2): mistakes planted in the oracle on the CPU
-- a wrong scale index, a dropped K block, a shifted or transposed operand, a
lost scale factor, mismatched K orders, a sign -- each put elements outside.
The bf16 rounding helper is pinned against the oracle's own fp32 -> bf16
narrowing (itself pinned against torch in test_oracle_codec.py).
"""
import numpy as np
import pytest

import oracle
import synth
from oracle import bounds


def quantized(M, N, K, seed=0, heavy=False):
    A, B = synth.operand_fp32(M, N, K, seed=seed, heavy=heavy)
    qa, sa = oracle.quant_blocks(A, 1, 128)
    qb, sb = oracle.quant_blocks(B, 128, 128)
    return qa, sa, qb, sb


def check(got_bits, acc_ref, ops):
    return bounds.check_bsgemm(got_bits, acc_ref, *ops)


def test_bf16_rne_f64_matches_fp32_narrowing():
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(300000) * np.exp2(rng.integers(-150, 120, 300000))).astype(np.float32)
    # exact ties: 8 significant bits plus a trailing half
    ties = (np.ldexp(rng.integers(256, 512, 20000) * 2 + 1, rng.integers(-140, 100, 20000) - 9)).astype(np.float32)
    for v in (x, ties, -ties):
        ref = bounds.bf16_bits_to_f64(oracle.bf16_rne_array(v))
        assert np.array_equal(bounds.bf16_rne_f64(v.astype(np.float64)), ref)


@pytest.mark.parametrize("M,N,K,heavy,seed", [
    (256, 512, 256, False, 0),     # the tiny workload
    (384, 512, 2048, True, 1),     # the benchmark's depth, heavy rows
])
def test_mfma_model_inside_bound(M, N, K, heavy, seed):
    qa, sa, qb, sb = quantized(M, N, K, seed=seed, heavy=heavy)
    acc, _ = oracle.bsgemm(qa, sa, qb, sb)
    _, cm = oracle.bsgemm(qa, sa, qb, sb, mfma=True)
    st = check(cm, acc, (qa, sa, qb, sb))
    assert st["bad"] == 0, st
    assert st["differing"] > 0     # the model does differ from the exact sum


def _random_codes(shape, rng, zero_frac=0.1):
    q = rng.integers(0, 256, size=shape).astype(np.uint8)
    q[(q & 0x7F) == 0x7F] = 0x7E | (q[(q & 0x7F) == 0x7F] & 0x80)      # no NaN codes
    q[rng.random(shape) < zero_frac] = 0
    return q


def test_mfma_model_inside_bound_adversarial():
    """codes over the whole e4m3 range (subnormals, both signs, zeros) and
    scales spread over +-30 binades"""
    rng = np.random.default_rng(3)
    M, N, K = 128, 256, 1024
    qa = _random_codes((M, K), rng)
    qb = _random_codes((N, K), rng)
    sa = np.exp2(rng.integers(-30, 30, size=(M, K // 128))).astype(np.float32) * \
        rng.uniform(1, 2, size=(M, K // 128)).astype(np.float32)
    sb = np.exp2(rng.integers(-30, 30, size=(N // 128, K // 128))).astype(np.float32) * \
        rng.uniform(1, 2, size=(N // 128, K // 128)).astype(np.float32)
    acc, _ = oracle.bsgemm(qa, sa, qb, sb)
    _, cm = oracle.bsgemm(qa, sa, qb, sb, mfma=True)
    st = check(cm, acc, (qa, sa, qb, sb))
    assert st["bad"] == 0, st
    # subnormal-only operands: exponents -6, products 2^-18 .. 2^-12
    sub_a = rng.integers(0, 8, size=(M, K)).astype(np.uint8) | (rng.integers(0, 2, size=(M, K)).astype(np.uint8) << 7)
    sub_b = rng.integers(0, 8, size=(N, K)).astype(np.uint8)
    acc, _ = oracle.bsgemm(sub_a, sa, sub_b, sb)
    _, cm = oracle.bsgemm(sub_a, sa, sub_b, sb, mfma=True)
    assert check(cm, acc, (sub_a, sa, sub_b, sb))["bad"] == 0


def _planted(name, qa, sa, qb, sb):
    """the 'device' side of a planted mistake: O4m on altered inputs"""
    qa, sa, qb, sb = qa.copy(), sa.copy(), qb.copy(), sb.copy()
    if name == "b_scale_block_shifted":          # b_scale row (n/128 + 1) instead of n/128
        sb = np.roll(sb, -1, axis=0)
    elif name == "a_scale_block_shifted":        # a_scale column kb + 1
        sa = np.roll(sa, -1, axis=1)
    elif name == "k_block_dropped":              # K block 1 never accumulated
        qa[:, 128:256] = 0
    elif name == "b_rows_shifted":               # column n computed from B row n + 1
        qb = np.roll(qb, -1, axis=0)
    elif name == "b_scale_missing":              # only the A scale applied
        sb = np.ones_like(sb)
    elif name == "k_order_mismatch":             # A's K slots reversed inside each block, B's not
        M, K = qa.shape
        qa = qa.reshape(M, K // 128, 128)[:, :, ::-1].reshape(M, K).copy()
    elif name == "one_row_negated":
        qa[5] ^= 0x80
    elif name == "k_blocks_swapped_in_b":        # B's first two K blocks exchanged
        qb[:, :256] = np.concatenate([qb[:, 128:256], qb[:, :128]], axis=1)
    return oracle.bsgemm(qa, sa, qb, sb, mfma=True)[1]


@pytest.mark.parametrize("name", ["b_scale_block_shifted", "a_scale_block_shifted", "k_block_dropped",
                                  "b_rows_shifted", "b_scale_missing", "k_order_mismatch",
                                  "one_row_negated", "k_blocks_swapped_in_b"])
def test_planted_mistakes_fall_outside(name):
    qa, sa, qb, sb = quantized(256, 512, 256, seed=0)
    acc, _ = oracle.bsgemm(qa, sa, qb, sb)
    st = check(_planted(name, qa, sa, qb, sb), acc, (qa, sa, qb, sb))
    assert st["bad"] > 0, (name, st)


def test_bound_is_not_vacuous():
    """the bound stays a small fraction of the values it guards: its median
    relative width is a few bf16 steps (2^-8 each)"""
    qa, sa, qb, sb = quantized(256, 512, 2048, seed=2, heavy=True)
    acc, _ = oracle.bsgemm(qa, sa, qb, sb)
    d = bounds.BsgemmBound(qa, sa, qb, sb).rows(0, qa.shape[0])
    rel = d / np.maximum(np.abs(acc.astype(np.float64)), 1e-30)
    assert np.median(rel) < 8 * 2.0 ** -8, np.median(rel)


# ---------------------------------------------------------------------------
# mxfp8

def mx_operands(M, N, K, seed, spread):
    rng = np.random.default_rng(seed)
    qa = _random_codes((M, K), rng, 0.05)
    qb = _random_codes((N, K), rng, 0.05)
    ea = (127 + rng.integers(-spread, spread + 1, size=(M, K // 32))).astype(np.uint8)
    eb = (127 + rng.integers(-spread, spread + 1, size=(N, K // 32))).astype(np.uint8)
    return qa, ea, qb, eb


@pytest.mark.parametrize("spread", [0, 10, 40])
def test_mx_model_inside_bound(spread):
    qa, ea, qb, eb = mx_operands(128, 256, 512, seed=spread, spread=spread)
    acc, _ = oracle.mxgemm(qa, ea, qb, eb)
    _, cm = oracle.mxgemm(qa, ea, qb, eb, mfma=True)
    st = bounds.check_mxgemm(cm, acc, qa, ea, qb, eb)
    assert st["bad"] == 0, st


@pytest.mark.parametrize("name", ["scale_of_next_block", "block_dropped", "b_rows_shifted"])
def test_mx_planted_mistakes_fall_outside(name):
    qa, ea, qb, eb = mx_operands(128, 256, 512, seed=5, spread=4)
    acc, _ = oracle.mxgemm(qa, ea, qb, eb)
    qa2, ea2, qb2 = qa.copy(), ea.copy(), qb.copy()
    if name == "scale_of_next_block":
        ea2 = np.roll(ea2, -1, axis=1)
    elif name == "block_dropped":
        qa2[:, 32:64] = 0
    elif name == "b_rows_shifted":
        qb2 = np.roll(qb2, -1, axis=0)
    _, cm = oracle.mxgemm(qa2, ea2, qb2, eb, mfma=True)
    st = bounds.check_mxgemm(cm, acc, qa, ea, qb, eb)
    assert st["bad"] > 0, (name, st)


def test_row_figures_expose_an_error_that_the_norm_hides():
    """relL2 over the whole output is dominated by the few x50 rows; an error
    confined to one ordinary row shows in the worst-row and other-rows
    figures while the global figure barely moves."""
    qa, sa, qb, sb = quantized(512, 256, 256, seed=4, heavy=True)
    acc, _ = oracle.bsgemm(qa, sa, qb, sb)
    _, cm = oracle.bsgemm(qa, sa, qb, sb, mfma=True)
    clean = check(cm, acc, (qa, sa, qb, sb))
    norms = np.sum(acc.astype(np.float64) ** 2, axis=1)
    r = int(np.argsort(norms)[len(norms) // 2])      # an ordinary row
    bad = cm.copy()
    bad[r] ^= 0x0040                                  # one bf16 mantissa bit flipped across the row
    st = check(bad, acc, (qa, sa, qb, sb))
    assert st["bad"] > 0
    assert st["rel_l2_row_max"] > 50 * clean["rel_l2_row_max"] or st["rel_l2_row_max"] > 1e-2
    assert st["rel_l2_rest"] > 2 * clean["rel_l2_rest"]
    assert st["rel_l2_heavy"] == clean["rel_l2_heavy"]
    assert st["rel_l2"] < 0.2 * st["rel_l2_row_max"]
