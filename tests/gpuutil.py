"""Helpers for the GPU parity tests: device transfer, output poisoning, the
seeded workload operands (cached: several tests use the same full-size
product), and the GEMM acceptance.

GEMM acceptance rests on the pages' definition, the exact block-scale product
O4 (O11 for mxfp8): every bf16 output must lie in the interval the
instruction's truncation and rounding allow around O4's fp32 accumulator
(oracle/bounds.py derives it; tests/test_oracle_bound.py pins it).  The
relL2 against O4 is printed for every check; it is above the 3e-5 that the
pages measure between two implementations sharing the same instruction
(sglang PR 40757, "Numbers"), because O4 sums each 128-deep block exactly
and the fp8 MFMA does not.  Agreement with the instruction model O4m is
printed as a diagnostic; it is asserted only in the conformance test
(test_gpu_mfma_conformance.py)."""
import sys

import numpy as np
import torch

import block_scaled_fp8_bsgemm_amd as bs
import oracle
import synth
from oracle import bounds


def device():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    bs.load()  # fail loudly if the library is missing
    return torch.device("cuda:0")


def say(msg):
    print(f"[gpu] {msg}", file=sys.stderr, flush=True)


def to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(device())


def bf16_dev(bits):
    """uint16 bf16 bit patterns (numpy) -> torch.bfloat16 device tensor"""
    return to_dev(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)


def bits16(t):
    """device bf16 tensor -> numpy uint16 bit patterns"""
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def poison_bf16(t):
    t.view(torch.int16).fill_(0x7FC0)  # NaN
    return t


def poison_u8(t):
    t.fill_(0x7F)  # e4m3 NaN
    return t


_OPERANDS = {}
_EXACT = {}


def workload_operands(M, N, K, seed=0, heavy=True, pad_to=None):
    """The seeded operands quantized by the oracle's block quantizer (O3),
    cached per shape: (qa, sa, qb, sb)."""
    key = (M, N, K, seed, heavy, pad_to)
    if key not in _OPERANDS:
        A, B = synth.operand_fp32(M, N, K, seed=seed, heavy=heavy)
        if pad_to:
            A = synth.pad_rows(A, pad_to)
        qa, sa = oracle.quant_blocks(A, 1, 128)
        qb, sb = oracle.quant_blocks(B, 128, 128)
        _OPERANDS[key] = (qa, sa, qb, sb)
    return _OPERANDS[key]


def exact_product(qa, sa, qb, sb, key=None):
    """O4's fp32 accumulator and bf16 output, cached under `key` if given."""
    if key is not None and key in _EXACT:
        return _EXACT[key]
    r = oracle.bsgemm(qa, sa, qb, sb)
    if key is not None:
        _EXACT[key] = r
    return r


def _report(what, st, extra=""):
    say(f"{what}: vs exact relL2={st['rel_l2']:.3e} (heaviest 1% of rows {st['rel_l2_heavy']:.3e}, "
        f"other rows {st['rel_l2_rest']:.3e}, worst row {st['rel_l2_row_max']:.3e}) "
        f"differing={st['differing']}/{st['elements']}; "
        f"bound: outside={st['bad']} largest share used={st['worst_used']:.3f}{extra}")


def gemm_accept(got_bits, qa, sa, qb, sb, what, key=None, model=True):
    """Every element of the device's bf16 GEMM output [M, N] against O4 under
    the derived bound; O4m agreement printed when `model`."""
    acc, _ = exact_product(qa, sa, qb, sb, key)
    st = bounds.check_bsgemm(got_bits, acc, qa, sa, qb, sb)
    extra = ""
    if model:
        _, cm = oracle.bsgemm(qa, sa, qb, sb, mfma=True)
        extra = f"; vs MFMA model differing={int(np.count_nonzero(got_bits != cm))}"
    _report(what, st, extra)
    assert st["bad"] == 0, (what, st)
    return st


def gemm_accept_rows(got_bits, rows, qa, sa, qb, sb, what):
    """Whole output rows `rows` of a product too large for the host
    (got_bits [len(rows), N]), against O4 on those rows."""
    qa_r, sa_r = np.ascontiguousarray(qa[rows]), np.ascontiguousarray(sa[rows])
    return gemm_accept(got_bits, qa_r, sa_r, qb, sb, what, model=False)


def mx_accept(got_bits, qa, ea, qb, eb, what, model=True):
    """The mxfp8 GEMM's bf16 output against O11 under its bound; agreement
    with the scaled-MFMA model O11m printed when `model`."""
    acc, _ = oracle.mxgemm(qa, ea, qb, eb)
    st = bounds.check_mxgemm(got_bits, acc, qa, ea, qb, eb)
    extra = ""
    if model:
        _, cm = oracle.mxgemm(qa, ea, qb, eb, mfma=True)
        extra = f"; vs MFMA model differing={int(np.count_nonzero(got_bits != cm))}"
    _report(what, st, extra)
    assert st["bad"] == 0, (what, st)
    return st
