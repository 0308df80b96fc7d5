"""Helpers for the GPU parity tests: device transfer, output poisoning and
the comparisons used against the oracle."""
import sys

import numpy as np
import torch

import block_scaled_fp8_bsgemm_amd as bs
import oracle

# acceptance for bf16 GEMM outputs against the instruction-faithful definition
# (O4m): what is left is accumulation order only
GEMM_REL_L2 = 3e-5


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


def gemm_compare(got_bits, ref_mfma_bits, ref_exact_bits, what):
    """bf16 GEMM output against the oracle's MFMA model (O4m, or O11m for
    mxfp8; relL2 <= 3e-5) and against its exact definition (O4 / O11: no
    further than the model itself is from it)."""
    got = oracle.bf16_to_f64(got_bits)
    ref_m = oracle.bf16_to_f64(ref_mfma_bits)
    ref_e = oracle.bf16_to_f64(ref_exact_bits)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output (unwritten or NaN)"
    r_m = oracle.rel_l2(got, ref_m)
    r_e = oracle.rel_l2(got, ref_e)
    r_me = oracle.rel_l2(ref_m, ref_e)
    flips_m = int(np.count_nonzero(got_bits != ref_mfma_bits))
    flips_e = int(np.count_nonzero(got_bits != ref_exact_bits))
    say(f"{what}: vs MFMA model relL2={r_m:.3e} differing={flips_m}/{got_bits.size}; "
        f"vs exact relL2={r_e:.3e} differing={flips_e} (model vs exact {r_me:.3e})")
    assert r_m <= GEMM_REL_L2, (what, "vs MFMA model", r_m)
    assert r_e <= r_me + GEMM_REL_L2, (what, "vs exact", r_e, r_me)
    return r_m, flips_m
