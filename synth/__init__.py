"""Seeded synthetic inputs for the block-scale fp8 GEMM path.

This is the one module both sides use: the oracle (in the tests) and the HIP
path (tests, smoke check, benchmark) consume the same arrays.  It draws
random numbers, shapes and scales them, and narrows fp32 draws to bf16 with
torch's own conversion; it holds none of the method's arithmetic (no fp8
encoding, no block scales, no products, no sums).

The workloads stand in for DeepSeek-V4-Pro's ``wo_b`` at TP8 with 16384-token
chunked prefill ("MORI GEMM + All-Reduce Benchmark", opening paragraph and
"Where the time goes"): real activations and weights are not available, so
the distributions below replace them.

  operand_fp32(M, N, K, seed, heavy)  A ~ N(0,1) [M,K] (optionally 1% of the
                                      rows x50), B ~ 0.02 * N(0,1) [N,K]
  partial_bands(rows, N, P, seed0)    P bf16 bands [rows,N], each N(0,1)/sqrt(P),
                                      band p drawn from seed seed0 + p
  wire_rows(rows, N, seed)            bf16 N(0,1) [rows,N]
  pad_rows(x, rows)                   append zero rows up to ``rows``
  sample_indices(M, N, count, seed)   (m, n) index pairs for sampled checks
"""
import numpy as np

# Workloads (sizes from the statement of the problem: the wo_b shard is
# [M, 7168] with K = 2048 under TP8, reduced over P = 8 ranks).
HIDDEN = 7168
K_SHARD = 2048
P_RANKS = 8

WORKLOADS = {
    "tiny": dict(M=256, N=512, K=256, heavy=False),
    "prefill4k": dict(M=4096, N=HIDDEN, K=K_SHARD, heavy=True),
    "chunk16k": dict(M=16384, N=HIDDEN, K=K_SHARD, heavy=True, bands=P_RANKS),
}


def operand_fp32(M, N, K, seed=0, heavy=True):
    """A [M,K] float32 ~ N(0,1), B [N,K] float32 ~ 0.02 * N(0,1).

    With ``heavy``, round(M/100) distinct rows of A (chosen after A is drawn)
    are multiplied by 50 so that per-block scales vary by orders of magnitude.
    """
    rng = np.random.default_rng(seed)
    A = rng.standard_normal((M, K), dtype=np.float32)
    if heavy:
        rows = rng.choice(M, size=int(round(M / 100)), replace=False)
        A[rows] *= np.float32(50.0)
    B = rng.standard_normal((N, K), dtype=np.float32) * np.float32(0.02)
    return A, B


def _to_bf16_bits(x):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def partial_bands(rows, N, P=P_RANKS, seed0=100):
    """P bf16 bit-pattern arrays [rows,N]; band p ~ N(0,1)/sqrt(P) from seed seed0+p."""
    out = []
    for p in range(P):
        rng = np.random.default_rng(seed0 + p)
        x = rng.standard_normal((rows, N), dtype=np.float32) / np.float32(np.sqrt(P))
        out.append(_to_bf16_bits(x))
    return out


def wire_rows(rows, N, seed=200):
    """bf16 bit patterns [rows,N] of N(0,1) draws (the dequantize workload)."""
    rng = np.random.default_rng(seed)
    return _to_bf16_bits(rng.standard_normal((rows, N), dtype=np.float32))


def pad_rows(x, rows):
    """x with zero rows appended up to ``rows`` (ragged M padded for the GEMM)."""
    if x.shape[0] == rows:
        return x
    out = np.zeros((rows,) + x.shape[1:], x.dtype)
    out[: x.shape[0]] = x
    return out


def sample_indices(M, N, count, seed=7):
    """``count`` (m, n) pairs: every row and column corner plus uniform draws."""
    rng = np.random.default_rng(seed)
    m = rng.integers(0, M, size=count, dtype=np.int64)
    n = rng.integers(0, N, size=count, dtype=np.int64)
    corners_m = np.array([0, 0, M - 1, M - 1], np.int64)
    corners_n = np.array([0, N - 1, 0, N - 1], np.int64)
    return np.concatenate([corners_m, m]), np.concatenate([corners_n, n])
