"""The per-GPU wo_b step: the four library calls of one row-parallel layer's
local work, on preallocated device buffers.

  1. bsgemm_fp8   C = A x B^T as P destination-major bands of M/P rows
  2. band_reduce  band 0 of C (this GPU's own band) + P-1 partial bands that
                  stand in for the bands the other ranks would send
  3. rowq_e4m3    the reduced band -> e4m3 + per-row scale (the fp8 wire),
                  written into rows [0, M/P) of the gathered wire buffer
  4. rowdq_e4m3   the gathered wire buffer [M, N] (own rows + P-1 stand-in
                  quantized bands) -> bf16

("MORI GEMM + All-Reduce Benchmark", "Where the time goes": gemm, reduce,
quantize, dequantize; the scatter and gather transfers between them are
collectives and are not part of a single-GPU step.)  With ``fused=True``
steps 2 and 3 are one call, band_rowq_e4m3, which writes the same codes and
scales without the reduced bf16 band in memory (the pages' "Negative
results" fusion).  Buffers are allocated once in the constructor; ``step()``
only enqueues the calls on the current stream, so it can be timed or
captured.
"""
import torch

from . import band_reduce, band_rowq_e4m3, bsgemm_fp8, rowdq_e4m3, rowq_e4m3


class WoBStep:
    def __init__(self, A, a_scale, B, b_scale, partials, wire_q, wire_s, bands, fused=False):
        """A/a_scale/B/b_scale: GEMM operands on the device.
        partials: list of bands-1 bf16 [M/bands, N] tensors (the other ranks' bands).
        wire_q/wire_s: uint8 [M, N] and fp32 [M] gathered wire; rows [0, M/bands)
        are overwritten by this GPU's quantized band each step.
        fused: reduce and quantize in one call (band_rowq_e4m3)."""
        M, K = A.shape
        N = B.shape[0]
        if M % bands:
            raise ValueError("M must be a multiple of bands")
        if len(partials) != bands - 1:
            raise ValueError("need bands-1 partial bands")
        self.M, self.N, self.K, self.bands = M, N, K, bands
        self.band_rows = M // bands
        self.A, self.a_scale, self.B, self.b_scale = A, a_scale, B, b_scale
        dev = A.device
        self.C = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        self.partials = list(partials)
        self.fused = fused
        self.PHASES = self.PHASES_FUSED if fused else self.PHASES_SPLIT
        self.reduced = None if fused else torch.empty((self.band_rows, N), dtype=torch.bfloat16, device=dev)
        self.wire_q, self.wire_s = wire_q, wire_s
        self.own_q = wire_q[: self.band_rows]
        self.own_s = wire_s[: self.band_rows]
        self.out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)

    def gemm(self):
        bsgemm_fp8(self.A, self.a_scale, self.B, self.b_scale, self.C.view(-1), bands=self.bands)

    def reduce(self):
        band_reduce([self.C[: self.band_rows]] + self.partials, self.reduced)

    def quantize(self):
        rowq_e4m3(self.reduced, self.own_q, self.own_s)

    def reduce_quantize(self):
        band_rowq_e4m3([self.C[: self.band_rows]] + self.partials, self.own_q, self.own_s)

    def dequantize(self):
        rowdq_e4m3(self.wire_q, self.wire_s, self.out)

    PHASES_SPLIT = ("gemm", "reduce", "quantize", "dequantize")
    PHASES_FUSED = ("gemm", "reduce_quantize", "dequantize")

    def step(self):
        for ph in self.PHASES:
            getattr(self, ph)()
