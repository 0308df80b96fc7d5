"""Benchmark of the per-GPU wo_b step on one MI355X.

One step = the whole hot path over one batch: block-scale fp8 GEMM
(M=16384, N=7168, K=2048) written as 8 destination-major bands, the fp32
reduce of the own band with 7 stand-in partial bands fused with the per-row
e4m3 quantize of the reduced band (one kernel, the same codes and scales as
the two separate calls), and dequantize of the [16384, 7168] wire buffer.

Residency: the timed steps rotate over 4 buffer sets (activations A and
their scales, C, the stand-in bands, the wire buffer and its dequantized
output; about 3 GB in all, against a 256 MB Infinity Cache), so that no step
finds the previous step's data in a cache.  Only the weight B is shared, as
in a real layer.  `resident_step` times the same step reusing one set.

Prints ONE JSON line.  `value` is the GEMM's own rate, 2*M*N*K over the
median of its launch times measured with HIP events on the launch stream
around each GEMM inside the K timed steps (the metric names the GEMM);
`ms_per_step` is the whole step's time and `step_tflops` the step's
throughput in GEMM flops.  `phases` gives each kernel's median, min and max
over max(11, K) further steps with events around every phase (the pages time
a median of 11).  Before the W warm-up steps, 300 untimed steps bring the
clock up from idle.  `gemm_m4096` is the GEMM alone at the prefill-chunk
size M=4096 (median of 25 launches over 4 rotating outputs).  `streaming`
gives the HBM-bound kernels measured alone on rotating buffers; `mxfp8_gemm`
the mxfp8 variant alone at M=16384, N=5120, K=2048; `pipeline_sweep` the
step at M=8192 and M=20000 (padded to 20096); `gemm_k_sweep` the GEMM at
K=512..4096 fitted as fixed + per-K-block cost.  `cpu_baseline` is the CPU
oracle timed on a bounded row sample of the same workload and projected to a
full step; the same leg checks those rows of the last timed step's C against
the oracle (every element inside the bound the fp8 MFMA allows around the
exact product) and reports it as `validated`.  After that line, stderr gets
one `RESULT_JSON` record per (configuration, phase) with the median, the
rate and its roofline share; `streaming.copy_kernel` (a plain copy through
the library's streaming path) and `streaming.device_copy_runtime` (the
runtime's blit) are the practical HBM ceilings.

  python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--no-cpu-baseline]
"""
import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "blockscale fp8 GEMM TFLOP/s @16384x7168x2048 (% MFMA peak); reduce/quant GB/s"
PEAK_FP8_TFLOPS = 5000.0     # MI355X dense fp8 MFMA, published
PEAK_HBM_GBS = 8000.0        # MI355X HBM3E, published
# the pages' GEMM-alone time at this shape on MI355X ("MORI GEMM + All-Reduce
# Benchmark", "Headline": gemm-only, median of 11, per rank of an 8-GPU run)
PAGES_GEMM_ONLY_US = 369.4
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "bsgemm_m16384_traffic.json")
HOST_LEAD_CYCLES = 4_000_000  # spin-kernel cycles (~2 ms) queued ahead of a timed loop
CLOCK_RAMP_STEPS = 300       # untimed steps before the warm-up, to bring the clock up
NSETS = 4                    # rotating buffer sets of the timed step


def kernel_hash():
    """Hash of the GEMM kernel's source with comments and whitespace removed, so
    that the stored counter readings stay tied to the code, not its comments."""
    import re
    h = hashlib.sha256()
    for f in ("gemm.hip", "codec.hpp"):
        with open(os.path.join(ROOT, "block_scaled_fp8_bsgemm_amd", "csrc", f)) as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def load_traffic():
    """HBM bytes per GEMM launch from the committed counter runs, if they were
    taken on the current kernel source; otherwise None."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_hash") != kernel_hash():
        return None
    return t.get("traffic_bytes")


def say(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def stats_us(ms_list):
    us = [x * 1e3 for x in ms_list]
    return {"median_us": statistics.median(us), "min_us": min(us), "max_us": max(us), "n": len(us)}


def build_inputs(M, N, K, P, dev, M_real=None):
    """The seeded set: GEMM operands for M rows (the first M_real drawn, the
    rest zero padding; quantized on the device, bit-identical to the oracle's
    block quantizer), the P-1 stand-in bands and the quantized wire buffer."""
    import numpy as np
    import torch
    import block_scaled_fp8_bsgemm_amd as bs
    import synth

    A, B = synth.operand_fp32(M_real or M, N, K, seed=0, heavy=True)
    A = synth.pad_rows(A, M)
    dA32 = torch.from_numpy(A).to(dev)
    dB32 = torch.from_numpy(B).to(dev)
    qa, sa = bs.blockq_e4m3(dA32, 1)
    qb, sb = bs.blockq_e4m3(dB32, 128)
    del dA32, dB32
    band_rows = M // P
    parts = [torch.from_numpy(p.view(np.int16)).to(dev).view(torch.bfloat16)
             for p in synth.partial_bands(band_rows, N, P=P, seed0=100)[1:]]
    wire = torch.from_numpy(synth.wire_rows(M, N, seed=200).view(np.int16)).to(dev).view(torch.bfloat16)
    wq, ws = bs.rowq_e4m3(wire)
    del wire
    torch.cuda.synchronize()
    return qa, sa, qb, sb, parts, wq, ws


def device_set(M, N, K, P, dev, seed):
    """A further rotating set drawn on the device from a seeded generator with
    the same distributions: A ~ N(0,1) with 1% of rows x50, stand-in bands
    N(0,1)/sqrt(P) in bf16, wire rows N(0,1) in bf16 quantized per row."""
    import torch
    import block_scaled_fp8_bsgemm_amd as bs
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    A = torch.randn(M, K, device=dev, generator=g)
    heavy = torch.randperm(M, device=dev, generator=g)[: round(M / 100)]
    A[heavy] *= 50.0
    qa, sa = bs.blockq_e4m3(A, 1)
    del A
    band_rows = M // P
    parts = [(torch.randn(band_rows, N, device=dev, generator=g) / P ** 0.5).to(torch.bfloat16)
             for _ in range(P - 1)]
    wire = torch.randn(M, N, device=dev, generator=g).to(torch.bfloat16)
    wq, ws = bs.rowq_e4m3(wire)
    del wire
    return qa, sa, parts, wq, ws


class Rotation:
    """Steps over several buffer sets, set i % n for the i-th call."""

    def __init__(self, steps):
        self.steps = steps
        self.i = 0
        self.PHASES = steps[0].PHASES

    def next(self):
        s = self.steps[self.i % len(self.steps)]
        self.i += 1
        return s


def ramp_clock(rot, n=CLOCK_RAMP_STEPS):
    """`n` untimed steps (≈ 0.1 s at the default shape) before the warm-up: the
    clock comes up from idle over milliseconds, and a few warm-up steps alone
    leave the first timed steps at a lower clock (≈ 15 % slower GEMM)."""
    import torch
    for _ in range(n):
        rot.next().step()
    torch.cuda.synchronize()


def time_steps(rot, steps, warmup):
    """W untimed warm-up steps, then exactly `steps` timed steps.  Inside the
    timed region only the GEMM is bracketed by events (on the launch stream,
    for the roofline); the per-phase breakdown comes from a second, separate
    pass of max(11, steps) steps with events around every phase, since eight
    events per step add ≈ 6 % to a step."""
    import torch
    for _ in range(warmup):
        rot.next().step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    t0 = time.perf_counter()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    gemm_ev = []
    start.record(stream)
    last = None
    for _ in range(steps):
        st = rot.next()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        st.gemm()
        e1.record(stream)
        gemm_ev.append((e0, e1))
        for ph in st.PHASES[1:]:
            getattr(st, ph)()
        last = st
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    total_ms = start.elapsed_time(end)
    gemm_ms = [a.elapsed_time(b) for a, b in gemm_ev]

    nph = max(11, steps)
    ev = {ph: [] for ph in rot.PHASES}
    for _ in range(nph):
        st = rot.next()
        for ph in st.PHASES:
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            getattr(st, ph)()
            e1.record(stream)
            ev[ph].append((e0, e1))
    torch.cuda.synchronize()
    phase_ms = {ph: [a.elapsed_time(b) for a, b in ev[ph]] for ph in rot.PHASES}
    return total_ms / steps, gemm_ms, phase_ms, wall, last


def phase_report(phase_ms, flops, bytes_of):
    out = {}
    for ph, ms in phase_ms.items():
        s = stats_us(ms)
        t = s["median_us"] * 1e-6
        if ph == "gemm":
            s["TFLOP/s"] = flops / t / 1e12
            s["frac_fp8_peak"] = s["TFLOP/s"] / PEAK_FP8_TFLOPS
        else:
            s["bytes"] = bytes_of[ph]
            s["GB/s"] = bytes_of[ph] / t / 1e9
            s["frac_hbm"] = s["GB/s"] / PEAK_HBM_GBS
        out[ph] = s
    return out


def streaming_rates(M, N, P, dev, iters=20):
    """band_reduce / rowq / rowdq / actq alone, rotating over buffer sets larger
    than the Infinity Cache."""
    import torch
    import block_scaled_fp8_bsgemm_amd as bs
    band_rows = M // P
    out = {}

    def timed(fn, nsets):
        for i in range(nsets):
            fn(i)
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        # a ~1 ms spin ahead of the first event lets the host queue every
        # timed call before the GPU reaches it, so the events see the kernels
        # back to back and not the Python call overhead between them
        torch.cuda._sleep(HOST_LEAD_CYCLES)
        e0.record()
        for i in range(iters):
            fn(i % nsets)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / iters * 1e-3

    def rec(t, b, **extra):
        d = {"us": t * 1e6, "bytes": b, "GB/s": b / t / 1e9, "frac_hbm": b / t / 1e9 / PEAK_HBM_GBS}
        d.update(extra)
        return d

    # reduce: 8 x [2048,7168] bf16 in, one out: 264 MB per call; 5 sets
    nset = 5
    red_in = [[torch.randn(band_rows, N, device=dev).to(torch.bfloat16) for _ in range(P)] for _ in range(nset)]
    red_out = [torch.empty(band_rows, N, dtype=torch.bfloat16, device=dev) for _ in range(nset)]
    t = timed(lambda i: bs.band_reduce(red_in[i], red_out[i]), nset)
    out["band_reduce"] = rec(t, (P + 1) * band_rows * N * 2)
    # rowq: [2048,7168] bf16 -> u8 + scales: 44 MB per call; 8 sets (352 MB: more
    # than the Infinity Cache, few enough pages to keep the TLB warm)
    nset = 8
    rq_in = [red_out[i % len(red_out)] if i < len(red_out) else torch.randn(band_rows, N, device=dev).to(torch.bfloat16)
             for i in range(nset)]
    rq_q = [torch.empty(band_rows, N, dtype=torch.uint8, device=dev) for _ in range(nset)]
    rq_s = [torch.empty(band_rows, dtype=torch.float32, device=dev) for _ in range(nset)]
    nset_red = len(red_in)
    t = timed(lambda i: bs.rowq_e4m3(rq_in[i], rq_q[i], rq_s[i]), nset)
    out["rowq_e4m3"] = rec(t, band_rows * N * 3 + band_rows * 4)
    # the fused reduce + quantize of the same band (the pages' negative result):
    # reads the P parts once, writes codes and scales; compare with band_reduce
    # + rowq_e4m3 above
    t = timed(lambda i: bs.band_rowq_e4m3(red_in[i], rq_q[i], rq_s[i]), nset_red)
    out["band_rowq_e4m3"] = rec(t, P * band_rows * N * 2 + band_rows * N + band_rows * 4,
                                separate_us=out["band_reduce"]["us"] + out["rowq_e4m3"]["us"])
    # rowdq: [16384,7168] u8 -> bf16: 352 MB per call; 4 sets
    nset = 4
    dq_q = [torch.randint(0, 0x7E, (M, N), dtype=torch.uint8, device=dev) for _ in range(nset)]
    dq_s = [torch.rand(M, device=dev) for _ in range(nset)]
    dq_y = [torch.empty(M, N, dtype=torch.bfloat16, device=dev) for _ in range(nset)]
    del rq_in, rq_q, rq_s, red_in
    t = timed(lambda i: bs.rowdq_e4m3(dq_q[i], dq_s[i], dq_y[i]), nset)
    out["rowdq_e4m3"] = rec(t, M * N * 3 + M * 4)
    del dq_q, dq_s, dq_y
    # actq: the bf16 activation [M,K] -> e4m3 + [M,K/128] scales (the GEMM's A);
    # 102 MB per call; 4 sets
    nset, K = 4, 2048
    aq_x = [torch.randn(M, K, device=dev).to(torch.bfloat16) for _ in range(nset)]
    aq_q = [torch.empty(M, K, dtype=torch.uint8, device=dev) for _ in range(nset)]
    aq_s = [torch.empty(M, K // 128, dtype=torch.float32, device=dev) for _ in range(nset)]
    t = timed(lambda i: bs.actq_e4m3(aq_x[i], aq_q[i], aq_s[i]), nset)
    out["actq_e4m3"] = rec(t, M * K * 3 + M * (K // 128) * 4)
    # mxq: the bf16 operand [M,K] -> e4m3 + [M,K/32] E8M0 bytes (mxgemm's A);
    # 101 MB per call; 4 sets
    mq_s = [torch.empty(M, K // 32, dtype=torch.uint8, device=dev) for _ in range(nset)]
    t = timed(lambda i: bs.mxq_e4m3(aq_x[i], aq_q[i], mq_s[i]), nset)
    out["mxq_e4m3"] = rec(t, M * K * 3 + M * (K // 32))
    del aq_x, aq_q, aq_s, mq_s
    torch.cuda.empty_cache()
    # practical ceilings: a plain copy through this library's streaming path
    # (band_reduce of a single part: 16-byte non-temporal loads and stores,
    # bf16 in and the same bf16 out), [16384,7168] bf16 = 235 MB per call, 2
    # sets; and the runtime's device copy (a blit kernel), 512 MiB per call
    nset = 2
    cp_in = [torch.randn(M, N, device=dev).to(torch.bfloat16) for _ in range(nset)]
    cp_out = [torch.empty(M, N, dtype=torch.bfloat16, device=dev) for _ in range(nset)]
    t = timed(lambda i: bs.band_reduce([cp_in[i]], cp_out[i]), nset)
    out["copy_kernel"] = rec(t, 2 * M * N * 2)
    del cp_in, cp_out
    # the same copy at the row quantizer's size, [2048,7168] bf16 (59 MB per
    # call), over 8 sets: the ceiling for a kernel of that size
    nset = 8
    cp_in = [torch.randn(band_rows, N, device=dev).to(torch.bfloat16) for _ in range(nset)]
    cp_out = [torch.empty(band_rows, N, dtype=torch.bfloat16, device=dev) for _ in range(nset)]
    t = timed(lambda i: bs.band_reduce([cp_in[i]], cp_out[i]), nset)
    out["copy_kernel_band"] = rec(t, 2 * band_rows * N * 2)
    del cp_in, cp_out
    nset = 2
    n = 1 << 27
    cp_src = [torch.ones(n, dtype=torch.float32, device=dev) for _ in range(nset)]
    cp_dst = [torch.empty(n, dtype=torch.float32, device=dev) for _ in range(nset)]
    t = timed(lambda i: cp_dst[i].copy_(cp_src[i]), nset)
    out["device_copy_runtime"] = rec(t, 2 * n * 4)
    del cp_src, cp_dst
    torch.cuda.empty_cache()
    return out


def gemm_alone(dev, M, N, K, bands, qb, sb, launches=25, seed=31):
    """The GEMM alone at M rows (seeded A drawn on the device, the benchmark's
    weight), C rotating over 4 outputs; 100 untimed launches, then `launches`
    launches each bracketed by events on the launch stream."""
    import torch
    import block_scaled_fp8_bsgemm_amd as bs
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    A = torch.randn(M, K, device=dev, generator=g)
    A[torch.randperm(M, device=dev, generator=g)[: round(M / 100)]] *= 50.0
    qa, sa = bs.blockq_e4m3(A, 1)
    del A
    Cs = [torch.empty(M * N, dtype=torch.bfloat16, device=dev) for _ in range(4)]
    s = torch.cuda.current_stream()
    for i in range(100):
        bs.bsgemm_fp8(qa, sa, qb, sb, Cs[i % 4], bands=bands)
    torch.cuda.synchronize()
    torch.cuda._sleep(HOST_LEAD_CYCLES)
    ev = []
    for i in range(launches):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(s)
        bs.bsgemm_fp8(qa, sa, qb, sb, Cs[i % 4], bands=bands)
        e1.record(s)
        ev.append((e0, e1))
    torch.cuda.synchronize()
    st = stats_us([a.elapsed_time(b) for a, b in ev])
    tf = 2.0 * M * N * K / (st["median_us"] * 1e-6) / 1e12
    st.update({"M": M, "N": N, "K": K, "bands": bands, "TFLOP/s": tf, "frac_fp8_peak": tf / PEAK_FP8_TFLOPS})
    del qa, sa, Cs
    torch.cuda.empty_cache()
    return st


def pipeline_sweep(N, K, P, dev, steps=11, warmup=3):
    """The step at the sweep's other sizes (M=8192, and M=20000 zero-padded to
    20096 = 157 * 128): time per step and median per phase, HIP events as
    above (one buffer set each)."""
    import torch
    from block_scaled_fp8_bsgemm_amd.pipeline import WoBStep
    out = {}
    for M_real in (8192, 20000):
        M = -(-M_real // 128) * 128
        qa, sa, qb, sb, parts, wq, ws = build_inputs(M, N, K, P, dev, M_real=M_real)
        rot = Rotation([WoBStep(qa, sa, qb, sb, parts, wq, ws, P, fused=True)])
        ramp_clock(rot, 100)
        ms, gemm_ms, phase_ms, _, _ = time_steps(rot, steps, warmup)
        gm = statistics.median(gemm_ms)
        out[str(M_real)] = {"M_padded": M, "steps": steps, "us_per_step": ms * 1e3,
                            "phases_median_us": {k: statistics.median(v) * 1e3 for k, v in phase_ms.items()},
                            "gemm_TFLOP/s": 2.0 * M * N * K / (gm * 1e-3) / 1e12}
        del rot, qa, sa, qb, sb, parts, wq, ws
        torch.cuda.empty_cache()
    return out


def gemm_k_sweep(dev, iters=10):
    """The blockscale GEMM at M=16384, N=7168, 8 bands and K = 512 .. 4096,
    fitted as t = fixed + per_kblock * K/128 (the decomposition the MORI
    benchmark page uses to compare GEMMs, "Negative results": a CK-shaped
    kernel).  Operands: device N(0,1) / 0.02 N(0,1) draws, block-quantized."""
    import numpy as np
    import torch
    import block_scaled_fp8_bsgemm_amd as bs
    M, N = 16384, 7168
    g = torch.Generator(device=dev)
    g.manual_seed(11)
    Ks, ts = [512, 1024, 2048, 4096], []
    C = torch.empty(M * N, dtype=torch.bfloat16, device=dev)
    for K in Ks:
        qa, sa = bs.blockq_e4m3(torch.randn(M, K, device=dev, generator=g), 1)
        qb, sb = bs.blockq_e4m3(0.02 * torch.randn(N, K, device=dev, generator=g), 128)
        for _ in range(100):   # untimed: bring the clock up, as for the step
            bs.bsgemm_fp8(qa, sa, qb, sb, C, bands=8)
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda._sleep(HOST_LEAD_CYCLES)
        e0.record()
        for _ in range(iters):
            bs.bsgemm_fp8(qa, sa, qb, sb, C, bands=8)
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1) / iters * 1e3)
        del qa, sa, qb, sb
    kb = np.array(Ks, dtype=np.float64) / 128
    per, fixed = np.polyfit(kb, np.array(ts), 1)
    torch.cuda.empty_cache()
    return {"M": M, "N": N, "K": Ks, "us": ts, "fixed_us": float(fixed), "per_kblock_us": float(per),
            "pages_mori_gemm": {"fixed_us": 51.6, "per_kblock_us": 20.9},
            "pages_ck_gemm": {"fixed_us": 66.0, "per_kblock_us": 14.5}}


def mx_gemm_rate(dev, iters=20):
    """The mxfp8 variant of the GEMM alone at M=16384, N=5120, K=2048 (one
    band), seeded random codes with E8M0 scales around 2^0; 100 untimed
    launches first, as the step's clock ramp."""
    import torch
    import block_scaled_fp8_bsgemm_amd as bs
    M, N, K = 16384, 5120, 2048
    g = torch.Generator(device=dev)
    g.manual_seed(7)
    qa = torch.randint(0, 0x7E, (M, K), dtype=torch.uint8, device=dev, generator=g)
    qa |= torch.randint(0, 2, (M, K), dtype=torch.uint8, device=dev, generator=g) << 7
    qb = torch.randint(0, 0x7E, (N, K), dtype=torch.uint8, device=dev, generator=g)
    qb |= torch.randint(0, 2, (N, K), dtype=torch.uint8, device=dev, generator=g) << 7
    ea = torch.randint(117, 128, (M, K // 32), dtype=torch.uint8, device=dev, generator=g)
    eb = torch.randint(117, 128, (N, K // 32), dtype=torch.uint8, device=dev, generator=g)
    C = torch.empty(M * N, dtype=torch.bfloat16, device=dev)
    s = torch.cuda.current_stream(dev)
    for _ in range(100):
        bs.mxgemm_fp8(qa, ea, qb, eb, C, stream=s)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    torch.cuda._sleep(HOST_LEAD_CYCLES)
    e0.record(s)
    for _ in range(iters):
        bs.mxgemm_fp8(qa, ea, qb, eb, C, stream=s)
    e1.record(s)
    torch.cuda.synchronize()
    t = e0.elapsed_time(e1) / iters * 1e-3
    tf = 2.0 * M * N * K / t / 1e12
    del qa, qb, ea, eb, C
    torch.cuda.empty_cache()
    return {"kernel": "mxgemm_persistent_kernel", "M": M, "N": N, "K": K, "us": t * 1e6, "TFLOP/s": tf,
            "frac_fp8_peak": tf / PEAK_FP8_TFLOPS, "pages_gemm_only_us": 180.2}


def cpu_baseline(ops, c_dev, M, N, K, P, target_s=10.0):
    """The oracle (test infrastructure, not tuned) on a bounded sample of the
    same workload: the GEMM on the first R rows of the operands the timed
    step used (R sized so that one call takes about target_s), the reduce and
    quantize on one full band and the dequantize on one band's rows;
    projected to one full step.  The same R rows of the last timed step's C
    are then checked against the oracle's exact product, every element
    inside the bound the fp8 MFMA allows (oracle/bounds.py): `validated`."""
    import numpy as np
    import oracle
    import synth
    from oracle import bounds

    qa, sa, qb, sb = ops

    def gemm_rows(R):
        t0 = time.perf_counter()
        acc, _ = oracle.bsgemm(qa[:R], sa[:R], qb, sb)
        t = time.perf_counter() - t0
        say(f"cpu_baseline: oracle GEMM on {R} rows took {t:.2f} s")
        return t, acc

    # a short probe sizes the timed sample to about target_s
    R = 128
    tg, acc = gemm_rows(R)
    if tg < target_s:
        R = min(M, max(R, int(R * target_s / max(tg, 1e-3)) // 128 * 128))
        tg, acc = gemm_rows(R)
    band_rows = M // P
    parts = synth.partial_bands(band_rows, N, P=P, seed0=100)
    t0 = time.perf_counter()
    red = oracle.band_reduce(parts)
    tr = time.perf_counter() - t0
    t0 = time.perf_counter()
    oracle.rowq(red)
    tq = time.perf_counter() - t0
    wq, ws = oracle.rowq(synth.wire_rows(band_rows, N, seed=200))
    t0 = time.perf_counter()
    oracle.rowdq(wq, ws)
    td = (time.perf_counter() - t0) * (M / band_rows)
    step_s = tg * (M / R) + tr + tq + td
    flops = 2.0 * M * N * K
    base = {"value": flops / step_s / 1e12, "unit": "TFLOP/s", "cores": oracle.threads(), "kind": "oracle",
            "sample": f"GEMM on the first {R} of {M} rows ({tg:.2f} s, scaled x{M / R:.2f}); reduce and quantize "
                      f"of one full [{band_rows},{N}] band ({tr:.2f} s, {tq:.2f} s); dequantize of "
                      f"{band_rows} rows scaled x{M // band_rows} ({td:.2f} s projected)",
            "projected_step_s": step_s, "projected_gemm_s": tg * (M / R),
            "projected_reduce_quantize_s": tr + tq, "projected_dequantize_s": td}
    t0 = time.perf_counter()
    st = bounds.check_bsgemm(c_dev[:R], acc, qa[:R], sa[:R], qb, sb)
    say(f"validated {R} rows in {time.perf_counter() - t0:.1f} s: {st}")
    val = {"ok": st["bad"] == 0, "rows": R, "elements": st["elements"], "outside_bound": st["bad"],
           "rel_l2_vs_exact": st["rel_l2"], "rel_l2_heaviest_1pct_rows": st["rel_l2_heavy"],
           "rel_l2_other_rows": st["rel_l2_rest"], "rel_l2_worst_row": st["rel_l2_row_max"],
           "bf16_differing_from_exact": st["differing"],
           "check": "every element of the last timed step's C on these rows inside the interval the fp8 "
                    "MFMA's truncation and rounding allow around the oracle's exact product"}
    return base, val


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def result_records(rec):
    """One record per (configuration, phase) of the workload statement, with the
    measured median, rate and roofline share; printed on stderr after the
    JSON line (stdout carries that one line only).  Fields the bench does not
    measure are null (bitexactness is the tests' job; the clock comes from
    the counter profiles)."""
    cores = (rec.get("cpu_baseline") or {}).get("cores") or os.cpu_count()
    common = {"host_cores": cores, "cpu_model": cpu_model(), "sclk_mhz": None, "bitexact": None}
    val = rec.get("validated") or {}
    oracle_s = (rec.get("cpu_baseline") or {}).get("projected_step_s")
    out = []

    def add(config, phase, M, N, K, us, tflops=None, gbps=None, pct=None, **kw):
        r = {"config": config, "phase": phase, "M": M, "N": N, "K": K, "time_us_median": us,
             "tflops": tflops, "gbps": gbps, "pct_roofline": pct, "rel_l2": None, "validated": None,
             "oracle_time_s": None}
        r.update(common)
        r.update(kw)
        out.append(r)

    ph = rec["phases"]
    cb = rec.get("cpu_baseline") or {}
    add("full_chunk_16384", "gemm", 16384, 7168, 2048, ph["gemm"]["median_us"],
        tflops=ph["gemm"]["TFLOP/s"], pct=100 * ph["gemm"]["frac_fp8_peak"],
        rel_l2=val.get("rel_l2_vs_exact"), validated=val.get("ok"), oracle_time_s=cb.get("projected_gemm_s"))
    add("reduce_wire_16384", "reduce_quantize", 2048, 7168, None, ph["reduce_quantize"]["median_us"],
        gbps=ph["reduce_quantize"]["GB/s"], pct=100 * ph["reduce_quantize"]["frac_hbm"],
        oracle_time_s=cb.get("projected_reduce_quantize_s"))
    add("reduce_wire_16384", "dequantize", 16384, 7168, None, ph["dequantize"]["median_us"],
        gbps=ph["dequantize"]["GB/s"], pct=100 * ph["dequantize"]["frac_hbm"],
        oracle_time_s=cb.get("projected_dequantize_s"))
    add("full_chunk_16384", "step", 16384, 7168, 2048, rec["ms_per_step"] * 1e3, tflops=rec["step_tflops"],
        oracle_time_s=oracle_s)
    if "gemm_m4096" in rec:
        g = rec["gemm_m4096"]
        add("prefill_chunk_4096", "gemm", 4096, 7168, 2048, g["median_us"], tflops=g["TFLOP/s"],
            pct=100 * g["frac_fp8_peak"])
    for name, d in (rec.get("streaming") or {}).items():
        rows, N = {"rowdq_e4m3": (16384, 7168), "actq_e4m3": (16384, 2048), "mxq_e4m3": (16384, 2048),
                   "copy_kernel": (16384, 7168), "copy_kernel_band": (2048, 7168),
                   "device_copy_runtime": (None, None)}.get(name, (2048, 7168))
        add("hbm_ceiling" if "copy" in name else "streaming_alone", name, rows, N, None, d["us"],
            gbps=d["GB/s"], pct=100 * d["frac_hbm"])
    if "mxfp8_gemm" in rec:
        m = rec["mxfp8_gemm"]
        add("mxfp8_16384x5120", "gemm", m["M"], m["N"], m["K"], m["us"], tflops=m["TFLOP/s"],
            pct=100 * m["frac_fp8_peak"])
    for key, d in (rec.get("pipeline_sweep") or {}).items():
        Mp = d["M_padded"]
        for phase, us in d["phases_median_us"].items():
            kw = {"tflops": 2.0 * Mp * 7168 * 2048 / (us * 1e-6) / 1e12} if phase == "gemm" else {}
            add(f"pipeline_{key}", phase, Mp, 7168, 2048, us, **kw)
        add(f"pipeline_{key}", "step", Mp, 7168, 2048, d["us_per_step"])
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-streaming", action="store_true")
    ap.add_argument("--calib-copy", action="store_true",
                    help="after the steps, copy 1 GiB device-to-device once (a plain copy kernel of "
                         "known size, for scaling the HBM byte counters of a profiler run)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py runs on exactly one GPU: this build has no multi-GPU path "
              "(the collectives between ranks are out of scope); use --gpus 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import block_scaled_fp8_bsgemm_amd as bs
    from block_scaled_fp8_bsgemm_amd.pipeline import WoBStep

    bs.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    M, N, K, P = 16384, 7168, 2048, 8
    say(f"building inputs M={M} N={N} K={K} P={P}, {NSETS} rotating sets")
    qa, sa, qb, sb, parts, wq, ws = build_inputs(M, N, K, P, dev)
    sets = [(qa, sa, parts, wq, ws)] + [device_set(M, N, K, P, dev, 1000 + i) for i in range(1, NSETS)]
    torch.cuda.synchronize()
    rot = Rotation([WoBStep(a, s_a, qb, sb, pt, q, s, P, fused=True) for a, s_a, pt, q, s in sets])
    ramp_clock(rot)
    say(f"timing {args.steps} steps after {args.warmup} warmup")
    ms, gemm_ms, phase_ms, wall, last = time_steps(rot, args.steps, args.warmup)
    # the last timed step's C, for the oracle check in the cpu_baseline leg
    # (time_steps' phase pass reused the sets, but C of a set only ever holds
    # that set's product)
    last_ops = (last.A.cpu().numpy(), last.a_scale.cpu().numpy(), qb.cpu().numpy(), sb.cpu().numpy())
    last_c = last.C.view(torch.int16).cpu().numpy().view(np.uint16).reshape(M, N)

    say("the same step on one resident buffer set, and with reduce and quantize as two calls")
    res = Rotation([rot.steps[0]])
    ramp_clock(res, 100)
    ms_r, gemm_r, phase_r, _, _ = time_steps(res, args.steps, args.warmup)
    unf = Rotation([WoBStep(a, s_a, qb, sb, pt, q, s, P) for a, s_a, pt, q, s in sets])
    ramp_clock(unf, 100)
    ms_u, gemm_u, phase_u, _, _ = time_steps(unf, args.steps, args.warmup)
    del unf, res

    flops = 2.0 * M * N * K
    band_rows = M // P
    bytes_of = {
        "reduce_quantize": P * band_rows * N * 2 + band_rows * N + band_rows * 4,
        "reduce": P * band_rows * N * 2 + band_rows * N * 2,
        "quantize": band_rows * N * 2 + band_rows * N + band_rows * 4,
        "dequantize": M * N + M * 4 + M * N * 2,
    }
    gemm_med = statistics.median(gemm_ms)
    gemm_tflops = flops / (gemm_med * 1e-3) / 1e12
    traffic = load_traffic()
    rec = {
        "metric": METRIC,
        "value": gemm_tflops,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": gemm_tflops / (flops / (PAGES_GEMM_ONLY_US * 1e-6) / 1e12),
        "dtype": "e4m3",
        "data": "synthetic",
        "config": {"workload": "wo_b per-GPU step (blockscale fp8 GEMM + 8-band epilogue, band reduce P=8 "
                               "fused with row e4m3 quantize, dequantize); value = the GEMM's own rate",
                   "M": M, "N": N, "K": K, "P": P, "bands": P, "rotating_sets": NSETS},
        "roofline": {"bound": "mfma", "achieved": gemm_tflops, "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s",
                     "frac": gemm_tflops / PEAK_FP8_TFLOPS, "traffic": traffic,
                     "kernel": "bsgemm_persistent_kernel", "algorithmic_flop_per_launch": flops,
                     "launch_us": stats_us(gemm_ms)},
        "step_tflops": flops / (ms * 1e-3) / 1e12,
        "phases": phase_report(phase_ms, flops, bytes_of),
        "resident_step": {"ms_per_step": ms_r, "gemm_median_us": statistics.median(gemm_r) * 1e3,
                          "phases": phase_report(phase_r, flops, bytes_of)},
        "unfused_step": {"ms_per_step": ms_u, "gemm_median_us": statistics.median(gemm_u) * 1e3,
                         "phases": phase_report(phase_u, flops, bytes_of)},
        "pages_context": {"gemm_only_us": PAGES_GEMM_ONLY_US, "per_layer_us": {"gemm": 438.2, "reduce": 42.5,
                                                                  "quantize": 11.8, "dequantize": 61.0},
                          "note": "8-GPU pipeline, per rank; context only"},
        "wall_s_timed": wall,
        "validated": None,
    }
    if args.calib_copy:
        src = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        say("calibration copy: 1073741824 B read, 1073741824 B written")
        del src, dst
    if not args.no_streaming:
        del rot, sets, parts, wq, ws, last
        torch.cuda.empty_cache()
        say("the GEMM alone at M=4096")
        rec["gemm_m4096"] = gemm_alone(dev, 4096, N, K, 1, qb, sb)
        say("streaming kernels alone (rotating buffers)")
        rec["streaming"] = streaming_rates(M, N, P, dev)
        say("mxfp8 GEMM alone")
        rec["mxfp8_gemm"] = mx_gemm_rate(dev)
        say("GEMM K sweep")
        rec["gemm_k_sweep"] = gemm_k_sweep(dev)
        say("pipeline sweep M=8192, 20000")
        rec["pipeline_sweep"] = pipeline_sweep(N, K, P, dev)
    if not args.no_cpu_baseline:
        say("cpu_baseline (oracle on a row sample) and the check of the last step's C")
        rec["cpu_baseline"], rec["validated"] = cpu_baseline(last_ops, last_c, M, N, K, P)
    print(json.dumps(rec), flush=True)
    for r in result_records(rec):
        print("RESULT_JSON " + json.dumps(r), file=sys.stderr, flush=True)


if __name__ == "__main__":
    main()
