"""The boundary's stream contract on the device: every call enqueues on the
stream it is given, ordered after earlier work on that stream, and the
step's calls can be captured into a HIP graph and replayed (no allocation,
synchronisation or memset inside them).  Results are compared with the same
calls run eagerly on the default stream."""
import numpy as np
import pytest
import torch

import block_scaled_fp8_bsgemm_amd as bs
import oracle
import synth
from block_scaled_fp8_bsgemm_amd.pipeline import WoBStep
from gpuutil import bf16_dev, bits16, device, poison_bf16, say, to_dev

pytestmark = pytest.mark.gpu

SPIN_CYCLES = 200_000_000   # ~0.1 s of torch's spin kernel


def small_step(M=1024, N=512, K=512, bands=8, fused=False):
    band_rows = M // bands
    A, B = synth.operand_fp32(M, N, K, seed=4, heavy=True)
    qa, sa = oracle.quant_blocks(A, 1, 128)
    qb, sb = oracle.quant_blocks(B, 128, 128)
    parts = synth.partial_bands(band_rows, N, P=bands, seed0=100)[1:]
    wq, ws = oracle.rowq(synth.wire_rows(M, N, seed=200))
    return WoBStep(to_dev(qa), to_dev(sa), to_dev(qb), to_dev(sb), [bf16_dev(p) for p in parts],
                   to_dev(wq), to_dev(ws), bands, fused=fused)


def outputs(step):
    reduced = [] if step.reduced is None else [bits16(step.reduced)]
    return [bits16(step.C)] + reduced + [step.own_q.cpu().numpy(),
                                         step.own_s.cpu().numpy().view(np.uint32), bits16(step.out)]


def test_calls_follow_their_stream():
    """Inputs written on a side stream, the GEMM and the reduce enqueued on it
    right after, the results read after that stream alone is synchronised."""
    dev = device()
    say("side-stream ordering")
    ref = small_step()
    ref.step()
    torch.cuda.synchronize()
    want = outputs(ref)

    step = small_step()
    qa_host = step.A.clone()
    step.A.zero_()
    torch.cuda.synchronize()
    s = torch.cuda.Stream(device=dev)
    with torch.cuda.stream(s):
        torch.cuda._sleep(SPIN_CYCLES // 4)      # the copy below lands late
        step.A.copy_(qa_host, non_blocking=True)
        poison_bf16(step.C)
        step.step()                              # every call takes the current stream, s
    s.synchronize()
    got = outputs(step)
    for g, w in zip(got, want):
        assert np.array_equal(g, w)


@pytest.mark.parametrize("fused", [False, True])
def test_step_graph_capture_and_replay(fused):
    """The whole step (split, or with the fused reduce + quantize the benchmark
    runs) captured into a graph on a side stream and replayed three times, with
    eager work on the same buffers between replays; every replay equals the
    eager result."""
    dev = device()
    say(f"graph capture of the step (fused={fused})")
    step = small_step(fused=fused)
    step.step()
    torch.cuda.synchronize()
    want = outputs(step)

    s = torch.cuda.Stream(device=dev)
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step.step()                               # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        step.step()
    torch.cuda.synchronize()
    for r in range(3):
        poison_bf16(step.C)
        if step.reduced is not None:
            poison_bf16(step.reduced)
        poison_bf16(step.out)
        step.own_q.fill_(0x7F)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = outputs(step)
        for k, (a, b) in enumerate(zip(got, want)):
            assert np.array_equal(a, b), (r, k)
        step.step()                               # eager work between replays
        torch.cuda.synchronize()
