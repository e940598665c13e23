"""Calls from several host threads, each on its own HIP stream.

The library keeps no device state of its own (rings, workspaces and outputs
belong to the caller) and its host state is a thread-local error text and a
lock-guarded device-property cache, so calls on different streams must not
interfere.  Four threads (ctypes releases the interpreter lock during each
call) each run 12 steps of ring quantize -> dual quantize -> GEMM, plus a
current-scaling quantize on their own workspace, on their own stream and
buffers; every thread's outputs and ring words equal, bit for bit, the same
sequence run alone on one stream.  (That a rejected call's error text stays
in its own thread is a CPU test: tests/test_abi_cpu.py.)
"""
import threading

import pytest
import torch

import synth
from tests.gpu_util import DEV

pytestmark = pytest.mark.gpu

fp8mi = pytest.importorskip("fp8_tensor_scaled_quantize_amd")

THREADS, STEPS = 4, 12


def inputs(t):
    xs = [synth.device_gaussian((1024, 768), 1.0, torch.bfloat16, 9600 + 100 * t + s) for s in range(STEPS)]
    w = synth.device_gaussian((512, 768), 0.02, torch.bfloat16, 9700 + t)
    return xs, w


def run_sequence(xs, w):
    """The per-thread work on torch's current stream; returns host copies."""
    ring = fp8mi.new_ring(8, 1.0, DEV)
    sx, sw = torch.empty(1, device=DEV), torch.empty(1, device=DEV)
    ws = torch.empty(fp8mi.DYNAMIC_WORKSPACE_BYTES, dtype=torch.uint8, device=DEV)
    wscale = torch.full((1,), 448.0 / float(w.float().abs().max()), device=DEV)
    outs = []
    for x in xs:
        xq = fp8mi.fp8_quantize(x, fp8mi.E4M3, ring=ring, scale_inv_out=sx)
        wq, wq_t = fp8mi.fp8_quantize_dual(w, fp8mi.E4M3, scale=wscale, scale_inv_out=sw)
        y = fp8mi.fp8_mm(xq, wq, fp8mi.E4M3, fp8mi.E4M3, sx, sw)
        dq, _ = fp8mi.fp8_quantize_dynamic(x, fp8mi.E5M2, workspace=ws)
        outs.append((xq, wq_t, y.view(torch.int16), dq))
    torch.cuda.current_stream().synchronize()
    return [[t.cpu() for t in o] for o in outs], ring.cpu()


def test_threads_on_separate_streams_match_a_single_stream():
    data = [inputs(t) for t in range(THREADS)]
    reference = [run_sequence(*data[t]) for t in range(THREADS)]     # one after another, default stream
    results, errors = [None] * THREADS, [None] * THREADS

    def worker(t):
        try:
            stream = torch.cuda.Stream(device=DEV)
            with torch.cuda.stream(stream):
                results[t] = run_sequence(*data[t])
        except Exception as e:  # reported below, with the thread index
            errors[t] = e

    threads = [threading.Thread(target=worker, args=(t,)) for t in range(THREADS)]
    for th in threads:
        th.start()
    for th in threads:
        th.join(timeout=120)
    assert not any(th.is_alive() for th in threads), "a thread did not finish"
    assert errors == [None] * THREADS, errors
    for t in range(THREADS):
        (outs, ring), (ref_outs, ref_ring) = results[t], reference[t]
        assert torch.equal(ring, ref_ring), t
        for s in range(STEPS):
            for got, want in zip(outs[s], ref_outs[s]):
                assert torch.equal(got, want), (t, s)

