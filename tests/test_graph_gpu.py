"""HIP graph capture of a whole delayed-scaling training step.

Every library call is ordered on torch's current stream, allocates no device
memory and never waits on the host, so one fp8 linear step can be captured
once and replayed.  The step is: x, W and dY quantized into both layouts with
their rings folding in-kernel, the forward GEMM with bias, the dY quantize
with the fused bias gradient, and both backward GEMMs.  A replay re-runs the
captured kernels on whatever the static input buffers hold, and the rings
carry the delayed scaling from one replay to the next.

x bf16 [4096, 1024] N(0,1) and dY bf16 [4096, 4096] N(0,1e-3) are fresh for
every replay.  They are copied into the static inputs eagerly between
replays, followed by a synchronization.  W [4096, 1024] N(0,0.02) and bias
[4096] N(0,0.1) stay fixed; histories hold 16 entries.  The forward GEMM
(4096x4096x1024) runs the 256x256 tiles, dX and dW (4096x1024x4096) the
64-row tiles.

The same step under dynamic (current) scaling -- no rings; every quantize
measures its tensor in an amax pass over a shared workspace -- is captured
and checked the same way.

Checks, for every replay:
* the outputs (Y, dX, dW, db), all codes, the scale snapshots and the three
  rings' words equal, bit for bit, those of a second layer stepped eagerly on
  the same inputs;
* x's codes (and, delayed, its ring words) equal the oracle's.
"""
import numpy as np
import pytest
import torch

import oracle as O
import synth
from tests.gpu_util import DEV, np_codes, ring_state_words

pytestmark = pytest.mark.gpu

fp8mi = pytest.importorskip("fp8_tensor_scaled_quantize_amd")
from fp8_tensor_scaled_quantize_amd.linear import Fp8Linear  # noqa: E402

STEPS = 4
M, K, N = 4096, 1024, 4096


def step(layer, x, dy):
    y = layer.forward(x)
    dx, dw, db = layer.backward(dy)
    xq, wq = layer.last_codes
    gq, gq_t = layer.last_grad_codes
    return {"y": y, "dx": dx, "dw": dw, "db": db, "xq": xq, "wq": wq, "gq": gq, "gq_t": gq_t,
            "scale_inv": layer.scale_inv, "ring_x": layer.ring_x, "ring_w": layer.ring_w, "ring_g": layer.ring_g}


def bits(t):
    t = t.contiguous()
    return t.view(torch.int16) if t.dtype in (torch.bfloat16, torch.float16) else t.view(torch.uint8)


@pytest.mark.parametrize("dynamic", [False, True], ids=["delayed", "dynamic"])
def test_graph_replays_match_eager_steps(dynamic):
    x_host = [synth.gaussian((M, K), 1.0, "bf16", 11, synth.T_X, t) for t in range(STEPS)]
    xs = [synth.to_torch(x, "bf16").to(DEV) for x in x_host]
    dys = [synth.device_gaussian((M, N), 1e-3, torch.bfloat16, 1100 + t) for t in range(STEPS)]
    w = synth.to_torch(synth.gaussian((N, K), 0.02, "bf16", 11, synth.T_W, 0), "bf16").to(DEV)
    b = synth.to_torch(synth.gaussian((N,), 0.1, "bf16", 11, synth.T_BIAS, 0), "bf16").to(DEV)

    # load every kernel's code object outside the capture
    warm = Fp8Linear(w, b, hist_len=16, dynamic=dynamic)
    step(warm, xs[0], dys[0])
    torch.cuda.synchronize()

    graph_layer = Fp8Linear(w, b, hist_len=16, dynamic=dynamic)
    eager_layer = Fp8Linear(w, b, hist_len=16, dynamic=dynamic)
    x_static = torch.empty_like(xs[0])
    dy_static = torch.empty_like(dys[0])
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        captured = step(graph_layer, x_static, dy_static)
    torch.cuda.synchronize()
    # capture records the kernels without running them: the rings are untouched
    if not dynamic:
        assert not ring_state_words(graph_layer.ring_x)[:16].any()

    rx = O.Ring.new(16, 1.0)
    for t in range(STEPS):
        x_static.copy_(xs[t])
        dy_static.copy_(dys[t])
        torch.cuda.synchronize()
        g.replay()
        eager = step(eager_layer, xs[t], dys[t])
        torch.cuda.synchronize()
        for name, ref in eager.items():
            got = captured[name]
            assert got is None or got.shape == ref.shape, (t, name)
            if name.startswith("ring_"):
                assert (got is None) == dynamic and (ref is None) == dynamic, (t, name)
                if not dynamic:
                    assert np.array_equal(ring_state_words(got), ring_state_words(ref)), (t, name)
            else:
                assert torch.equal(bits(got), bits(ref)), (t, name)
        if dynamic:
            ref_x = O.quantize_dynamic(x_host[t], "bf16", O.E4M3)
        else:
            ref_x = O.quantize(x_host[t], "bf16", O.E4M3, ring=rx)
            rx = ref_x["ring"]
            assert np.array_equal(ring_state_words(captured["ring_x"]), rx.words()), t
        assert np.array_equal(np_codes(captured["xq"]), ref_x["codes"]), t
