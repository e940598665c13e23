"""torch autograd over the fp8 linear (fp8_linear).

fp8_linear(x, layer) puts one Fp8Linear forward on the autograd tape and
loss.backward() runs the layer's backward.  It is checked against a twin
layer stepped explicitly (forward, backward) from identical rings on the same
inputs, bit for bit -- y, x.grad, weight.grad and bias.grad over three steps,
under delayed and under dynamic scaling.  Gradients go only to the inputs
that require them, and a backward whose forward was followed by another
forward of the same layer raises instead of using the newer step's codes.

x bf16 [2, 512, 768] N(0,1), W [1024, 768] N(0,0.02), bias [1024] N(0,0.1),
dY N(0,1e-3), fresh x and dY every step.
"""
import pytest
import torch

import synth
from tests.gpu_util import DEV

pytestmark = pytest.mark.gpu

fp8mi = pytest.importorskip("fp8_tensor_scaled_quantize_amd")
from fp8_tensor_scaled_quantize_amd.linear import Fp8Linear, fp8_linear  # noqa: E402


def bits(t):
    return t.contiguous().view(torch.int16)


def inputs(step):
    x = synth.device_gaussian((2, 512, 768), 1.0, torch.bfloat16, 7100 + step)
    dy = synth.device_gaussian((2, 512, 1024), 1e-3, torch.bfloat16, 7200 + step)
    return x, dy


@pytest.mark.parametrize("dynamic", [False, True], ids=["delayed", "dynamic"])
def test_autograd_matches_explicit_steps(dynamic):
    w = synth.device_gaussian((1024, 768), 0.02, torch.bfloat16, 7000)
    b = synth.device_gaussian((1024,), 0.1, torch.bfloat16, 7001)
    wa, ba = w.clone().requires_grad_(), b.clone().requires_grad_()
    auto = Fp8Linear(wa, ba, hist_len=8, dynamic=dynamic)
    expl = Fp8Linear(w.clone(), b.clone(), hist_len=8, dynamic=dynamic)
    for step in range(3):
        x, dy = inputs(step)
        xa = x.clone().requires_grad_()
        wa.grad = ba.grad = None
        y = fp8_linear(xa, auto)
        y.backward(dy)
        y_ref = expl.forward(x)
        dx_ref, dw_ref, db_ref = expl.backward(dy)
        torch.cuda.synchronize()
        assert torch.equal(bits(y), bits(y_ref)), step
        assert torch.equal(bits(xa.grad), bits(dx_ref)), step
        assert torch.equal(bits(wa.grad), bits(dw_ref)), step
        assert torch.equal(bits(ba.grad), bits(db_ref)), step


def test_gradients_only_where_required():
    w = synth.device_gaussian((1024, 768), 0.02, torch.bfloat16, 7000).requires_grad_()
    layer = Fp8Linear(w, None, hist_len=8)
    x, dy = inputs(0)
    y = fp8_linear(x, layer)                      # x does not require a gradient, there is no bias
    y.backward(dy)
    torch.cuda.synchronize()
    assert x.grad is None and w.grad is not None and w.grad.shape == w.shape


def test_stale_backward_raises():
    w = synth.device_gaussian((1024, 768), 0.02, torch.bfloat16, 7000).requires_grad_()
    layer = Fp8Linear(w, None, hist_len=8)
    x0, dy = inputs(0)
    x1, _ = inputs(1)
    y0 = fp8_linear(x0, layer)
    fp8_linear(x1, layer)                         # overwrites the codes saved for y0
    with pytest.raises(RuntimeError, match="another forward"):
        y0.backward(dy)
