"""fp8 linear layer driven through the C ABI (host harness), delayed or
current (dynamic) scaling.

The layer owns three amax-history rings -- x, W and the output gradient g --
the per-operand rings of the pages' FP8TensorMeta (log:tests/extension, the
commit turning FP8TensorMeta into three per-operand rings).  Every operation
is one library call on torch's current stream; the rings never leave the
device, so a step has no host synchronisation:

forward(x):   x -> E4M3 codes in both layouts with ring x  (fp8_quantize_dual)
              W -> E4M3 codes in both layouts with ring W  (fp8_quantize_dual)
              Y = Xq Wq^T * sx_inv * sw_inv + b             (fp8_mm, bf16 out)
backward(dY): dY -> E5M2 codes in both layouts with ring g (fp8_quantize_dual)
              dX = Gq (Wq^T)^T * sg_inv * sw_inv            (fp8_mm, NT on W^T codes)
              dW = Gq^T (Xq^T)^T * sg_inv * sx_inv          (fp8_mm, NT on the
                                                            transposed codes)
              db = sum of dY over leading dims              (fused into dY's dual
                                                            quantize: fp8_quantize_dual_bias_grad)

The scale_inv values a quantize writes are the snapshot of the scale it used,
taken before its fold publishes the next one, and backward reuses the
forward's x / W snapshots (log:tests/extension, the commit snapshotting
sx/sw/sg before the ring finalize and carrying the forward's scale to the
backward).  E5M2 for gradients, E4M3 for x and W (log:tests/extension, the
commit on the fp8 backward with E5M2 gradients; log:csrc/kernels/fp8_mm.cu,
commit 5244f1a8fc).

With dynamic=True the layer follows the recipe's dynamic flag instead: no
rings are allocated and every quantize measures its scale from the tensor it
quantizes (fp8_quantize_dynamic; log:tests/extension, the commits merging the
two recipes behind one flag and skipping the rings on the dynamic path); the
bias gradient then comes from fp8_bias_grad.

fp8 operands (log:tests/extension, the commit letting the linear forward take
a pre-quantized fp8 weight and an fp8 bias with a bias_scale, and the commit
adding the FP8-in/FP8-out GEMM):
* Fp8Linear.from_fp8_weight(codes, scale_inv, ...) takes E4M3 weight codes and
  their dequantisation multiplier; the weight quantize is skipped and the
  weight's amax reads 0 (no high-precision weight values are seen).  Backward
  needs the transposed codes too (codes_t).
* bias may be fp8 codes (bias_fmt, bias_scale = dequantisation multiplier).
* forward(x, out_fp8=True) returns E4M3 output codes and their scale_inv,
  quantized in the GEMM epilogue with the layer's output ring ring_y;
  forward accepts such codes as x (x_scale_inv given) -- inference chaining
  with no quantize between layers.

fp8_linear(x, layer) records one forward on torch's autograd tape
(log:tests/extension, the commit giving the fp8 linear's forward/backward
pair to an autograd function whose backward reads only its context and masks
the gradients by needs_input_grad): loss.backward() then runs the layer's
backward and leaves dX in x.grad, dW in weight.grad and db in bias.grad.
"""
from __future__ import annotations

import torch

from . import (DYNAMIC_WORKSPACE_BYTES, E4M3, E5M2, LAYOUT_DUAL, LAYOUT_ROW, fp8_bias_grad, fp8_mm, fp8_mm_ex,
               fp8_quantize, fp8_quantize_dual, fp8_quantize_dual_bias_grad, fp8_quantize_dynamic, fp8_ring_seed,
               new_ring)


class Fp8Linear:
    def __init__(self, weight: torch.Tensor, bias: torch.Tensor | None = None, hist_len: int = 16,
                 dynamic: bool = False, bias_fmt=None, bias_scale: torch.Tensor | None = None):
        if weight.dim() != 2:
            raise ValueError("weight must be [out_features, in_features]")
        if (bias_fmt is None) != (bias_scale is None):
            raise ValueError("an fp8 bias needs both bias_fmt and bias_scale")
        self.weight = weight
        self.bias = bias
        self.bias_fmt, self.bias_scale = bias_fmt, bias_scale
        self.hist_len = hist_len
        self.dynamic = dynamic
        dev = weight.device
        self._w_codes = None  # pre-quantized weight: (codes, codes_t or None)
        if dynamic:  # no rings; one workspace serves every call (they run in stream order)
            self.ring_x = self.ring_w = self.ring_g = None
            self._ws = torch.empty(DYNAMIC_WORKSPACE_BYTES, dtype=torch.uint8, device=dev)
        else:
            self.ring_x = new_ring(hist_len, 1.0, dev)
            self.ring_w = new_ring(hist_len, 1.0, dev)
            self.ring_g = new_ring(hist_len, 1.0, dev)
        self.ring_y = new_ring(hist_len, 1.0, dev)  # output ring of the FP8-out forward
        # scale_inv snapshots [x, w, g], the output's [y], amaxes [x, w] and an amax word for seeding
        self.scale_inv = torch.empty(3, dtype=torch.float32, device=dev)
        self.y_scale_inv = torch.empty(1, dtype=torch.float32, device=dev)
        self.amax = torch.zeros(2, dtype=torch.float32, device=dev)
        self._amax = torch.empty(1, dtype=torch.float32, device=dev)
        self._one = torch.ones(1, dtype=torch.float32, device=dev)
        self._saved = None
        self._forwards = 0  # forwards saved for backward so far (fp8_linear's pairing check)

    @classmethod
    def from_fp8_weight(cls, codes: torch.Tensor, scale_inv: torch.Tensor, bias: torch.Tensor | None = None,
                        codes_t: torch.Tensor | None = None, hist_len: int = 16, dynamic: bool = False,
                        bias_fmt=None, bias_scale: torch.Tensor | None = None) -> "Fp8Linear":
        """A layer over pre-quantized E4M3 weight codes [out, in] (and
        optionally their transpose [in, out] for backward) whose
        dequantisation multiplier is scale_inv."""
        layer = cls(codes, bias, hist_len, dynamic, bias_fmt, bias_scale)
        layer._w_codes = (codes, codes_t)
        layer.scale_inv[1:2].copy_(scale_inv.reshape(1))
        return layer

    # ------------------------------------------------------------------
    def _seed(self, ring: torch.Tensor, t: torch.Tensor, fmt) -> None:
        """Seed a ring from a first tensor: its raw amax (a quantize at scale
        1 whose codes are discarded) -> fp8_ring_seed."""
        t2 = t.reshape(-1, t.shape[-1])
        fp8_quantize(t2, fmt, False, scale=self._one, amax_out=self._amax)
        fp8_ring_seed(ring, self._amax, fmt)

    def seed(self, x: torch.Tensor, dy: torch.Tensor | None = None) -> None:
        """Seed the x and W rings (and g, given a first gradient); nothing to
        seed under dynamic scaling, nor for a pre-quantized weight."""
        if self.dynamic:
            return
        self._seed(self.ring_x, x, E4M3)
        if self._w_codes is None:
            self._seed(self.ring_w, self.weight, E4M3)
        if dy is not None:
            self._seed(self.ring_g, dy, E5M2)

    # ------------------------------------------------------------------
    def _quantize_x(self, x2, save):
        sx, ax = self.scale_inv[0:1], self.amax[0:1]
        if self.dynamic:
            return fp8_quantize_dynamic(x2, E4M3, LAYOUT_DUAL if save else LAYOUT_ROW, scale_inv_out=sx,
                                        amax_out=ax, workspace=self._ws)
        if save:
            return fp8_quantize_dual(x2, E4M3, ring=self.ring_x, scale_inv_out=sx, amax_out=ax)
        return fp8_quantize(x2, E4M3, False, ring=self.ring_x, scale_inv_out=sx, amax_out=ax), None

    def _quantize_w(self, save):
        sw, aw = self.scale_inv[1:2], self.amax[1:2]
        if self._w_codes is not None:  # pre-quantized: nothing to quantize, amax_w = 0
            aw.zero_()
            wq, wq_t = self._w_codes
            if save and wq_t is None:
                raise RuntimeError("backward over a pre-quantized weight needs its transposed codes (codes_t)")
            return wq, wq_t
        if self.dynamic:
            return fp8_quantize_dynamic(self.weight, E4M3, LAYOUT_DUAL if save else LAYOUT_ROW, scale_inv_out=sw,
                                        amax_out=aw, workspace=self._ws)
        if save:
            return fp8_quantize_dual(self.weight, E4M3, ring=self.ring_w, scale_inv_out=sw, amax_out=aw)
        return fp8_quantize(self.weight, E4M3, False, ring=self.ring_w, scale_inv_out=sw, amax_out=aw), None

    def forward(self, x: torch.Tensor, save_for_backward: bool = True, out_fp8: bool = False,
                x_scale_inv: torch.Tensor | None = None):
        """Y = x W^T + b.  x: bf16/fp16/fp32 [..., in], or E4M3 codes (uint8)
        with x_scale_inv (forward only).  Returns bf16 Y, or with out_fp8 the
        pair (E4M3 codes of Y, their scale_inv) from the quantizing epilogue."""
        K = self.weight.shape[1]
        x2 = x.reshape(-1, K)
        sx, sw = self.scale_inv[0:1], self.scale_inv[1:2]
        if x.dtype == torch.uint8:
            if x_scale_inv is None or save_for_backward:
                raise ValueError("fp8 x needs x_scale_inv and save_for_backward=False")
            sx = x_scale_inv.reshape(1)
            xq, xq_t = x2, None
        else:
            xq, xq_t = self._quantize_x(x2, save_for_backward)
        wq, wq_t = self._quantize_w(save_for_backward)
        self._saved = (xq_t, wq_t, x.shape) if save_for_backward else None
        self._forwards += 1 if save_for_backward else 0
        self.last_codes = (xq, wq)
        out_shape = (*x.shape[:-1], self.weight.shape[0])
        if out_fp8 or self.bias_fmt is not None:
            y = fp8_mm_ex(xq, wq, E4M3, E4M3, sx, sw, self.bias, self.bias_fmt, self.bias_scale,
                          out_fmt=E4M3 if out_fp8 else None, out_ring=self.ring_y if out_fp8 else None,
                          out_scale_inv=self.y_scale_inv if out_fp8 else None)
            return (y.reshape(out_shape), self.y_scale_inv) if out_fp8 else y.reshape(out_shape)
        return fp8_mm(xq, wq, E4M3, E4M3, sx, sw, self.bias).reshape(out_shape)

    def backward(self, dy: torch.Tensor):
        if self._saved is None:
            raise RuntimeError("backward needs a forward with save_for_backward=True")
        xq_t, wq_t, x_shape = self._saved
        N = self.weight.shape[0]
        dy2 = dy.reshape(-1, N)
        sx, sw, sg = self.scale_inv[0:1], self.scale_inv[1:2], self.scale_inv[2:3]
        if self.dynamic:
            gq, gq_t = fp8_quantize_dynamic(dy2, E5M2, LAYOUT_DUAL, scale_inv_out=sg, workspace=self._ws)
            db = fp8_bias_grad(dy2) if self.bias is not None else None
        elif self.bias is not None:  # the bias gradient comes from the quantize's own read of dY
            gq, gq_t, db = fp8_quantize_dual_bias_grad(dy2, E5M2, ring=self.ring_g, scale_inv_out=sg)
        else:
            gq, gq_t = fp8_quantize_dual(dy2, E5M2, ring=self.ring_g, scale_inv_out=sg)
            db = None
        dx = fp8_mm(gq, wq_t, E5M2, E4M3, sg, sw)
        dw = fp8_mm(gq_t, xq_t, E5M2, E4M3, sg, sx)
        self.last_grad_codes = (gq, gq_t)
        return dx.reshape(x_shape), dw, db


class _Fp8LinearFn(torch.autograd.Function):
    """One Fp8Linear step on torch's autograd tape.  The layer keeps a single
    forward's saved codes and scale snapshots, so a backward must belong to
    the layer's latest saved forward."""

    @staticmethod
    def forward(ctx, x, weight, bias, layer):
        y = layer.forward(x, save_for_backward=True)
        ctx.layer, ctx.step = layer, layer._forwards
        ctx.dtypes = (x.dtype, weight.dtype, None if bias is None else bias.dtype)
        return y

    @staticmethod
    def backward(ctx, dy):
        layer = ctx.layer
        if layer._forwards != ctx.step:
            raise RuntimeError("fp8_linear: the layer ran another forward since the one being differentiated")
        dx, dw, db = layer.backward(dy.contiguous())
        tx, tw, tb = ctx.dtypes
        need = ctx.needs_input_grad
        return (dx.to(tx) if need[0] else None, dw.to(tw) if need[1] else None,
                db.to(tb) if need[2] and db is not None else None, None)


def fp8_linear(x: torch.Tensor, layer: Fp8Linear) -> torch.Tensor:
    """y = layer.forward(x) recorded for autograd: the backward pass runs
    layer.backward (dY quantized with the layer's gradient ring, the dX and
    dW GEMMs with the forward's scales, the fused bias gradient) and returns
    dX, dW and db to x, layer.weight and layer.bias."""
    return _Fp8LinearFn.apply(x, layer.weight, layer.bias, layer)
