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
"""
from __future__ import annotations

import torch

from . import (DYNAMIC_WORKSPACE_BYTES, E4M3, E5M2, LAYOUT_DUAL, LAYOUT_ROW, fp8_bias_grad, fp8_mm, fp8_quantize,
               fp8_quantize_dual, fp8_quantize_dual_bias_grad, fp8_quantize_dynamic, fp8_ring_seed, new_ring)


class Fp8Linear:
    def __init__(self, weight: torch.Tensor, bias: torch.Tensor | None = None, hist_len: int = 16,
                 dynamic: bool = False):
        if weight.dim() != 2:
            raise ValueError("weight must be [out_features, in_features]")
        self.weight = weight
        self.bias = bias
        self.hist_len = hist_len
        self.dynamic = dynamic
        dev = weight.device
        if dynamic:  # no rings; one workspace serves every call (they run in stream order)
            self.ring_x = self.ring_w = self.ring_g = None
            self._ws = torch.empty(DYNAMIC_WORKSPACE_BYTES, dtype=torch.uint8, device=dev)
        else:
            self.ring_x = new_ring(hist_len, 1.0, dev)
            self.ring_w = new_ring(hist_len, 1.0, dev)
            self.ring_g = new_ring(hist_len, 1.0, dev)
        # scale_inv snapshots [x, w, g] and an amax word for seeding
        self.scale_inv = torch.empty(3, dtype=torch.float32, device=dev)
        self._amax = torch.empty(1, dtype=torch.float32, device=dev)
        self._one = torch.ones(1, dtype=torch.float32, device=dev)
        self._saved = None

    # ------------------------------------------------------------------
    def _seed(self, ring: torch.Tensor, t: torch.Tensor, fmt) -> None:
        """Seed a ring from a first tensor: its raw amax (a quantize at scale
        1 whose codes are discarded) -> fp8_ring_seed."""
        t2 = t.reshape(-1, t.shape[-1])
        fp8_quantize(t2, fmt, False, scale=self._one, amax_out=self._amax)
        fp8_ring_seed(ring, self._amax, fmt)

    def seed(self, x: torch.Tensor, dy: torch.Tensor | None = None) -> None:
        """Seed the x and W rings (and g, given a first gradient); nothing to
        seed under dynamic scaling."""
        if self.dynamic:
            return
        self._seed(self.ring_x, x, E4M3)
        self._seed(self.ring_w, self.weight, E4M3)
        if dy is not None:
            self._seed(self.ring_g, dy, E5M2)

    # ------------------------------------------------------------------
    def forward(self, x: torch.Tensor, save_for_backward: bool = True) -> torch.Tensor:
        K = self.weight.shape[1]
        x2 = x.reshape(-1, K)
        sx, sw = self.scale_inv[0:1], self.scale_inv[1:2]
        if self.dynamic:
            layout = LAYOUT_DUAL if save_for_backward else LAYOUT_ROW
            xq, xq_t = fp8_quantize_dynamic(x2, E4M3, layout, scale_inv_out=sx, workspace=self._ws)
            wq, wq_t = fp8_quantize_dynamic(self.weight, E4M3, layout, scale_inv_out=sw, workspace=self._ws)
            self._saved = (xq_t, wq_t, x.shape) if save_for_backward else None
        elif save_for_backward:
            xq, xq_t = fp8_quantize_dual(x2, E4M3, ring=self.ring_x, scale_inv_out=sx)
            wq, wq_t = fp8_quantize_dual(self.weight, E4M3, ring=self.ring_w, scale_inv_out=sw)
            self._saved = (xq_t, wq_t, x.shape)
        else:
            xq = fp8_quantize(x2, E4M3, False, ring=self.ring_x, scale_inv_out=sx)
            wq = fp8_quantize(self.weight, E4M3, False, ring=self.ring_w, scale_inv_out=sw)
            self._saved = None
        y = fp8_mm(xq, wq, E4M3, E4M3, sx, sw, self.bias)
        self.last_codes = (xq, wq)
        return y.reshape(*x.shape[:-1], self.weight.shape[0])

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
