"""fp8_quantize_dual_bias_grad_noalloc (the entry point for callers that
cannot allocate) against fp8_quantize_dual_bias_grad with a caller workspace:
codes, transposed codes, bias gradient, scale_inv, amax and ring words equal
bit for bit, on two calls in a row through the library's one scratch array,
the second with a smaller (and misaligned, padded) gradient, then a third at
the first shape again so stale sums of the smaller call cannot leak."""
import numpy as np
import pytest
import torch

import oracle as O
import synth
from tests.gpu_util import DEV, np_bf16_bits, np_codes, ring_from_oracle, scalar, to_device

pytestmark = pytest.mark.gpu
fp8mi = pytest.importorskip("fp8_tensor_scaled_quantize_amd")


def run_pair(dy_dev, rows, cols, fmt, ring0, tag):
    """Both entry points on the same gradient, each with its own ring copy."""
    outs = []
    for noalloc in (False, True):
        ring = ring_from_oracle(ring0)
        o = torch.full((rows, cols), 0xA5, dtype=torch.uint8, device=DEV)
        ot = torch.full((cols, rows), 0xA5, dtype=torch.uint8, device=DEV)
        db = torch.full((cols,), 7.0, dtype=torch.bfloat16, device=DEV)
        sinv, amax = scalar(-1), scalar(-1)
        if noalloc:
            fp8mi.fp8_quantize_dual_bias_grad_noalloc(dy_dev, fmt, o, ot, db, ring=ring, scale_inv_out=sinv,
                                                      amax_out=amax)
        else:
            fp8mi.fp8_quantize_dual_bias_grad(dy_dev, fmt, out_row=o, out_t=ot, ring=ring, scale_inv_out=sinv,
                                              amax_out=amax, bias_grad_out=db)
        torch.cuda.synchronize()
        outs.append((np_codes(o), np_codes(ot), np_bf16_bits(db), sinv.cpu().numpy().view(np.uint32),
                     amax.cpu().numpy().view(np.uint32), ring.cpu().numpy().view(np.uint32)))
    for name, a, b in zip(("codes", "codes_t", "bias_grad", "scale_inv", "amax", "ring"), outs[0], outs[1]):
        assert np.array_equal(a, b), f"{tag}: {name} differs from the workspace entry point"
    return outs[1]


def test_noalloc_matches_workspace_entry_point():
    ring0 = O.Ring.new(16, 1.0)
    ring0.hist[:5] = [3e-3, 1e-3, 2e-3, 0.0, 5e-3]
    ring0.scale, ring0.idx = np.float32(57344.0 / 5e-3), 5
    cases = [((8192, 6912), 0, fp8mi.E5M2), ((1000, 1535), 1, fp8mi.E4M3), ((8192, 6912), 0, fp8mi.E5M2)]
    for i, ((rows, cols), mis, fmt) in enumerate(cases):
        print(f"noalloc call {i}: {rows}x{cols} misalign={mis} fmt={fmt}", flush=True)
        dy = synth.gaussian((rows, cols), 1e-3, "bf16", 98, i)
        dy_dev = to_device(dy, "bf16", misalign=mis, ld=cols + 8 * mis)
        codes, codes_t, db, _, _, _ = run_pair(dy_dev, rows, cols, fmt, ring0, f"call {i}")
        # and the bias gradient against the oracle's fp64 sum (the fused path's bar)
        ref, mag = O.grad_bias(dy)
        assert O.within_tolerance(db, ref, mag).all(), f"call {i}: bias gradient outside the bound"
        assert (db == ref).mean() > 0.999, f"call {i}"
