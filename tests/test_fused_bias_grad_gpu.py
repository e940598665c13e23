"""fp8_quantize_dual_bias_grad: the dual quantize of an output gradient with
its bias gradient from the same read.  Codes, scale_inv and ring words must be
bit-identical to fp8_quantize_dual on an identical ring; the bias gradient is
checked against the oracle (fp64 column sums, one bf16 rounding)."""
import numpy as np
import pytest
import torch

import oracle as O
import synth
from tests.gpu_util import DEV, np_bf16_bits, np_codes, ring_state_words, to_device

pytestmark = pytest.mark.gpu
fp8mi = pytest.importorskip("fp8_tensor_scaled_quantize_amd")

# (rows, cols, dtype, fmt id, misalign): one-shot grids, ragged 128-row tiles and
# odd widths, a misaligned base, and the persistent grid of the 8192 x 6912 gradient
CASES = [
    (64, 256, "bf16", 1, 0),
    (300, 1100, "bf16", 1, 0),
    (1000, 1535, "bf16", 0, 1),
    (129, 65, "f16", 1, 0),
    (1, 7, "bf16", 1, 0),
    (8192, 1536, "bf16", 1, 0),
    (8192, 6912, "bf16", 1, 0),
]


@pytest.mark.parametrize("rows,cols,dt,fid,misalign", CASES)
def test_fused_matches_dual_and_oracle(rows, cols, dt, fid, misalign):
    fmt = (O.E4M3, O.E5M2)[fid]
    dy = synth.gaussian((rows, cols), 1e-3, dt, 90, rows, cols)
    x = to_device(dy, dt, misalign=misalign)
    r1 = fp8mi.new_ring(16, 50.0, DEV)
    r1[:16] = torch.arange(16, dtype=torch.float32, device=DEV).view(torch.int32)  # a non-trivial window
    r2 = r1.clone()
    s1 = torch.empty(1, dtype=torch.float32, device=DEV)
    s2 = torch.empty(1, dtype=torch.float32, device=DEV)
    q_row, q_t = fp8mi.fp8_quantize_dual(x, fid, ring=r1, scale_inv_out=s1)
    f_row, f_t, db = fp8mi.fp8_quantize_dual_bias_grad(x, fid, ring=r2, scale_inv_out=s2)
    torch.cuda.synchronize()
    assert torch.equal(q_row, f_row) and torch.equal(q_t, f_t)
    assert torch.equal(s1, s2)
    assert np.array_equal(ring_state_words(r1), ring_state_words(r2))
    ref, mag = O.grad_bias(dy, dt)
    got = np_bf16_bits(db)
    assert O.within_tolerance(got, ref, mag).all()
    assert (got == ref).mean() > 0.999
    # the codes themselves against the oracle on a sample of rows
    rs = np.unique(np.linspace(0, rows - 1, 16).astype(int))
    ref_codes = O.encode(O.scaled_values(O.widen_to_f32(dy[rs], dt), np.float32(50.0)), fmt)
    assert np.array_equal(np_codes(f_row)[rs], ref_codes)


def test_fused_deterministic_and_workspace_reuse():
    dy = to_device(synth.gaussian((2048, 3000), 1e-3, "bf16", 91, 0), "bf16")
    ws = torch.full((fp8mi.fp8_bias_grad_workspace_bytes(2048, 3000) // 8,), float("nan"), dtype=torch.float64,
                    device=DEV)
    outs = []
    for _ in range(5):
        _, _, db = fp8mi.fp8_quantize_dual_bias_grad(dy, 1, scale=torch.ones(1, device=DEV), workspace=ws)
        outs.append(db.clone())
    for o in outs[1:]:
        assert torch.equal(o, outs[0])


def test_fused_rejects_before_launch():
    x = torch.zeros((4, 4), dtype=torch.float32, device=DEV)
    with pytest.raises(fp8mi.Fp8Error):  # fp32 gradient
        fp8mi.fp8_quantize_dual_bias_grad(x, 1, scale=torch.ones(1, device=DEV))
    xb = torch.zeros((300, 16), dtype=torch.bfloat16, device=DEV)
    small = torch.empty(fp8mi.fp8_bias_grad_workspace_bytes(300, 16) - 8, dtype=torch.uint8, device=DEV)
    with pytest.raises(fp8mi.Fp8Error):
        fp8mi.fp8_quantize_dual_bias_grad(xb, 1, scale=torch.ones(1, device=DEV), workspace=small)


def test_fused_empty_rows_gives_zero_bias_grad():
    x = torch.empty((0, 33), dtype=torch.bfloat16, device=DEV)
    _, _, db = fp8mi.fp8_quantize_dual_bias_grad(x, 1, scale=torch.ones(1, device=DEV))
    assert torch.all(db == 0)
