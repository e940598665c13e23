"""fp8_bias_grad and fp8_ring_seed against the oracle."""
import numpy as np
import pytest
import torch

import oracle as O
import synth
from tests.gpu_util import DEV, np_bf16_bits, ring_state_words, scalar, to_device

pytestmark = pytest.mark.gpu
fp8mi = pytest.importorskip("fp8_tensor_scaled_quantize_amd")


@pytest.mark.parametrize("shape,misalign", [((8192, 6912), 0), ((7, 5), 0), ((1000, 130), 1), ((1, 64), 0),
                                            ((513, 1537), 1), ((3, 2, 200), 0)])
def test_bias_grad_bf16(shape, misalign):
    dy = synth.gaussian(shape, 1e-3, "bf16", 80, *shape[:2])
    rows, cols = int(np.prod(shape[:-1])), shape[-1]
    d2 = dy.reshape(rows, cols)
    t = to_device(d2, "bf16", misalign=misalign)
    db = fp8mi.fp8_bias_grad(t)
    ref, mag = O.grad_bias(dy)
    got = np_bf16_bits(db)
    assert O.within_tolerance(got, ref, mag).all()
    # sums of bf16 values over this range are exact in fp64: one rounding each side
    assert np.array_equal(got, ref)


def test_bias_grad_f16_and_strided():
    dy = synth.gaussian((300, 96), 2.0, "f16", 81, 1)
    buf = torch.zeros((300, 128), dtype=torch.float16, device=DEV)
    buf[:, :96] = torch.from_numpy(dy).to(DEV)
    db = fp8mi.fp8_bias_grad(buf[:, :96])
    v = dy.astype(np.float64).sum(axis=0)
    assert np.array_equal(np_bf16_bits(db), O.bf16_bits_from_f64(v))


def test_bias_grad_caller_workspace_reused_and_checked():
    # one caller-owned workspace (filled with garbage) serves two shapes in a row;
    # 300 rows = 3 row chunks (the last ragged), 1100 columns = 3 column blocks (ragged)
    ws = torch.full((fp8mi.fp8_bias_grad_workspace_bytes(300, 1100) // 8,), float("nan"), dtype=torch.float64,
                    device=DEV)
    for shape, seed in (((300, 1100), 82), ((129, 700), 83)):
        dy = synth.gaussian(shape, 1e-3, "bf16", seed, 0)
        db = fp8mi.fp8_bias_grad(to_device(dy, "bf16"), workspace=ws)
        ref, mag = O.grad_bias(dy)
        assert np.array_equal(np_bf16_bits(db), ref), shape
    small = torch.empty(fp8mi.fp8_bias_grad_workspace_bytes(300, 1100) - 8, dtype=torch.uint8, device=DEV)
    with pytest.raises(fp8mi.Fp8Error):
        fp8mi.fp8_bias_grad(to_device(synth.gaussian((300, 1100), 1e-3, "bf16", 84, 0), "bf16"), workspace=small)


def test_bias_grad_zero_rows():
    db = fp8mi.fp8_bias_grad(torch.empty((0, 33), dtype=torch.bfloat16, device=DEV))
    assert torch.all(db == 0)


@pytest.mark.parametrize("fmt,fid", [(O.E4M3, 0), (O.E5M2, 1)])
def test_ring_seed(fmt, fid):
    for amax, H in ((3.5, 4), (0.0, 2), (float("inf"), 1), (1e-3, 16)):
        ring = fp8mi.new_ring(H, 7.0, DEV)
        ring[:H] = 99  # garbage history, scratch words set too
        ring[-5:] = 3
        fp8mi.fp8_ring_seed(ring, scalar(amax), fid)
        ref = O.Ring.new(H, O.next_scale(np.array([amax], np.float32), fmt))
        assert np.array_equal(ring_state_words(ring), ref.words())
