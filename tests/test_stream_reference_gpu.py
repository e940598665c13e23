"""The streaming reference kernel (the practical HBM ceiling the benchmark
reports beside the quantize) moves the bytes it claims to: dst holds the top
byte of every 16-bit pair of src, or src itself, and nothing past dst's end
is written."""
import numpy as np
import pytest
import torch

from tests.gpu_util import DEV

pytestmark = pytest.mark.gpu
fp8mi = pytest.importorskip("fp8_tensor_scaled_quantize_amd")


@pytest.mark.parametrize("nbytes", [16, 4096 * 3 + 16 * 7, 8192 * 1536 * 2])
def test_stream_reference_bytes(nbytes):
    src = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, device=DEV)
    for half in (True, False):
        n_out = nbytes // 2 if half else nbytes
        buf = torch.full((n_out + 64,), 0x5A, dtype=torch.uint8, device=DEV)
        fp8mi.stream_reference(src, buf[:n_out])
        torch.cuda.synchronize()
        s, d = src.cpu().numpy(), buf.cpu().numpy()
        want = s[1::2] if half else s
        assert np.array_equal(d[:n_out], want)
        assert (d[n_out:] == 0x5A).all()
