"""Maximum sizes: operands past the 32-bit limits of the fast paths.

* A GEMM whose A operand spans more than 2^31 bytes runs on the plain-load
  kernel (the LDS-DMA kernels address operands with 32-bit buffer offsets);
  small-integer codes make every partial sum exact, so sampled output rows
  must equal the oracle bit for bit.  A K-major operand that large is refused.
* A quantize of more than 2^31 elements (bf16, 8.6 GB with both layouts) with
  the amax element planted past element 2^31: amax, the ring fold and the
  codes of sampled rows / columns against the oracle (64-bit indexing)."""
import numpy as np
import pytest
import torch

import oracle as O
import synth
from tests.gpu_util import DEV, np_bf16_bits, ring_from_oracle, ring_state_words

pytestmark = pytest.mark.gpu
fp8mi = pytest.importorskip("fp8_tensor_scaled_quantize_amd")


def int_codes_on_device(shape, seed):
    """E4M3 codes of integers -4..4 drawn on the device."""
    table = torch.from_numpy(O.encode(np.arange(-4, 5, dtype=np.float32), O.E4M3)).to(DEV)
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    return table[torch.randint(0, 9, shape, generator=g, device=DEV)]


@pytest.mark.timeout(600)
def test_gemm_operand_beyond_2_31_bytes():
    M, N, K = 131088, 96, 16384                # A: 2,147,745,792 bytes
    assert M * K > 2 ** 31
    A = int_codes_on_device((M, K), 60)
    B = int_codes_on_device((N, K), 61)
    bias = torch.arange(N, dtype=torch.float32, device=DEV) - 48.0
    y = fp8mi.fp8_mm(A, B, 0, 0, None, None, bias)
    torch.cuda.synchronize()
    rows = np.concatenate([np.sort(synth.rng(62).choice(M - 64, 40, replace=False)), np.arange(M - 24, M)])
    ridx = torch.from_numpy(rows).to(DEV)
    ref, _ = O.mm(A[ridx].cpu().numpy(), O.E4M3, B.cpu().numpy(), O.E4M3, 1.0, 1.0,
                  np.arange(N, dtype=np.float64) - 48.0)
    assert np.array_equal(np_bf16_bits(y[ridx]), ref[0])
    with pytest.raises(fp8mi.Fp8Error):         # K-major views of that size: no 32-bit-offset fallback
        fp8mi.fp8_mm(A.t().contiguous().t(), B, 0, 0)


@pytest.mark.timeout(900)
def test_quantize_beyond_2_31_elements():
    R, C = 65537, 32768                        # 2,147,516,416 elements
    assert R * C > 2 ** 31
    x = synth.device_gaussian((R, C), 0.5, torch.bfloat16, 63, DEV)
    flat = 2 ** 31 + 12345                     # past element 2^31: row 65536, column 12345
    r_p, c_p = divmod(flat, C)
    x[r_p, c_p] = 7.5
    ring0 = O.Ring.new(4, 64.0)
    ring = ring_from_oracle(ring0)
    codes, codes_t = fp8mi.fp8_quantize_dual(x, fp8mi.E5M2, ring=ring)
    torch.cuda.synchronize()
    ref_ring = O.fold(ring0, np.float32(7.5), O.E5M2)
    assert np.array_equal(ring_state_words(ring), ref_ring.words())   # amax found past 2^31
    s = ring0.scale
    rows = np.concatenate([[0, 1, r_p - 1, r_p], np.sort(synth.rng(64).choice(R, 12, replace=False))])
    ridx = torch.from_numpy(rows).to(DEV)
    xr = x[ridx].cpu().view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(codes[ridx].cpu().numpy(), O.quantize(xr, "bf16", O.E5M2, scale=s)["codes"])
    cols = np.array([0, c_p, C - 1, 777])
    for c in cols:
        xc = x[:, int(c)].contiguous().cpu().view(torch.int16).numpy().view(np.uint16)
        want = O.quantize(xc[None, :], "bf16", O.E5M2, scale=s)["codes"][0]
        assert np.array_equal(codes_t[int(c)].cpu().numpy(), want), c
    del codes, codes_t
    # the row layout alone takes the flat streaming kernel
    ring2 = ring_from_oracle(ring0)
    amax_t = torch.empty(1, dtype=torch.float32, device=DEV)
    row = fp8mi.fp8_quantize(x, fp8mi.E5M2, False, ring=ring2, amax_out=amax_t)
    torch.cuda.synchronize()
    assert float(amax_t.item()) == 7.5
    assert np.array_equal(ring_state_words(ring2), ref_ring.words())
    assert np.array_equal(row[ridx].cpu().numpy(), O.quantize(xr, "bf16", O.E5M2, scale=s)["codes"])
