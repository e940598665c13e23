"""Layout tags in the GEMM: operands given K-major (transposed views of
[K, M] / [K, N] storage) are read without a transposed copy through
ds_read_b64_tr_b8 fragments.  The MFMA sees the same fragments as in NT
form, so every result must equal the NT result of the same codes bit for bit
(bf16 values, or fp8 codes, amax and ring words with the quantizing
epilogue); on exact small-integer data it must also equal the oracle bit for
bit."""
import numpy as np
import pytest
import torch

import oracle as O
import synth
from tests.gpu_util import DEV, check, np_bf16_bits, scalar
from tests.test_mm_gpu import make_codes, make_int_codes, sample_rows, to_dev_codes

pytestmark = pytest.mark.gpu
fp8mi = pytest.importorskip("fp8_tensor_scaled_quantize_amd")
FID = {O.E4M3: 0, O.E5M2: 1}


def km_view(codes: np.ndarray, pad: int = 0) -> torch.Tensor:
    """Device [.., rows, K] view of K-major storage [.., K, ld], ld = rows
    rounded up to 16, plus pad (a multiple of 16)."""
    t = np.ascontiguousarray(np.swapaxes(codes, -1, -2))
    extra = (-codes.shape[-2]) % 16 + pad
    if extra:
        t = np.concatenate([t, np.full(t.shape[:-1] + (extra,), 0x7F, np.uint8)], axis=-1)
    d = torch.from_numpy(np.ascontiguousarray(t)).to(DEV)
    rows = codes.shape[-2]
    return d[..., :rows].transpose(-1, -2)


SHAPES = [(64, 256, 256, 1), (130, 257, 272, 1), (1000, 1537, 2048, 1), (2048, 1536, 1536, 1),
          (256, 384, 640, 3), (17, 33, 48, 2), (64, 4096, 1024, 1)]   # the last: 64 x 32 tiles


@pytest.mark.parametrize("layout", ["A", "B", "AB"])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_exact_integer_data_every_layout(shape, layout):
    M, N, K, batch = shape
    a = make_int_codes((batch, M, K), O.E5M2, 50, M, K, 0)
    b = make_int_codes((batch, N, K), O.E4M3, 50, M, K, 1)
    bias = synth.rng(50, M, 2).integers(-8, 9, size=N).astype(np.float32)
    sa, sb = 0.5, 0.125
    ref, mag = O.mm(a, O.E5M2, b, O.E4M3, sa, sb, bias.astype(np.float64))
    A = km_view(a, pad=16) if "A" in layout else to_dev_codes(a)
    B = km_view(b, pad=32) if "B" in layout else to_dev_codes(b)
    y = fp8mi.fp8_mm(A, B, 1, 0, scalar(sa), scalar(sb), torch.from_numpy(bias).to(DEV))
    y_nt = fp8mi.fp8_mm(to_dev_codes(a), to_dev_codes(b), 1, 0, scalar(sa), scalar(sb), torch.from_numpy(bias).to(DEV))
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y_nt.view(torch.int16))
    assert np.array_equal(np_bf16_bits(y).reshape(ref.shape), ref)


@pytest.mark.parametrize("layout", ["A", "B", "AB"])
def test_gaussian_4096_against_nt(layout):
    M = N = K = 4096
    a = make_codes((M, K), O.E4M3, 51, 0)
    b = make_codes((N, K), O.E4M3, 51, 1)
    sa, sb = 0.01, 0.02
    A = km_view(a) if "A" in layout else to_dev_codes(a)
    B = km_view(b) if "B" in layout else to_dev_codes(b)
    y = fp8mi.fp8_mm(A, B, 0, 0, scalar(sa), scalar(sb))
    y_nt = fp8mi.fp8_mm(to_dev_codes(a), to_dev_codes(b), 0, 0, scalar(sa), scalar(sb))
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y_nt.view(torch.int16))
    rows = sample_rows(M, 32, 51, 2)
    check(np_bf16_bits(y), a, O.E4M3, b, O.E4M3, sa, sb, None, rows, tag=f"4096^3 {layout}")


def test_backward_without_transposed_codes():
    """dX = G W and dW = G^T X of the training shapes straight from the row
    codes of W, G and X (K-major B for dX, K-major A and B for dW) equal the
    NT GEMMs on the transposed codes."""
    M, Kin, Nout = 2048, 1536, 6912
    g = make_codes((M, Nout), O.E5M2, 52, 0)
    w = make_codes((Nout, Kin), O.E4M3, 52, 1)
    x = make_codes((M, Kin), O.E4M3, 52, 2)
    G, W, X = to_dev_codes(g), to_dev_codes(w), to_dev_codes(x)
    sg, sw, sx = scalar(1 / 512), scalar(1 / 64), scalar(1 / 128)
    dx = fp8mi.fp8_mm(G, W.t(), 1, 0, sg, sw)                   # B = W^T view: K-major over Nout
    dx_nt = fp8mi.fp8_mm(G, to_dev_codes(w.T), 1, 0, sg, sw)
    dw = fp8mi.fp8_mm(G.t(), X.t(), 1, 0, sg, sx)               # A = G^T, B = X^T: both K-major over M
    dw_nt = fp8mi.fp8_mm(to_dev_codes(g.T), to_dev_codes(x.T), 1, 0, sg, sx)
    torch.cuda.synchronize()
    assert torch.equal(dx.view(torch.int16), dx_nt.view(torch.int16))
    assert torch.equal(dw.view(torch.int16), dw_nt.view(torch.int16))
    rows = sample_rows(M, 24, 52, 3)
    check(np_bf16_bits(dx), g, O.E5M2, np.ascontiguousarray(w.T), O.E4M3, 1 / 512, 1 / 64, None, rows, tag="dX")


FP8_OUT_CASES = [((64, 256, 256, 1), "AB"), ((130, 257, 272, 1), "A"), ((130, 257, 272, 1), "B"),
                 ((64, 4096, 1024, 1), "AB"),
                 ((1000, 1537, 2048, 1), "AB"), ((256, 384, 640, 3), "A"), ((17, 33, 48, 2), "B"),
                 ((8000, 6900, 1536, 1), "A")]


@pytest.mark.parametrize("case", FP8_OUT_CASES, ids=lambda c: "x".join(map(str, c[0])) + "-" + c[1])
@pytest.mark.parametrize("fmt_c", [O.E4M3, O.E5M2], ids=["e4m3", "e5m2"])
def test_layout_fp8_output_equals_nt(case, fmt_c):
    """K-major operands with the quantizing epilogue: codes, 1/s, amax and the
    output ring's words equal those of the NT call on the same codes, bit for
    bit -- with the output's ring (a fresh ring per call, folded once) and with
    an explicit scale (K = 256 takes the precise accumulation; 8000 x 6900 x
    1536 the mixed grid)."""
    (M, N, K, batch), layout = case
    a = make_codes((batch, M, K), O.E4M3, 53, M, K, 0)
    b = make_codes((batch, N, K), O.E5M2, 53, M, K, 1)
    bias = torch.from_numpy(synth.rng(53, M, 2).standard_normal(N).astype(np.float32)).to(DEV)
    sa, sb = scalar(0.03125), scalar(0.5)
    A = km_view(a, pad=16) if "A" in layout else to_dev_codes(a)
    B = km_view(b, pad=32) if "B" in layout else to_dev_codes(b)
    outs = []
    for x, y in ((A, B), (to_dev_codes(a), to_dev_codes(b))):
        ring = fp8mi.new_ring(16, 1.0, DEV)
        sinv_r, amax_r = torch.zeros(1, device=DEV), torch.zeros(1, device=DEV)
        q_r = fp8mi.fp8_mm_ex(x, y, 0, 1, sa, sb, bias, out_fmt=FID[fmt_c], out_ring=ring, out_scale_inv=sinv_r,
                              out_amax=amax_r)
        sinv_s, amax_s = torch.zeros(1, device=DEV), torch.zeros(1, device=DEV)
        q_s = fp8mi.fp8_mm_ex(x, y, 0, 1, sa, sb, bias, out_fmt=FID[fmt_c], out_scale=scalar(0.75),
                              out_scale_inv=sinv_s, out_amax=amax_s)
        torch.cuda.synchronize()
        outs.append([q_r.cpu(), ring.cpu(), sinv_r.cpu(), amax_r.cpu(), q_s.cpu(), sinv_s.cpu(), amax_s.cpu()])
    names = ["codes (ring)", "ring words", "1/s (ring)", "amax (ring)", "codes (scale)", "1/s (scale)", "amax (scale)"]
    for name, km, nt in zip(names, outs[0], outs[1]):
        assert torch.equal(km.contiguous().view(torch.uint8), nt.contiguous().view(torch.uint8)), name
    assert float(outs[1][3]) > 0 and float(outs[1][6]) > 0
