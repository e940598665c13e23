"""Seeded random cases.  Sizes, paddings, base offsets, formats, input dtypes,
layouts, batches, broadcast operands, K-major operands and bias types are
drawn together, so combinations that the fixed matrices of the other tests do
not list still meet the bar.

* quantize (150 cases): rows, cols in [1, 700]; bf16 / fp16 / fp32 input
  N(0, sigma^2) with sigma log-uniform in [2^-8, 2^8], at a base 0-7
  elements past an allocation start, with 0-40 elements of row padding;
  outputs at a base 0-15 bytes past an allocation start, with 0-40 bytes of
  row padding; E4M3 / E5M2; row, transposed and dual layout with an explicit
  scale or a ring holding a random history, or current scaling (row / dual).
  Codes bit-exact with the padding bytes untouched; amax, scale_inv and ring
  words bit-exact.
* GEMM (150 cases): M, N in [1, 600], K a multiple of 16 in [16, 1024],
  batch 1-3 with A or B broadcast, padded leading dimensions, each operand
  K-major with probability 1/3, E4M3 / E5M2 operands, no / f32 / f16 / bf16
  bias, a bf16 output with a padded ldc.  Small-integer data and power-of-two
  scales make every partial sum exact, so every output is bit-exact.
* quantizing epilogue (60 cases): NT operands as above, E4M3 / E5M2 output
  codes with an explicit scale or a ring, no / bf16 / fp8-stored bias; codes,
  amax, scale_inv and ring words bit-exact.
* bias gradient (60 cases), standalone or fused into the dual quantize, on
  random shapes, offsets and paddings with exactly summable data: bit-exact.
"""
import numpy as np
import pytest
import torch

import oracle as O
import synth
from tests.gpu_util import DEV, as_bits, check, codes_out, f32_bits, padding_untouched, ring_from_oracle, \
    ring_state_words, scalar, to_device
from tests.test_mm_gpu import make_int_codes

pytestmark = pytest.mark.gpu

fp8mi = pytest.importorskip("fp8_tensor_scaled_quantize_amd")
FID = {O.E4M3: 0, O.E5M2: 1}
DTYPES = ["bf16", "f16", "f32"]
N_CASES = 150


def quant_case(i):
    r = synth.rng(9100, i)
    c = {"rows": int(r.integers(1, 701)), "cols": int(r.integers(1, 701)), "dtype": DTYPES[int(r.integers(0, 3))],
         "fmt": [O.E4M3, O.E5M2][int(r.integers(0, 2))], "sigma": float(2.0 ** r.uniform(-8, 8)),
         "misalign": int(r.integers(0, 8)), "pad": int(r.integers(0, 41)), "out_misalign": int(r.integers(0, 16)),
         "out_pad": int(r.integers(0, 41)), "mode": ["row", "trans", "dual", "dyn_row", "dyn_dual"][int(r.integers(0, 5))],
         "ring": bool(r.integers(0, 2)), "H": [1, 4, 16][int(r.integers(0, 3))], "scale_log2": float(r.uniform(-6, 6))}
    return c


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_quantize(i):
    c = quant_case(i)
    rows, cols, fmt = c["rows"], c["cols"], c["fmt"]
    x = synth.gaussian((rows, cols), c["sigma"], c["dtype"], 9101, i)
    xd = to_device(x, c["dtype"], c["misalign"], cols + c["pad"])
    dyn = c["mode"].startswith("dyn")
    row_out = c["mode"] in ("row", "dual", "dyn_row", "dyn_dual")
    t_out = c["mode"] in ("trans", "dual", "dyn_dual")
    o_row = codes_out(rows, cols, cols + c["out_pad"], c["out_misalign"]) if row_out else None
    o_t = codes_out(cols, rows, rows + c["out_pad"], c["out_misalign"]) if t_out else None
    sinv, amax = scalar(-1), scalar(-1)
    ring = None
    if dyn:
        ref = O.quantize_dynamic(x, c["dtype"], fmt)
        layout = fp8mi.LAYOUT_DUAL if t_out else fp8mi.LAYOUT_ROW
        fp8mi.fp8_quantize_dynamic(xd, FID[fmt], layout, out_row=o_row, out_t=o_t, scale_inv_out=sinv, amax_out=amax)
    else:
        if c["ring"]:
            r = synth.rng(9102, i)
            ring0 = O.Ring.new(c["H"], 1.0)
            ring0.hist[:] = (r.uniform(0, 4, size=c["H"]) * c["sigma"]).astype(np.float32)
            ring0.idx = int(r.integers(0, c["H"]))
            ring0.scale = np.float32(2.0 ** c["scale_log2"] / c["sigma"])
            ref = O.quantize(x, c["dtype"], fmt, ring=ring0)
            ring, scale_t = ring_from_oracle(ring0), None
        else:
            s = np.float32(2.0 ** c["scale_log2"] / c["sigma"])
            ref = O.quantize(x, c["dtype"], fmt, scale=s)
            scale_t = scalar(s)
        if c["mode"] == "dual":
            fp8mi.fp8_quantize_dual(xd, FID[fmt], out_row=o_row, out_t=o_t, scale=scale_t, ring=ring,
                                    scale_inv_out=sinv, amax_out=amax)
        else:
            fp8mi.fp8_quantize(xd, FID[fmt], c["mode"] == "trans", out=o_row if row_out else o_t, scale=scale_t,
                               ring=ring, scale_inv_out=sinv, amax_out=amax)
    torch.cuda.synchronize()
    if row_out:
        assert np.array_equal(o_row.cpu().numpy(), ref["codes"]), c
        assert padding_untouched(o_row), c
    if t_out:
        assert np.array_equal(o_t.cpu().numpy(), ref["codes_t"]), c
        assert padding_untouched(o_t), c
    assert f32_bits(amax) == as_bits(ref["amax"]), c
    assert f32_bits(sinv) == as_bits(ref["scale_inv"]), c
    if ring is not None:
        assert np.array_equal(ring_state_words(ring), ref["ring"].words()), c


def mm_case(i):
    r = synth.rng(9200, i)
    batch = int(r.integers(1, 4))
    c = {"M": int(r.integers(1, 601)), "N": int(r.integers(1, 601)), "K": 16 * int(r.integers(1, 65)),
         "batch": batch, "bcast": ["none", "a", "b"][int(r.integers(0, 3))] if batch > 1 else "none",
         "fa": [O.E4M3, O.E5M2][int(r.integers(0, 2))], "fb": [O.E4M3, O.E5M2][int(r.integers(0, 2))],
         "a_km": bool(r.integers(0, 3) == 0), "b_km": bool(r.integers(0, 3) == 0),
         "pad_a": 16 * int(r.integers(0, 3)), "pad_b": 16 * int(r.integers(0, 3)), "pad_c": int(r.integers(0, 9)),
         "bias": [None, "f32", "f16", "bf16"][int(r.integers(0, 4))],
         "sa_log2": int(r.integers(-2, 3)), "sb_log2": int(r.integers(-2, 3))}
    return c


def operand(codes, km, pad):
    """Device operand [b, rows, K] holding `codes`: row-major with ld = K +
    pad, or K-major -- [b, K, ld] storage with ld = rows rounded up to 16 +
    pad, viewed transposed."""
    b, rows, K = codes.shape
    if not km:
        store = torch.zeros((b, rows, K + pad), dtype=torch.uint8)
        store[:, :, :K] = torch.from_numpy(codes)
        return store.to(DEV)[:, :, :K]
    ld = (rows + 15) // 16 * 16 + pad
    store = torch.zeros((b, K, ld), dtype=torch.uint8)
    store[:, :, :rows] = torch.from_numpy(np.ascontiguousarray(codes.transpose(0, 2, 1)))
    return store.to(DEV)[:, :, :rows].transpose(1, 2)


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_gemm(i):
    c = mm_case(i)
    M, N, K, batch = c["M"], c["N"], c["K"], c["batch"]
    ba = 1 if c["bcast"] == "a" else batch
    bb = 1 if c["bcast"] == "b" else batch
    a = make_int_codes((ba, M, K), c["fa"], 9201, i)
    b = make_int_codes((bb, N, K), c["fb"], 9202, i)
    sa, sb = 2.0 ** c["sa_log2"], 2.0 ** c["sb_log2"]
    bias_np = bias_t = None
    if c["bias"] is not None:
        bias_np = synth.rng(9203, i).integers(-8, 9, size=N).astype(np.float64)
        bias_t = torch.from_numpy(bias_np).to({"f32": torch.float32, "f16": torch.float16,
                                                "bf16": torch.bfloat16}[c["bias"]]).to(DEV)
    out = torch.full((batch, M, N + c["pad_c"]), float("nan"), dtype=torch.bfloat16, device=DEV)[:, :, :N]
    if batch == 1:
        out = out[0]
    y = fp8mi.fp8_mm(operand(a, c["a_km"], c["pad_a"]), operand(b, c["b_km"], c["pad_b"]), FID[c["fa"]], FID[c["fb"]],
                     scalar(sa), scalar(sb), bias_t, out=out)
    torch.cuda.synchronize()
    assert y.data_ptr() == out.data_ptr()
    got = y.contiguous().cpu().view(torch.int16).numpy().view(np.uint16)
    check(got, a if ba > 1 or batch > 1 else a[0], c["fa"], b if bb > 1 or batch > 1 else b[0], c["fb"], sa, sb,
          bias_np, tag=str(c), exact=True)


@pytest.mark.parametrize("i", range(60))
def test_random_gemm_fp8_out(i):
    """The quantizing epilogue on random cases: operands as above (K-major
    with probability 1/3 each), E4M3 / E5M2 output codes with an
    explicit scale or a ring holding a random history, no / bf16 / fp8 bias
    (E4M3 / E5M2 codes with a power-of-two bias scale).  Small-integer data and
    power-of-two scales: codes, amax, scale_inv and ring words bit-exact."""
    c = mm_case(1000 + i)
    r = synth.rng(9300, i)
    fmt_c = [O.E4M3, O.E5M2][int(r.integers(0, 2))]
    bias_kind = [None, "bf16", O.E4M3, O.E5M2][int(r.integers(0, 4))]
    use_ring = bool(r.integers(0, 2))
    M, N, K, batch = c["M"], c["N"], c["K"], c["batch"]
    ba = 1 if c["bcast"] == "a" else batch
    bb = 1 if c["bcast"] == "b" else batch
    a = make_int_codes((ba, M, K), c["fa"], 9301, i)
    b = make_int_codes((bb, N, K), c["fb"], 9302, i)
    sa, sb = 2.0 ** c["sa_log2"], 2.0 ** c["sb_log2"]
    bias_v = bias_t = bias_fmt = bias_scale = None
    if bias_kind == "bf16":
        bias_v = r.integers(-8, 9, size=N).astype(np.float64)
        bias_t = torch.from_numpy(bias_v).to(torch.bfloat16).to(DEV)
    elif bias_kind is not None:
        codes = make_int_codes((N,), bias_kind, 9303, i)
        sbias = 2.0 ** int(r.integers(-2, 3))
        bias_v = O.dequant_bias(codes, bias_kind, sbias).astype(np.float64)
        bias_t, bias_fmt, bias_scale = torch.from_numpy(codes).to(DEV), FID[bias_kind], scalar(sbias)
    # output scale near fmt_max / (a typical |y|) so codes spread over the range
    s_c = np.float32(O.FMT_MAX[fmt_c] / 2.0 ** int(r.integers(6, 14)))
    ring = scale_t = None
    if use_ring:
        ring0 = O.Ring.new(4, 1.0)
        ring0.hist[:] = r.uniform(0, 4000, size=4).astype(np.float32)
        ring0.idx, ring0.scale = int(r.integers(0, 4)), s_c
        ref = O.mm_quantized(a if batch > 1 else a[0], c["fa"], b if batch > 1 else b[0], c["fb"], fmt_c, sa, sb,
                             bias_v, ring=ring0)
        ring = ring_from_oracle(ring0)
    else:
        ref = O.mm_quantized(a if batch > 1 else a[0], c["fa"], b if batch > 1 else b[0], c["fb"], fmt_c, sa, sb,
                             bias_v, scale=s_c)
        scale_t = scalar(s_c)
    sinv, amax = scalar(-1), scalar(-1)
    out = fp8mi.fp8_mm_ex(operand(a, c["a_km"], c["pad_a"]) if batch > 1 else operand(a, c["a_km"], c["pad_a"])[0],
                          operand(b, c["b_km"], c["pad_b"]) if batch > 1 else operand(b, c["b_km"], c["pad_b"])[0],
                          FID[c["fa"]], FID[c["fb"]], scalar(sa), scalar(sb), bias_t, bias_fmt, bias_scale,
                          out_fmt=FID[fmt_c], out_scale=scale_t, out_ring=ring, out_scale_inv=sinv, out_amax=amax)
    torch.cuda.synchronize()
    want = ref["codes"].reshape(out.shape)
    assert np.array_equal(out.cpu().numpy(), want), c
    assert f32_bits(amax) == as_bits(ref["amax"]), c
    assert f32_bits(sinv) == as_bits(ref["scale_inv"]), c
    if ring is not None:
        assert np.array_equal(ring_state_words(ring), ref["ring"].words()), c


@pytest.mark.parametrize("i", range(60))
def test_random_bias_grad(i):
    """The bias gradient, standalone and fused into the dual quantize, on
    random shapes (rows, cols in [1, 1500]), bf16 / fp16 gradients at a base
    0-7 elements past an allocation start with 0-40 elements of row padding.
    Values are small integers times 2^-6, so every float64 sum is exact and
    the once-rounded bf16 result must equal the oracle's bit for bit; the
    fused call's codes, amax and scale_inv are bit-exact too."""
    r = synth.rng(9400, i)
    rows, cols = int(r.integers(1, 1501)), int(r.integers(1, 1501))
    dt = ["bf16", "f16"][int(r.integers(0, 2))]
    fused = bool(r.integers(0, 2))
    v = (r.integers(-64, 65, size=(rows, cols)) * 2.0 ** -6).astype(np.float32)
    dy = synth.f32_to_bf16_bits(v) if dt == "bf16" else v.astype(np.float16)
    dyd = to_device(dy, dt, int(r.integers(0, 8)), cols + int(r.integers(0, 41)))
    ref_db, _ = O.grad_bias(dy, dt)
    if fused:
        fmt = [O.E4M3, O.E5M2][int(r.integers(0, 2))]
        s = np.float32(2.0 ** int(r.integers(-2, 6)))
        ref = O.quantize(dy, dt, fmt, scale=s)
        sinv, amax = scalar(-1), scalar(-1)
        q, qt, db = fp8mi.fp8_quantize_dual_bias_grad(dyd, FID[fmt], scale=scalar(s), scale_inv_out=sinv,
                                                      amax_out=amax)
        torch.cuda.synchronize()
        assert np.array_equal(q.cpu().numpy(), ref["codes"]) and np.array_equal(qt.cpu().numpy(), ref["codes_t"])
        assert f32_bits(amax) == as_bits(ref["amax"]) and f32_bits(sinv) == as_bits(ref["scale_inv"])
    else:
        db = fp8mi.fp8_bias_grad(dyd)
        torch.cuda.synchronize()
    got = db.cpu().view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, ref_db), (rows, cols, dt, fused)
