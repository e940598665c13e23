"""Quantize with scales that are not finite nonzero numbers, against the oracle.

The oracle defines the code of every element as enc(fl32(x * s)) for any
fp32 s.  With s = 0, +-inf or NaN, the product is NaN for some inputs that are
not NaN (0 * inf, inf * 0, anything * NaN), so the raw input alone no longer
says which elements are NaN.  Inputs hold +-0, +-inf, NaN of both signs, fp32
or fp16 subnormals and Gaussian values; every kernel form is run: row
(contiguous, misaligned, persistent), transposed and dual (one-shot and
persistent), delayed scaling through a ring whose scale word holds the
irregular value, and the GEMM's quantizing epilogue with an irregular output
scale.

Codes are compared bit for bit, except the sign bit of a NaN code whose NaN
arose in the multiply itself (0 * inf, or a NaN scale): IEEE leaves the sign
of such a NaN unspecified (the NaN-sign rule for GEMM outputs is the same).  A
NaN input times a non-NaN scale keeps its sign on both sides, and that sign is
compared.  amax (raw input), scale_inv (1 / s) and ring words are bit-exact."""
import numpy as np
import pytest
import torch

import oracle as O
import synth
from tests.gpu_util import (DEV, as_bits, codes_out, f32_bits, np_codes, ring_from_oracle, ring_state_words,
                            scalar, to_device)
from tests.test_mm_gpu import make_int_codes, to_dev_codes

pytestmark = pytest.mark.gpu
fp8mi = pytest.importorskip("fp8_tensor_scaled_quantize_amd")

SCALES = [0.0, -0.0, np.inf, -np.inf, np.nan, 2.0 ** -149, -1.5]
FID = {O.E4M3: 0, O.E5M2: 1}

# special storage values per dtype: +0, -0, +inf, -inf, +NaN, -NaN, smallest subnormal, largest finite
SPECIAL_BITS = {
    "bf16": np.array([0x0000, 0x8000, 0x7F80, 0xFF80, 0x7FC0, 0xFFC1, 0x0001, 0x7F7F], np.uint16),
    "f16": np.array([0x0000, 0x8000, 0x7C00, 0xFC00, 0x7E00, 0xFE01, 0x0001, 0x7BFF], np.uint16),
    "f32": np.array([0x00000000, 0x80000000, 0x7F800000, 0xFF800000, 0x7FC00000, 0xFFC00001, 0x00000001,
                     0x7F7FFFFF], np.uint32),
}


def special_input(shape, dtype, key):
    """Gaussian values with a special value planted at every 5th element of
    every row (shifted per row, cycling through SPECIAL_BITS)."""
    x = synth.gaussian(shape, 1.0, dtype, 95, key)
    rows, cols = shape
    sp = SPECIAL_BITS[dtype]
    if dtype == "f16":
        sp = sp.view(np.float16)
    elif dtype == "f32":
        sp = sp.view(np.float32)
    r, c = np.meshgrid(np.arange(rows), np.arange(cols), indexing="ij")
    sel = (c + r) % 5 == 0
    x[sel] = sp[((c + 3 * r) // 5 % len(sp))[sel]]
    return x


def assert_codes_match(got, x_f32, s, ref, tag):
    """Bit-exact, except the sign bit of NaN codes produced by the multiply."""
    with np.errstate(invalid="ignore", over="ignore"):
        prod = O.scaled_values(x_f32, s)
    arith_nan = np.isnan(prod) & ~(np.isnan(x_f32) & ~np.isnan(np.float32(s)))
    mask = np.where(arith_nan, 0x7F, 0xFF).astype(np.uint8)
    bad = (got & mask) != (ref & mask)
    assert not bad.any(), f"{tag}: {bad.sum()} of {bad.size} codes differ"


def assert_f32_same(dev_word, ref, tag):
    g = np.array([f32_bits(dev_word)], np.uint32).view(np.float32)[0]
    r = np.float32(ref)
    assert (np.isnan(g) and np.isnan(r)) or as_bits(g) == as_bits(r), f"{tag}: {g} != {r}"


@pytest.mark.parametrize("dtype", O.DTYPES)
@pytest.mark.parametrize("shape,misalign", [((64, 512), 0), ((130, 257), 1), ((1, 7), 0)],
                         ids=["flat", "tiled-misaligned", "tiny"])
def test_irregular_explicit_scales(shape, misalign, dtype):
    rows, cols = shape
    x = special_input(shape, dtype, 1 + rows)
    xf = O.widen_to_f32(x, dtype)
    xd = to_device(x, dtype, misalign=misalign)
    for fmt, fid in FID.items():
        for s in SCALES:
            with np.errstate(invalid="ignore", over="ignore", divide="ignore"):
                ref = O.quantize(x, dtype, fmt, scale=np.float32(s))
            tag = f"{dtype} {shape} {fmt} s={s}"
            for layout in ("row", "t", "dual"):
                amax_t, sinv_t = scalar(-1.0), scalar(-1.0)
                if layout == "row":
                    o = codes_out(rows, cols)
                    fp8mi.fp8_quantize(xd, fid, False, out=o, scale=scalar(s), scale_inv_out=sinv_t, amax_out=amax_t)
                    outs = [(np_codes(o), ref["codes"], xf)]
                elif layout == "t":
                    o = codes_out(cols, rows)
                    fp8mi.fp8_quantize(xd, fid, True, out=o, scale=scalar(s), scale_inv_out=sinv_t, amax_out=amax_t)
                    outs = [(np_codes(o), ref["codes_t"], xf.T)]
                else:
                    o, ot = fp8mi.fp8_quantize_dual(xd, fid, scale=scalar(s), scale_inv_out=sinv_t, amax_out=amax_t)
                    outs = [(np_codes(o), ref["codes"], xf), (np_codes(ot), ref["codes_t"], xf.T)]
                torch.cuda.synchronize()
                for got, want, xs in outs:
                    assert_codes_match(got, xs, s, want, f"{tag} {layout}")
                assert f32_bits(amax_t) == as_bits(ref["amax"]), f"{tag} {layout} amax"
                assert_f32_same(sinv_t, ref["scale_inv"], f"{tag} {layout} scale_inv")


@pytest.mark.parametrize("s", [0.0, np.inf, np.nan], ids=["zero", "inf", "nan"])
def test_irregular_scale_persistent_kernels(s):
    """Tensors above the one-shot size (4160 x 4096 bf16: the persistent row
    and tiled kernels), checked on seeded rows and columns."""
    rows, cols = 4160, 4096
    x = special_input((rows, cols), "bf16", 7)
    xd = to_device(x, "bf16")
    rs = np.sort(synth.rng(96, 1).choice(rows, 40, replace=False))
    cs = np.sort(synth.rng(96, 2).choice(cols, 40, replace=False))
    xf = O.widen_to_f32(x, "bf16")
    for fmt, fid in FID.items():
        with np.errstate(invalid="ignore", over="ignore"):
            want_r = O.encode(O.scaled_values(xf[rs], s), fmt)
            want_c = O.encode(O.scaled_values(xf[:, cs], s), fmt).T
        row = fp8mi.fp8_quantize(xd, fid, False, scale=scalar(s))
        o, ot = fp8mi.fp8_quantize_dual(xd, fid, scale=scalar(s))
        torch.cuda.synchronize()
        tag = f"persistent {fmt} s={s}"
        assert_codes_match(np_codes(row[rs]), xf[rs], s, want_r, tag + " row")
        assert_codes_match(np_codes(o[rs]), xf[rs], s, want_r, tag + " dual rows")
        assert_codes_match(np_codes(ot[cs]), xf[:, cs].T, s, want_c, tag + " dual cols")


@pytest.mark.parametrize("s", [0.0, np.inf, np.nan], ids=["zero", "inf", "nan"])
def test_irregular_scale_in_ring(s):
    """Delayed scaling whose ring holds an irregular current scale (a restored
    checkpoint can hold any word): the call quantizes with it, snapshots 1/s,
    folds the raw amax and publishes a regular next scale."""
    x = special_input((96, 320), "f32", 11)
    r0 = O.Ring.new(4, 1.0)
    r0.hist[:] = [2.0, 0.0, 9.0, 1.0]
    r0.scale, r0.idx = np.float32(s), 3
    for fmt, fid in FID.items():
        with np.errstate(invalid="ignore", over="ignore", divide="ignore"):
            ref = O.quantize(x, "f32", fmt, ring=r0)
        ring = ring_from_oracle(r0)
        sinv_t, amax_t = scalar(-1.0), scalar(-1.0)
        o, ot = fp8mi.fp8_quantize_dual(to_device(x, "f32"), fid, ring=ring, scale_inv_out=sinv_t, amax_out=amax_t)
        torch.cuda.synchronize()
        assert_codes_match(np_codes(o), x, s, ref["codes"], f"ring {fmt} s={s}")
        assert_codes_match(np_codes(ot), x.T, s, ref["codes_t"], f"ring {fmt} s={s} t")
        assert_f32_same(sinv_t, ref["scale_inv"], "ring scale_inv")
        assert np.array_equal(ring_state_words(ring), ref["ring"].words())


@pytest.mark.parametrize("s_c", [0.0, np.inf, np.nan], ids=["zero", "inf", "nan"])
@pytest.mark.parametrize("K", [64, 512], ids=["short-k", "long-k"])
def test_irregular_output_scale_in_gemm(s_c, K):
    """FP8-out GEMM with an irregular explicit output scale: small-integer
    codes make y exact; zero rows of A and zero bias columns give y = 0 (0 * inf
    = NaN for s_c = inf), an E5M2 +-inf code in B gives y = +-inf (inf * 0 = NaN
    for s_c = 0).  Codes as the oracle's quantize of fl32(y), NaN positions
    exact, arithmetic NaN signs not compared; amax and 1/s bit-exact."""
    M, N = 160, 96
    a = make_int_codes((M, K), O.E4M3, 97, K, 1)
    b = make_int_codes((N, K), O.E5M2, 97, K, 2)
    a[3] = 0                                   # row of y = bias
    b[5, 16] = 0x7C                            # column 5: + inf * a[:, 16]
    b[9, 0] = 0xFC                             # column 9: - inf * a[:, 0]
    a[:, 16] = np.where(np.arange(M) % 4 == 0, 0, a[:, 16])   # 0 * inf = NaN in y too
    bias = synth.rng(97, K, 3).integers(-8, 9, size=N).astype(np.float32)
    bias[::7] = 0.0                            # y = 0 in row 3 at these columns
    for fmt_c in (O.E4M3, O.E5M2):
        with np.errstate(invalid="ignore", over="ignore", divide="ignore"):
            ref = O.mm_quantized(a, O.E4M3, b, O.E5M2, fmt_c, 0.5, 2.0, bias.astype(np.float64), scale=np.float32(s_c))
        sinv_t, amax_t = scalar(-1.0), scalar(-1.0)
        out = fp8mi.fp8_mm_ex(to_dev_codes(a), to_dev_codes(b), 0, 1, scalar(0.5), scalar(2.0),
                              torch.from_numpy(bias).to(DEV), out_fmt=FID[fmt_c], out_scale=scalar(s_c),
                              out_scale_inv=sinv_t, out_amax=amax_t)
        torch.cuda.synchronize()
        got, want = out.cpu().numpy(), ref["codes"].reshape(M, N)
        nan = (want & 0x7F) == 0x7F
        assert nan.any() and (nan.all() == bool(np.isnan(s_c)))
        assert np.array_equal((got & 0x7F) == 0x7F, nan), f"{fmt_c} s_c={s_c}: NaN codes at different positions"
        assert np.array_equal(got[~nan], want[~nan]), f"{fmt_c} s_c={s_c}: {(got[~nan] != want[~nan]).sum()} differ"
        assert f32_bits(amax_t) == as_bits(ref["amax"])
        assert_f32_same(sinv_t, ref["scale_inv"], f"gemm {fmt_c} s_c={s_c} scale_inv")
