"""GPU parity of fp8_quantize_dynamic (current scaling) against the oracle's
quantize_dynamic: codes, amax and scale_inv bit-exact, for every layout,
input type, alignment and stride, including where the amax element sits in
the unaligned head or the ragged tail of the input."""
import numpy as np
import pytest
import torch

import oracle as O
import synth
from tests.gpu_util import DEV, as_bits, codes_out, f32_bits, np_codes, padding_untouched, scalar, to_device

pytestmark = pytest.mark.gpu
fp8mi = pytest.importorskip("fp8_tensor_scaled_quantize_amd")

FMTS = [(O.E4M3, 0), (O.E5M2, 1)]
SHAPES = [(1, 1), (1, 7), (7, 1), (3, 1535), (64, 32), (65, 33), (127, 129), (128, 1536), (256, 256),
          (2048, 1536), (1535, 8192), (8192, 1535), (8192, 1536)]
LAYOUTS = [("row", 0), ("t", 1), ("dual", 2)]


def garbage_workspace():
    return torch.full((fp8mi.DYNAMIC_WORKSPACE_BYTES // 4,), float("nan"), dtype=torch.float32, device=DEV)


def run(xd, fid, layout, rows, cols, ws=None, pad=0):
    amax_t, sinv_t = scalar(-1.0), scalar(-1.0)
    o = codes_out(rows, cols, cols + pad) if layout != 1 else None
    ot = codes_out(cols, rows, rows + pad) if layout != 0 else None
    fp8mi.fp8_quantize_dynamic(xd, fid, layout, out_row=o, out_t=ot, scale_inv_out=sinv_t, amax_out=amax_t,
                               workspace=garbage_workspace() if ws is None else ws)
    torch.cuda.synchronize()
    return o, ot, amax_t, sinv_t


def check(ref, o, ot, a, si, tag, pad=False):
    if o is not None:
        assert np.array_equal(np_codes(o), ref["codes"]), tag
    if ot is not None:
        assert np.array_equal(np_codes(ot), ref["codes_t"]), tag
    assert f32_bits(a) == as_bits(ref["amax"]), tag
    assert f32_bits(si) == as_bits(ref["scale_inv"]), tag
    if pad:
        assert all(padding_untouched(v) for v in (o, ot) if v is not None), tag


@pytest.mark.parametrize("dtype", O.DTYPES)
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: f"{s[0]}x{s[1]}")
def test_dynamic_matrix(shape, dtype):
    """Current scaling over the same shape list, every input dtype, both
    formats and the three layouts, each from an aligned base, a base one
    element off and padded rows: codes, amax and 1/s equal the oracle's."""
    rows, cols = shape
    sid = SHAPES.index(shape)
    sigma = (1.0, 3e-3, 250.0)[sid % 3]
    x = synth.gaussian(shape, sigma, dtype, 95, sid, O.DTYPES.index(dtype))
    inputs = [("aligned", to_device(x, dtype), 0), ("misaligned", to_device(x, dtype, misalign=1), 16),
              ("strided", to_device(x, dtype, misalign=3, ld=cols + 5), 0)]
    for fmt, fid in FMTS:
        ref = O.quantize_dynamic(x, dtype, fmt)
        for name, xd, pad in inputs:
            for lname, layout in LAYOUTS:
                o, ot, a, si = run(xd, fid, layout, rows, cols, pad=pad)
                check(ref, o, ot, a, si, f"{fmt} {name} {lname}", pad=bool(pad))


@pytest.mark.parametrize("dtype", O.DTYPES)
def test_dynamic_amax_element_anywhere(dtype):
    """One spike, larger than everything else, placed in the unaligned head,
    the 16-byte body, the ragged tail and the last element, of contiguous and
    strided inputs: the scale must follow it every time."""
    rows, cols = 37, 203
    base = synth.gaussian((rows, cols), 1.0, dtype, 96, 0)
    n = rows * cols
    spike = {"bf16": np.uint16(0x4300), "f16": np.float16(2000.0), "f32": np.float32(3.0e4)}[dtype]  # 128.0 as bf16
    for pos in (0, 1, 2, 6, 7, 8, 9, 100, cols - 1, cols, n // 2, n - 9, n - 8, n - 2, n - 1):
        x = base.copy()
        x.reshape(-1)[pos] = spike
        for fmt, fid in FMTS:
            ref = O.quantize_dynamic(x, dtype, fmt)
            for mis, ld in ((0, None), (1, None), (3, cols + 9)):
                xd = to_device(x, dtype, misalign=mis, ld=ld)
                o, ot, a, si = run(xd, fid, 2, rows, cols)
                check(ref, o, ot, a, si, f"pos={pos} {fmt} mis={mis} ld={ld}")


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("fmt,fid", FMTS)
def test_dynamic_every_16bit_pattern(dtype, fmt, fid):
    """All 65536 patterns: the infinities make amax inf and the scale 1; NaN
    stays out of amax.  Without the infinities amax is the largest finite."""
    bits = np.arange(65536, dtype=np.uint16).reshape(256, 256)
    inf = 0x7F80 if dtype == "bf16" else 0x7C00
    finite = bits.copy()
    finite[(finite & 0x7FFF) == inf] = 0
    for b in (bits, finite):
        x = b if dtype == "bf16" else b.view(np.float16)
        ref = O.quantize_dynamic(x, dtype, fmt)
        for lname, layout in LAYOUTS:
            o, ot, a, si = run(to_device(x, dtype), fid, layout, 256, 256)
            check(ref, o, ot, a, si, f"{lname}")


def test_dynamic_degenerate_tensors():
    cases = [
        ("zeros", np.zeros((5, 70), np.float32)),
        ("negative zeros", np.full((3, 9), -0.0, np.float32)),
        ("nan and finite", np.array([[np.nan, -2.5, 1.0], [0.5, np.nan, 0.0]], np.float32)),
        ("all nan", np.full((4, 4), np.nan, np.float32)),
        ("quotient overflows", np.array([[1e-39, -2e-39, 0.0, 5e-40]], np.float32)),
        ("largest finite", np.array([[3.4028234e38, -1.0, 2.0]], np.float32)),
        ("inf", np.array([[np.inf, 1.0], [-3.0, 2.0]], np.float32)),
    ]
    for name, x in cases:
        for fmt, fid in FMTS:
            ref = O.quantize_dynamic(x, O.F32, fmt)
            for lname, layout in LAYOUTS:
                o, ot, a, si = run(to_device(x, "f32"), fid, layout, *x.shape)
                check(ref, o, ot, a, si, f"{name} {fmt} {lname}")


def test_dynamic_golden_worked_on_device():
    import os
    from tests.test_oracle_pins import _golden_input
    n = 0
    for line in open(os.path.join(os.path.dirname(__file__), "golden", "dynamic_worked.txt")):
        line = line.split("#")[0].strip()
        if not line:
            continue
        case, fmt, dtype, vals, sinv, am, codes = line.split()
        x = _golden_input([float(v) for v in vals.split(",")], dtype)[None, :]
        o, ot, a, si = run(to_device(x, dtype), {O.E4M3: 0, O.E5M2: 1}[fmt], 2, *x.shape)
        assert np_codes(o)[0].tolist() == [int(c, 16) for c in codes.split(",")], case
        assert f32_bits(si) == as_bits(np.float32(float(sinv))), case
        assert f32_bits(a) == as_bits(np.float32(float(am))), case
        n += 1
    assert n == 8


def test_dynamic_empty():
    for shape in ((0, 0), (0, 17), (9, 0)):
        x = np.zeros(shape, np.float32)
        o, ot, a, si = run(to_device(x, "f32"), 0, 2, *shape)
        assert f32_bits(a) == as_bits(0.0) and f32_bits(si) == as_bits(1.0), shape


def test_dynamic_workspace_reused_across_calls():
    """One workspace, a large call then a small one (fewer partials): the
    second must not see the first call's partials; a short workspace is
    refused before anything is written."""
    ws = garbage_workspace()
    big = synth.gaussian((4096, 3072), 50.0, "bf16", 97, 0)
    small = synth.gaussian((33, 65), 1e-2, "bf16", 97, 1)
    for x in (big, small, big):
        ref = O.quantize_dynamic(x, "bf16", O.E4M3)
        o, ot, a, si = run(to_device(x, "bf16"), 0, 0, *x.shape, ws=ws)
        check(ref, o, ot, a, si, f"{x.shape}")
    short = torch.empty(fp8mi.DYNAMIC_WORKSPACE_BYTES - 4, dtype=torch.uint8, device=DEV)
    with pytest.raises(fp8mi.Fp8Error):
        fp8mi.fp8_quantize_dynamic(to_device(small, "bf16"), 0, 0, workspace=short)


@pytest.mark.parametrize("fmt,fid", FMTS)
def test_dynamic_full_size_output_gradient(fmt, fid):
    """The output-gradient shape of the training step (bf16 8192 x 6912,
    persistent dual kernel): amax and scale exact, codes on sampled rows and
    columns against the oracle with the same scale."""
    x = synth.gaussian((8192, 6912), 1e-3, "bf16", 98, fid)
    xd = to_device(x, "bf16")
    o, ot, a, si = run(xd, fid, 2, 8192, 6912)
    xf = O.widen_to_f32(x, "bf16")
    amax = O.amax(xf)
    s = O.next_scale(np.array([amax], np.float32), fmt)
    assert f32_bits(a) == as_bits(amax)
    assert f32_bits(si) == as_bits(O.scale_inv(s))
    g = synth.rng(98, 2)
    rsel = np.sort(g.choice(8192, 48, replace=False))
    csel = np.sort(g.choice(6912, 48, replace=False))
    got_r = o[torch.from_numpy(rsel).to(DEV)].cpu().numpy()
    assert np.array_equal(got_r, O.quantize(x[rsel], "bf16", fmt, scale=s)["codes"])
    got_t = ot[torch.from_numpy(csel).to(DEV)].cpu().numpy()
    assert np.array_equal(got_t, O.quantize(np.ascontiguousarray(x[:, csel]), "bf16", fmt, scale=s)["codes_t"])
