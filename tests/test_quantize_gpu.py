"""GPU parity of fp8_quantize / fp8_quantize_dual / fp8_amax_fold against the
CPU oracle: codes, amax, scale_inv and ring words bit-exact."""
import numpy as np
import pytest
import torch

import oracle as O
import synth
from tests.gpu_util import (DEV, as_bits, codes_out, f32_bits, np_codes, padding_untouched, ring_from_oracle,
                            ring_state_words, ring_to_oracle, scalar, to_device)

pytestmark = pytest.mark.gpu

fp8mi = pytest.importorskip("fp8_tensor_scaled_quantize_amd")
FMTS = [(O.E4M3, 0), (O.E5M2, 1)]
SHAPES = [(1, 1), (1, 7), (7, 1), (3, 1535), (64, 32), (65, 33), (127, 129), (128, 1536), (256, 256),
          (2048, 1536), (1535, 8192), (8192, 1535), (8192, 1536)]


def run_layout(layout, xd, fmt_id, scale_t, misalign, rows, cols):
    """Run one layout; returns (row_codes | None, t_codes | None, amax, scale_inv, views)."""
    amax_t, sinv_t = scalar(-1.0), scalar(-1.0)
    ld_r = cols + (16 if misalign else 0)
    ld_t = rows + (16 if misalign else 0)
    if layout == "row":
        o = codes_out(rows, cols, ld_r)
        fp8mi.fp8_quantize(xd, fmt_id, False, out=o, scale=scale_t, scale_inv_out=sinv_t, amax_out=amax_t)
        return np_codes(o), None, amax_t, sinv_t, [o]
    if layout == "t":
        o = codes_out(cols, rows, ld_t)
        fp8mi.fp8_quantize(xd, fmt_id, True, out=o, scale=scale_t, scale_inv_out=sinv_t, amax_out=amax_t)
        return None, np_codes(o), amax_t, sinv_t, [o]
    o, ot = codes_out(rows, cols, ld_r), codes_out(cols, rows, ld_t)
    fp8mi.fp8_quantize_dual(xd, fmt_id, out_row=o, out_t=ot, scale=scale_t, scale_inv_out=sinv_t, amax_out=amax_t)
    return np_codes(o), np_codes(ot), amax_t, sinv_t, [o, ot]


@pytest.mark.parametrize("dtype", O.DTYPES)
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: f"{s[0]}x{s[1]}")
def test_quantize_matrix(shape, dtype):
    """Every combination of the shape list, input dtype, three scales, both
    formats, the three layouts and an aligned or off-by-one-element base must
    give the oracle's bytes exactly (the pages' quantize commits check their
    kernels against stored records over a similar grid of cases)."""
    rows, cols = shape
    sid = SHAPES.index(shape)
    x = synth.gaussian(shape, 1.0, dtype, 2, synth.T_QUANT, sid, O.DTYPES.index(dtype))
    xf = O.widen_to_f32(x, dtype)
    amax = O.amax(xf)
    x_al = to_device(x, dtype)
    x_mis = to_device(x, dtype, misalign=1)
    for fmt, fid in FMTS:
        fmax = np.float32(O.FMT_MAX[fmt])
        for s in (np.float32(1.0), fmax / amax, np.float32(4.0) * (fmax / amax)):
            ref = O.quantize(x, dtype, fmt, scale=s)
            st = scalar(s)
            for mis, xd in ((0, x_al), (1, x_mis)):
                for layout in ("row", "t", "dual"):
                    r, t, a, si, views = run_layout(layout, xd, fid, st, mis, rows, cols)
                    torch.cuda.synchronize()
                    tag = f"{fmt} s={s} mis={mis} {layout}"
                    if r is not None:
                        assert np.array_equal(r, ref["codes"]), tag
                    if t is not None:
                        assert np.array_equal(t, ref["codes_t"]), tag
                    assert f32_bits(a) == as_bits(ref["amax"]), tag
                    assert f32_bits(si) == as_bits(ref["scale_inv"]), tag
                    if mis:
                        assert all(padding_untouched(v) for v in views), tag


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("fmt,fid", FMTS)
def test_every_16bit_pattern(dtype, fmt, fid):
    """All 65536 bf16 / fp16 bit patterns (NaN, inf, subnormals included), at
    scale 1 and at an awkward scale."""
    bits = np.arange(65536, dtype=np.uint16).reshape(256, 256)
    x = bits if dtype == "bf16" else bits.view(np.float16)
    xd = to_device(x, dtype)
    for s in (np.float32(1.0), np.float32(3.3e-3), np.float32(771.25)):
        ref = O.quantize(x, dtype, fmt, scale=s)
        for tr in (False, True):
            a = scalar(0)
            o = fp8mi.fp8_quantize(xd, fid, tr, scale=scalar(s), amax_out=a)
            got = np_codes(o)
            assert np.array_equal(got, ref["codes_t"] if tr else ref["codes"]), (s, tr)
            assert f32_bits(a) == as_bits(ref["amax"])


@pytest.mark.parametrize("fmt,fid", FMTS)
def test_fp32_patterns(fmt, fid):
    """Random fp32 bit patterns of every class, and the values on and next to
    every rounding boundary of the format, row and transposed."""
    rnd = synth.random_bits_f32(1 << 20, 3, 1)
    grid = np.unique(np.abs(O.decode_table(fmt)[np.isfinite(O.decode_table(fmt))]))
    mids = ((grid[1:] + grid[:-1]) / 2).astype(np.float32)
    edge = []
    for m in list(mids) + [np.float32(O.FMT_MAX[fmt])]:
        for k in range(-3, 4):
            edge.append(np.float32(m).view(np.uint32) + np.uint32(k) if k >= 0 else np.float32(m).view(np.uint32) - np.uint32(-k))
    edge = np.array(edge, dtype=np.uint32).view(np.float32)
    edge = np.concatenate([edge, -edge])
    allv = np.concatenate([rnd, edge, np.zeros((-(len(rnd) + len(edge))) % 1024, np.float32)]).reshape(-1, 1024)
    xd = to_device(allv, "f32")
    for s in (np.float32(1.0), np.float32(0.75)):
        ref = O.quantize(allv, "f32", fmt, scale=s)
        a = scalar(0)
        o = fp8mi.fp8_quantize(xd, fid, False, scale=scalar(s), amax_out=a)
        assert np.array_equal(np_codes(o), ref["codes"])
        ot = fp8mi.fp8_quantize(xd, fid, True, scale=scalar(s))
        assert np.array_equal(np_codes(ot), ref["codes_t"])
        assert f32_bits(a) == as_bits(ref["amax"])


@pytest.mark.parametrize("layout", ["row", "t", "dual"])
@pytest.mark.parametrize("fmt,fid", FMTS)
def test_ring_fold_sequence(layout, fmt, fid):
    """Ring mode: each call quantizes with the ring's scale (snapshot in
    scale_inv_out), folds its raw amax, leaves ticket and accumulator at 0;
    16 calls with a changing amax, bit-exact ring words every call."""
    H = 5
    ring_o = O.Ring.new(H, 17.0)
    ring = ring_from_oracle(ring_o)
    for step in range(16):
        sigma = [1.0, 10.0, 0.1, 3.0][step % 4] * (1 + step)
        x = synth.gaussian((300, 200), sigma, "bf16", 4, step)
        ref = O.quantize(x, "bf16", fmt, ring=ring_o)
        xd = to_device(x, "bf16", misalign=step % 2)
        si, am = scalar(0), scalar(0)
        if layout == "dual":
            r, t = fp8mi.fp8_quantize_dual(xd, fid, ring=ring, scale_inv_out=si, amax_out=am)
            got = [np_codes(r), np_codes(t)]
            want = [ref["codes"], ref["codes_t"]]
        else:
            o = fp8mi.fp8_quantize(xd, fid, layout == "t", ring=ring, scale_inv_out=si, amax_out=am)
            got = [np_codes(o)]
            want = [ref["codes_t"] if layout == "t" else ref["codes"]]
        torch.cuda.synchronize()
        for g, w in zip(got, want):
            assert np.array_equal(g, w), step
        assert f32_bits(si) == as_bits(ref["scale_inv"]), step
        assert f32_bits(am) == as_bits(ref["amax"]), step
        words = ring_state_words(ring)
        assert np.array_equal(words, ref["ring"].words()), (step, words, ref["ring"].words())
        ring_o = ref["ring"]



@pytest.mark.parametrize("dtype", O.DTYPES)
@pytest.mark.parametrize("shape", [(256, 256), (512, 128), (2048, 1536)], ids=lambda s: f"{s[0]}x{s[1]}")
def test_ring_sequence_whole_aligned_tiles(shape, dtype):
    """Ring mode on tensors of whole 128 x 64 tiles with aligned rows (the
    one-shot kernels' specialised form and their early amax publication):
    codes, scale_inv, amax and ring words bit-exact over 6 calls per layout."""
    fmt, fid = FMTS[0]
    for layout in ("row", "t", "dual"):
        ring_o = O.Ring.new(4, 3.0)
        ring = ring_from_oracle(ring_o)
        for step in range(6):
            x = synth.gaussian(shape, [1.0, 20.0, 0.05][step % 3], dtype, 5, step, O.DTYPES.index(dtype))
            ref = O.quantize(x, dtype, fmt, ring=ring_o)
            xd = to_device(x, dtype)
            si, am = scalar(0), scalar(0)
            if layout == "dual":
                r, t = fp8mi.fp8_quantize_dual(xd, fid, ring=ring, scale_inv_out=si, amax_out=am)
                got, want = [np_codes(r), np_codes(t)], [ref["codes"], ref["codes_t"]]
            else:
                o = fp8mi.fp8_quantize(xd, fid, layout == "t", ring=ring, scale_inv_out=si, amax_out=am)
                got, want = [np_codes(o)], [ref["codes_t"] if layout == "t" else ref["codes"]]
            torch.cuda.synchronize()
            tag = f"{layout} step {step}"
            for g, w in zip(got, want):
                assert np.array_equal(g, w), tag
            assert f32_bits(si) == as_bits(ref["scale_inv"]), tag
            assert f32_bits(am) == as_bits(ref["amax"]), tag
            assert np.array_equal(ring_state_words(ring), ref["ring"].words()), tag
            ring_o = ref["ring"]

@pytest.mark.parametrize("fmt,fid", FMTS)
def test_in_kernel_fold_equals_standalone_fold(fmt, fid):
    """The quantize kernel's last-block fold and fp8_amax_fold of the same
    amax leave byte-identical rings."""
    for H in (1, 4, 16, 1000):
        r0 = O.Ring(synth.gaussian_f32((H,), 2.0, 5, H).__abs__(), np.float32(3.0), H // 3)
        ring_a, ring_b = ring_from_oracle(r0), ring_from_oracle(r0)
        x = synth.gaussian((512, 384), 7.0, "f32", 5, H, 1)
        am = scalar(0)
        fp8mi.fp8_quantize(to_device(x, "f32"), fid, False, ring=ring_a, amax_out=am)
        fp8mi.fp8_amax_fold(ring_b, am, fid)
        torch.cuda.synchronize()
        assert np.array_equal(ring_a.cpu().numpy(), ring_b.cpu().numpy()), H
        assert np.array_equal(ring_state_words(ring_a), O.fold(r0, O.amax(x), fmt).words())


def test_fold_special_cases():
    """Zero window -> 1.0, inf amax -> 1.0, tiny amax (quotient overflows) -> 1.0."""
    for amax_v, want in ((0.0, 1.0), (np.inf, 1.0), (1e-45, 1.0), (2.0, 224.0)):
        r0 = O.Ring.new(3, 5.0)
        ring = ring_from_oracle(r0)
        fp8mi.fp8_amax_fold(ring, scalar(amax_v), 0)
        ref = O.fold(r0, np.float32(amax_v), O.E4M3)
        torch.cuda.synchronize()
        assert ring_to_oracle(ring).scale == ref.scale == np.float32(want)
        assert np.array_equal(ring_state_words(ring), ref.words())


def test_empty_and_degenerate_shapes():
    ring = ring_from_oracle(O.Ring(np.array([4.0, 0.0], np.float32), np.float32(9.0), 1))
    x = torch.empty((0, 7), dtype=torch.bfloat16, device=DEV)
    am, si = scalar(-1), scalar(-1)
    fp8mi.fp8_quantize(x, 0, False, ring=ring, amax_out=am, scale_inv_out=si)
    ref = O.fold(O.Ring(np.array([4.0, 0.0], np.float32), np.float32(9.0), 1), np.float32(0), O.E4M3)
    torch.cuda.synchronize()
    assert np.array_equal(ring_state_words(ring), ref.words())
    assert float(am) == 0.0 and f32_bits(si) == as_bits(np.float32(1) / np.float32(9))
    o = fp8mi.fp8_quantize(torch.empty((5, 0), dtype=torch.float32, device=DEV), 1, True, scale=scalar(1.0))
    assert o.shape == (0, 5)


# bf16 inputs are stored as uint16 bit patterns: plant specials by their bits
_SPECIAL_BF16 = {"nan": 0x7FC0, "-nan": 0xFFC0, "inf": 0x7F80, "-inf": 0xFF80}
_SPECIAL_FLOAT = {"nan": np.nan, "-nan": -np.nan, "inf": np.inf, "-inf": -np.inf}


def special(x, dtype, i, j, kind):
    x[i, j] = _SPECIAL_BF16[kind] if dtype == "bf16" else _SPECIAL_FLOAT[kind]


@pytest.mark.parametrize("dtype", O.DTYPES)
@pytest.mark.parametrize("shape", [(512, 1024), (256, 256), (300, 200)], ids=lambda s: f"{s[0]}x{s[1]}")
def test_ring_sequence_with_nan_and_inf(shape, dtype):
    """Ring mode with NaN and infinities planted in different workgroups'
    shares (the one-shot row kernel, the aligned and general tiled forms,
    each publishing its amax before storing): NaN never reaches amax, an
    infinite amax folds into the window, codes and ring words bit-exact."""
    fmt, fid = FMTS[1]
    rows, cols = shape
    for layout in ("row", "t", "dual"):
        ring_o = O.Ring.new(3, 2.0)
        ring = ring_from_oracle(ring_o)
        for step in range(4):
            x = synth.gaussian(shape, 1.0, dtype, 8, step, O.DTYPES.index(dtype))
            special(x, dtype, (7 * step + 1) % rows, (13 * step + 5) % cols, "nan")
            special(x, dtype, rows - 1 - step, step, "-nan")
            if step in (1, 2):
                special(x, dtype, rows // 2, cols // 3 + step, "inf" if step == 1 else "-inf")
            ref = O.quantize(x, dtype, fmt, ring=ring_o)
            xd = to_device(x, dtype)
            si, am = scalar(0), scalar(0)
            if layout == "dual":
                r, t = fp8mi.fp8_quantize_dual(xd, fid, ring=ring, scale_inv_out=si, amax_out=am)
                got, want = [np_codes(r), np_codes(t)], [ref["codes"], ref["codes_t"]]
            else:
                o = fp8mi.fp8_quantize(xd, fid, layout == "t", ring=ring, scale_inv_out=si, amax_out=am)
                got, want = [np_codes(o)], [ref["codes_t"] if layout == "t" else ref["codes"]]
            torch.cuda.synchronize()
            tag = f"{layout} step {step}"
            for g, w in zip(got, want):
                assert np.array_equal(g, w), tag
            assert f32_bits(si) == as_bits(ref["scale_inv"]), tag
            assert f32_bits(am) == as_bits(ref["amax"]), tag
            assert np.array_equal(ring_state_words(ring), ref["ring"].words()), tag
            ring_o = ref["ring"]


@pytest.mark.parametrize("out_case", ["row_misaligned", "t_padded", "t_misaligned"])
def test_whole_tiles_with_unaligned_outputs(out_case):
    """Whole 128 x 64 tiles and an aligned input, but an output whose base or
    row pitch is not aligned: the one-shot kernel must take its general form
    (the aligned form stores 8 / 16 bytes at a time) and still give the
    oracle's bytes with the padding untouched, explicit scale and ring."""
    rows, cols = 256, 128
    x = synth.gaussian((rows, cols), 1.0, "bf16", 10, ["row_misaligned", "t_padded", "t_misaligned"].index(out_case))
    xd = to_device(x, "bf16")
    fmt, fid = FMTS[0]
    o_row = codes_out(rows, cols, cols, 3 if out_case == "row_misaligned" else 0)
    o_t = codes_out(cols, rows, rows + (8 if out_case == "t_padded" else 0), 5 if out_case == "t_misaligned" else 0)
    ring_o = O.Ring.new(4, 7.0)
    ring = ring_from_oracle(ring_o)
    ref = O.quantize(x, "bf16", fmt, ring=ring_o)
    fp8mi.fp8_quantize_dual(xd, fid, out_row=o_row, out_t=o_t, ring=ring)
    torch.cuda.synchronize()
    assert np.array_equal(np_codes(o_row), ref["codes"])
    assert np.array_equal(np_codes(o_t), ref["codes_t"])
    assert padding_untouched(o_row) and padding_untouched(o_t)
    assert np.array_equal(ring_state_words(ring), ref["ring"].words())
    o_t2 = codes_out(cols, rows, rows + (8 if out_case == "t_padded" else 0), 5 if out_case == "t_misaligned" else 0)
    s = np.float32(3.5)
    fp8mi.fp8_quantize(xd, fid, True, out=o_t2, scale=scalar(s))
    torch.cuda.synchronize()
    assert np.array_equal(np_codes(o_t2), O.quantize(x, "bf16", fmt, scale=s)["codes_t"])
    assert padding_untouched(o_t2)


def test_amax_ignores_scale_and_nan():
    """amax comes from the raw values: a huge scale that saturates every code
    leaves amax unchanged; NaN inputs do not reach it."""
    x = synth.gaussian((100, 100), 2.0, "f32", 6, 1)
    x[3, 3] = np.nan
    xd = to_device(x, "f32")
    a1, a2 = scalar(0), scalar(0)
    fp8mi.fp8_quantize(xd, 0, False, scale=scalar(1.0), amax_out=a1)
    o = fp8mi.fp8_quantize(xd, 0, False, scale=scalar(1e6), amax_out=a2)
    ref = O.quantize(x, "f32", O.E4M3, scale=1e6)
    assert f32_bits(a1) == f32_bits(a2) == as_bits(O.amax(x))
    assert np.array_equal(np_codes(o), ref["codes"])
    assert np_codes(o)[3, 3] == 0x7F or np_codes(o)[3, 3] == 0xFF


def test_repeat_launch_determinism():
    x = synth.gaussian((1024, 1536), 1.0, "bf16", 7, 1)
    xd = to_device(x, "bf16")
    ring = fp8mi.new_ring(4, 100.0, DEV)
    outs = set()
    for _ in range(50):
        r = ring.clone()
        a, b = fp8mi.fp8_quantize_dual(xd, 0, ring=r)
        outs.add((a.cpu().numpy().tobytes().__hash__(), b.cpu().numpy().tobytes().__hash__(),
                  r.cpu().numpy().tobytes()))
    assert len(outs) == 1
