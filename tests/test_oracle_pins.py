"""Pins for the CPU oracle against things other than itself: the library fp8
and bf16 casts of torch, brute force with exact rationals, closed forms that
reduce to integer arithmetic, hand-derived worked examples (tests/golden) and
invariants.  A plausible slip in the oracle (a dropped term, a wrong tie rule,
a transposed operand, an off-by-one in the ring index) fails one of these.
"""
import math
import os
import struct
from bisect import bisect_left
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle as O
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
TORCH_FP8 = {O.E4M3: torch.float8_e4m3fn, O.E5M2: torch.float8_e5m2}


def torch_decode(fmt):
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    return codes.view(TORCH_FP8[fmt]).to(torch.float64).numpy()


def f32_bits(x):
    return struct.unpack("<I", struct.pack("<f", x))[0]


# ---------------------------------------------------------------- decode ----
@pytest.mark.parametrize("fmt", O.FORMATS)
def test_decode_matches_torch_on_all_codes(fmt):
    mine, ref = O.decode_table(fmt), torch_decode(fmt)
    assert np.array_equal(np.isnan(mine), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(mine[ok], ref[ok])
    # signed zeros too
    assert np.array_equal(np.signbit(mine[ok]), np.signbit(ref[ok]))


@pytest.mark.parametrize("fmt,nfinite,vmax,vsub,vnorm", [
    (O.E4M3, 254, 448.0, 2.0 ** -9, 2.0 ** -6),
    (O.E5M2, 248, 57344.0, 2.0 ** -16, 2.0 ** -14),
])
def test_decode_invariants(fmt, nfinite, vmax, vsub, vnorm):
    t = O.decode_table(fmt)
    fin = np.isfinite(t)
    assert fin.sum() == nfinite
    assert np.nanmax(t[fin]) == vmax == O.FMT_MAX[fmt]
    pos = t[1:0x80][np.isfinite(t[1:0x80])]
    assert pos.min() == vsub
    assert np.all(np.diff(pos) > 0), "positive codes increase with the code"
    assert vnorm in pos and (pos < vnorm).sum() == (7 if fmt == O.E4M3 else 3)
    for c in range(0x80):  # sign symmetry
        a, b = t[c], t[c | 0x80]
        assert (np.isnan(a) and np.isnan(b)) or a == -b


# ---------------------------------------------------------------- encode ----
def _exact_grid(fmt):
    vals = []
    for c in range(0x80):
        v = torch_decode(fmt)[c]
        if np.isfinite(v):
            vals.append((Fraction(float(v)), c))
    return vals


def brute_encode(v: float, fmt: str) -> int:
    """Nearest finite value by exhaustive exact comparison; ties to the even
    code; saturation at fmt_max; NaN code with the input's sign."""
    sign = 0x80 if math.copysign(1.0, v) < 0 else 0
    if math.isnan(v):
        return 0x7F | sign
    a = abs(v)
    if a >= O.FMT_MAX[fmt]:
        best = max(_exact_grid(fmt))[1]
        return best | sign
    fa = Fraction(a)
    best, best_d = None, None
    for val, c in _exact_grid(fmt):
        d = abs(val - fa)
        if best_d is None or d < best_d or (d == best_d and c % 2 == 0):
            best, best_d = c, d
    return best | sign


def _edge_values(fmt):
    """fp32 values on and next to every midpoint between neighbouring codes,
    plus the saturation boundary."""
    t = torch_decode(fmt)
    pos = sorted(set(float(v) for v in t[:0x80] if np.isfinite(v)))
    out = []
    for lo, hi in zip(pos, pos[1:]):
        m = np.float32((lo + hi) / 2)  # exact: midpoints need few bits
        for d in (-1, 0, 1):
            out.append(float(np.float32(np.nextafter(m, np.float32(np.inf if d > 0 else -np.inf)))
                             if d else m))
    out += [O.FMT_MAX[fmt], float(np.nextafter(np.float32(O.FMT_MAX[fmt]), np.float32(np.inf))),
            1e-45, 1e-40, 3.4e38]
    return out + [-v for v in out]


@pytest.mark.parametrize("fmt", O.FORMATS)
def test_encode_brute_force_edges(fmt):
    vals = _edge_values(fmt)
    got = O.encode(np.array(vals, dtype=np.float32), fmt)
    exp = [brute_encode(float(np.float32(v)), fmt) for v in vals]
    assert list(got) == exp


@pytest.mark.parametrize("fmt", O.FORMATS)
def test_encode_brute_force_random(fmt):
    g = synth.rng(99, 1 if fmt == O.E4M3 else 2)
    # log-uniform magnitudes across and beyond the format's range, both signs
    lo, hi = (-12, 10) if fmt == O.E4M3 else (-19, 17)
    v = (2.0 ** g.uniform(lo, hi, size=600)) * g.choice([-1.0, 1.0], size=600)
    v = v.astype(np.float32)
    got = O.encode(v, fmt)
    exp = [brute_encode(float(x), fmt) for x in v]
    assert list(got) == exp


def _all_bf16_and_f16():
    b = (np.arange(65536, dtype=np.uint32) << 16).view(np.float32)
    h = np.arange(65536, dtype=np.uint16).view(np.float16).astype(np.float32)
    return np.concatenate([b, h])


@pytest.mark.parametrize("fmt", O.FORMATS)
def test_encode_matches_torch_exhaustive_bf16_f16(fmt):
    """Every bf16 and every fp16 bit pattern: equal to torch's RNE cast where
    torch does not overflow; saturated above."""
    v = _all_bf16_and_f16()
    got = O.encode(v, fmt)
    lim = 464.0 if fmt == O.E4M3 else 61440.0
    fin = np.isfinite(v)
    inrange = fin & (np.abs(v) < lim) | (fin & (np.abs(v) == 464.0) & (fmt == O.E4M3))
    ref = torch.from_numpy(v[inrange]).to(TORCH_FP8[fmt]).view(torch.uint8).numpy()
    assert np.array_equal(got[inrange], ref)
    big = fin & ~inrange
    max_code = 0x7E if fmt == O.E4M3 else 0x7B
    assert np.all((got[big] & 0x7F) == max_code)
    assert np.array_equal(got[big] >> 7, np.signbit(v[big]).astype(np.uint8))
    nan = np.isnan(v)
    assert np.all((got[nan] & 0x7F) == 0x7F)


@pytest.mark.parametrize("fmt", O.FORMATS)
def test_encode_roundtrip_every_code(fmt):
    t = O.decode_table(fmt)
    codes = np.array([c for c in range(256) if np.isfinite(t[c])], dtype=np.uint8)
    back = O.encode(t[codes].astype(np.float32), fmt)
    assert np.array_equal(back, codes)


@pytest.mark.parametrize("fmt", O.FORMATS)
def test_encode_error_at_most_half_spacing(fmt):
    v = synth.gaussian_f32((5000,), 8.0, 5, 5)
    t = O.decode_table(fmt)
    q = t[O.encode(v, fmt)]
    grid = np.sort(np.unique(np.abs(t[np.isfinite(t)])))
    for x, y in zip(v, q):
        i = bisect_left(grid, abs(x))
        if i == 0 or i >= len(grid):
            continue
        assert abs(abs(y) - abs(x)) <= (grid[i] - grid[i - 1]) / 2


def test_encode_golden_worked_values():
    n = 0
    for line in open(os.path.join(GOLDEN, "encode_worked.txt")):
        line = line.split("#")[0].strip()
        if not line:
            continue
        fmt, val, code = line.split()
        v = float(val)
        got = int(O.encode(np.array([v], dtype=np.float32), fmt)[0])
        assert got == int(code, 16), (fmt, val, hex(got), code)
        n += 1
    assert n >= 30


# ------------------------------------------------------ scaled multiply ----
def test_scaled_values_single_rounding():
    """fl32(x*s): float64 holds the exact product of two fp32 values, and one
    cast to fp32 rounds it once -- including into the subnormal range."""
    x = synth.random_bits_f32(20000, 7, 1)
    s = synth.random_bits_f32(20000, 7, 2)
    ok = np.isfinite(x) & np.isfinite(s)
    x, s = x[ok], s[ok]
    with np.errstate(over="ignore", under="ignore", invalid="ignore"):
        exact = (x.astype(np.float64) * s.astype(np.float64)).astype(np.float32)
        got = np.array([O.scaled_values(np.array([a]), b)[0] for a, b in zip(x[:3000], s[:3000])])
    assert np.array_equal(got.view(np.uint32), exact[:3000].view(np.uint32))


# ------------------------------------------------------------------ amax ----
def test_amax_raw_values_and_scale_independence():
    x = synth.gaussian((64, 33), 1.0, "f32", 3, 3)
    xs = list(map(float, x.ravel()))
    assert O.amax(x) == np.float32(max(abs(v) for v in xs))
    # amax is taken before scaling: the scale never reaches it
    r1 = O.quantize(x, O.F32, O.E4M3, scale=1.0)
    r2 = O.quantize(x, O.F32, O.E4M3, scale=1000.0)
    assert r1["amax"] == r2["amax"] == O.amax(x)
    assert O.amax(np.array([np.nan, -3.0, 2.0], np.float32)) == 3.0
    assert O.amax(np.zeros((0, 5), np.float32)) == 0.0
    assert O.amax(np.array([-0.0], np.float32)) == 0.0


@pytest.mark.parametrize("dtype", O.DTYPES)
def test_widen_exact(dtype):
    x = synth.gaussian((257,), 3.0, dtype, 4, 4)
    if dtype == "bf16":
        ref = synth.to_torch(x, "bf16").to(torch.float32).numpy()
    else:
        ref = torch.from_numpy(x).to(torch.float32).numpy()
    assert np.array_equal(O.widen_to_f32(x, dtype), ref)


# ------------------------------------------------------------------ fold ----
def test_fold_golden_sequences():
    rings = {}
    n = 0
    for line in open(os.path.join(GOLDEN, "fold_worked.txt")):
        line = line.split("#")[0].strip()
        if not line:
            continue
        case, fmt, h, a, s, idx, window = line.split()
        if case not in rings:
            rings[case] = O.Ring.new(int(h), 1.0)
        rings[case] = O.fold(rings[case], float(a), fmt)
        assert rings[case].scale == np.float32(float(s)), (case, a)
        assert rings[case].idx == int(idx)
        assert rings[case].hist.tolist() == [float(w) for w in window.split(",")]
        n += 1
    assert n == 11


def test_fold_window_is_last_H_amaxes():
    """After any sequence, the window holds exactly the last H amax values
    (in slot order) and the scale is fmt_max over their maximum."""
    g = synth.rng(11)
    for H in (1, 3, 16):
        r = O.Ring.new(H, 1.0)
        seq = []
        for _ in range(40):
            a = np.float32(g.exponential(2.0))
            seq.append(a)
            r = O.fold(r, a, O.E4M3)
            last = seq[-H:]
            window = sorted(map(float, r.hist))
            expect = sorted(map(float, last + [np.float32(0)] * (H - len(last))))
            assert window == expect
            assert r.idx == len(seq) % H
            m = Fraction(float(max(last)))
            want = np.float32(float(Fraction(448) / m))  # fp32 nearest of the exact quotient
            assert r.scale == want


def test_ring_words_roundtrip():
    r = O.Ring(np.array([1.5, 0, 3], np.float32), np.float32(7.0), 2)
    w = r.words()
    assert len(w) == 7 and w[5] == 0 and w[6] == 0 and w[4] == 2
    r2 = O.Ring.from_words(w)
    assert np.array_equal(r2.hist, r.hist) and r2.scale == 7.0 and r2.idx == 2


# ------------------------------------------------------- bf16 rounding ----
_BF16_POS = None


def _bf16_positive_values():
    global _BF16_POS
    if _BF16_POS is None:
        bits = np.arange(0, 0x7F80, dtype=np.uint32) << 16
        _BF16_POS = [float(v) for v in bits.view(np.float32)]
    return _BF16_POS


def brute_bf16(y: float) -> int:
    """bf16 bits of y by exact comparison with its two neighbours (ties to
    the even pattern); beyond the largest value, RNE against 2^128 -> inf."""
    sign = 0x8000 if math.copysign(1.0, y) < 0 else 0
    a = abs(y)
    pos = _bf16_positive_values()
    top = Fraction(2) ** 128
    if Fraction(a) >= (Fraction(pos[-1]) + top) / 2:
        return 0x7F80 | sign
    i = bisect_left(pos, a)
    if i < len(pos) and pos[i] == a:
        return i | sign
    lo, hi = i - 1, min(i, len(pos) - 1)
    dl, dh = Fraction(a) - Fraction(pos[lo]), Fraction(pos[hi]) - Fraction(a)
    pick = hi if (dh < dl or (dh == dl and hi % 2 == 0)) else lo
    return pick | sign


def test_bf16_rounding_brute_force():
    g = synth.rng(12)
    ys = list((2.0 ** g.uniform(-140, 129, 400)) * g.choice([-1, 1], 400))
    pos = _bf16_positive_values()
    for k in g.integers(1, len(pos) - 1, 200):  # exact midpoints and neighbours
        m = (pos[k] + pos[k + 1]) / 2
        ys += [m, -m, np.nextafter(m, 0.0), np.nextafter(m, np.inf)]
    ys += [0.0, -0.0, 2.0 ** -134, 2.0 ** -133 * 1.5, 2.0 ** 128 - 2.0 ** 119,
           2.0 ** 128 - 2.0 ** 119 - 1e20]
    got = O.bf16_bits_from_f64(np.array(ys))
    assert [int(x) for x in got] == [brute_bf16(float(y)) for y in ys]


def test_bf16_rounding_matches_torch_on_fp32_values():
    v = synth.random_bits_f32(200000, 13)
    v = v[np.isfinite(v)]
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(O.bf16_bits_from_f64(v.astype(np.float64)), ref)


def test_ulp_bf16_is_spacing_to_next_value():
    bits = synth.rng(14).integers(0x0001, 0x7F7F, 5000).astype(np.uint16)
    v = O.bf16_bits_to_f64(bits)
    nxt = O.bf16_bits_to_f64(bits + 1)
    assert np.array_equal(O.ulp_bf16(v), nxt - v)
    assert O.ulp_bf16(np.array([0.0]))[0] == 2.0 ** -133


# ------------------------------------------------------------------ GEMM ----
def _codes(shape, fmt, key):
    """Random finite codes (quantised N(0,1) data at scale fmt_max/amax)."""
    x = synth.gaussian_f32(shape, 1.0, *key)
    s = np.float32(O.FMT_MAX[fmt]) / np.float32(np.abs(x).max())
    return O.encode(x * s, fmt)


def _int_values(codes, fmt):
    """Integer numerators of the code values: E4M3 codes are multiples of
    2^-9, E5M2 codes multiples of 2^-16 (from torch's decode)."""
    shift = 9 if fmt == O.E4M3 else 16
    v = torch_decode(fmt)[codes] * 2.0 ** shift
    assert np.all(v == np.round(v))
    return v.astype(np.int64), shift


def test_gemm_e4m3_exact_against_integer_gemm():
    a = _codes((2, 37, 300), O.E4M3, (15, 1))
    b = _codes((2, 29, 300), O.E4M3, (15, 2))
    y, _ = O.mm_exact_f64(a, O.E4M3, b, O.E4M3)
    ia, sa = _int_values(a, O.E4M3)
    ib, sb = _int_values(b, O.E4M3)
    ref = np.matmul(ia, np.swapaxes(ib, 1, 2))            # int64, exact
    assert np.array_equal(y * 2.0 ** (sa + sb), ref.astype(np.float64))
    assert np.array_equal((y * 2.0 ** (sa + sb)).astype(np.int64), ref)


def test_gemm_mixed_formats_close_to_exact_rational():
    a = _codes((9, 64), O.E5M2, (16, 1))
    b = _codes((7, 64), O.E4M3, (16, 2))
    y, mag = O.mm_exact_f64(a, O.E5M2, b, O.E4M3, 0.5, 3.0)
    ia, sa = _int_values(a, O.E5M2)
    ib, sb = _int_values(b, O.E4M3)
    for i in range(9):
        for j in range(7):
            exact = Fraction(sum(int(p) * int(q) for p, q in zip(ia[i], ib[j])), 2 ** (sa + sb)) \
                * Fraction(1, 2) * 3
            assert abs(Fraction(float(y[0, i, j])) - exact) <= Fraction(float(mag[0, i, j])) * Fraction(1, 2 ** 45)


def test_gemm_bias_rounded_once_from_f64():
    """A single rounding: an exact sum that sits just above a bf16 midpoint
    must round up, which a detour through fp32 would lose."""
    # A = [1.0], B = [1.0] -> acc = 1.0; bias puts the sum 2^-20 above the
    # midpoint 1 + 2^-8 between bf16 values 1 and 1 + 2^-7.
    a = np.array([[0x38]], np.uint8)
    b = np.array([[0x38]], np.uint8)
    bias = np.array([2.0 ** -8 + 2.0 ** -40])
    bits, _ = O.mm(a, O.E4M3, b, O.E4M3, 1.0, 1.0, bias)
    assert O.bf16_bits_to_f64(bits)[0, 0, 0] == 1.0 + 2.0 ** -7


def test_gemm_identity_and_zero_special_cases():
    K = 64
    eye = np.zeros((K, K), np.uint8)
    np.fill_diagonal(eye, 0x38)                   # 1.0 on the diagonal
    b = _codes((48, K), O.E4M3, (17, 1))
    bias_bits = synth.gaussian((K,), 0.1, "bf16", 17, 2)
    bias = O.widen_to_f32(bias_bits, "bf16").astype(np.float64)
    # C = A B^T with A = I gives C[i,j] = B[j,i]
    bits, _ = O.mm(eye, O.E4M3, b, O.E4M3, 1.0, 1.0)
    bv = torch_decode(O.E4M3)[b]
    ref = torch.from_numpy(bv.T.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(bits[0], ref)
    # A = 0 gives bf16(bias) in every row
    zero = np.zeros((5, K), np.uint8)
    bits, _ = O.mm(zero, O.E4M3, b, O.E4M3, 2.0, 3.0, bias[:48])
    assert np.all(bits[0] == bias_bits[:48][None, :])


def test_gemm_k1_closed_form():
    a = _codes((6, 1), O.E4M3, (18, 1))
    b = _codes((5, 1), O.E5M2, (18, 2))
    y, _ = O.mm_exact_f64(a, O.E4M3, b, O.E5M2, 0.25, 8.0)
    ta, tb = torch_decode(O.E4M3), torch_decode(O.E5M2)
    for i in range(6):
        for j in range(5):
            assert y[0, i, j] == ta[a[i, 0]] * tb[b[j, 0]] * 2.0


def test_gemm_operand_orientation():
    """NT: C[i,j] pairs row i of A with row j of B (not column j)."""
    a = np.array([[0x38, 0x00], [0x00, 0x38]], np.uint8)      # I
    b = np.array([[0x40, 0x48], [0x50, 0x58]], np.uint8)      # [[2,4],[8,16]]
    y, _ = O.mm_exact_f64(a, O.E4M3, b, O.E4M3)
    assert y[0].tolist() == [[2.0, 8.0], [4.0, 16.0]]


def test_tolerance_bound_form():
    ref = O.bf16_bits_from_f64(np.array([1.0, 1.0, 1.0]))
    gpu = O.bf16_bits_from_f64(np.array([1.0 + 2.0 ** -7, 1.0 + 2.0 ** -6, 1.0 + 2.0 ** -6]))
    ok = O.within_tolerance(gpu, ref, np.array([0.0, 0.0, 2.0 ** -6 / 1e-5]))
    assert ok.tolist() == [True, False, True]


def test_grad_bias_exact_small():
    dy = synth.gaussian((3, 5, 7), 1e-3, "bf16", 19, 1)
    bits, _ = O.grad_bias(dy)
    v = [Fraction(float(x)) for x in O.widen_to_f32(dy, "bf16").reshape(-1)]
    for j in range(7):
        s = sum(v[i * 7 + j] for i in range(15))
        assert Fraction(float(s)) == s            # the float64 sum is exact here
        assert int(bits[j]) == brute_bf16(float(s))


# ------------------------------------------------------ the linear step ----
def test_linear_forward_recovers_exact_inputs():
    """Integers in [-2,2] through delayed-scaled E4M3 (scale 448/2) and an
    identity weight come back exactly, plus a bias that is exact in bf16."""
    x = synth.rng(20).integers(-2, 3, size=(8, 16)).astype(np.float32)
    x[0, 0] = 2.0
    xb = synth.f32_to_bf16_bits(x)
    w = np.eye(16, dtype=np.float32)
    wb = synth.f32_to_bf16_bits(w)
    bias = np.full(16, 0.5, np.float32)
    rx = O.seed_ring(4, xb, "bf16", O.E4M3)
    rw = O.seed_ring(4, wb, "bf16", O.E4M3)
    assert rx.scale == 224.0 and rw.scale == 448.0
    out = O.linear_forward(xb, wb, synth.f32_to_bf16_bits(bias), rx, rw)
    assert np.array_equal(O.bf16_bits_to_f64(out["y"][None])[0], (x + 0.5).astype(np.float64))
    # the fold republished the seeded scale: amax unchanged
    assert out["qx"]["ring"].scale == 224.0 and out["qx"]["ring"].idx == 1


def test_linear_backward_shapes_and_transposes():
    g = synth.rng(21)
    x = synth.gaussian((8, 16), 1.0, "bf16", 21, 1)
    w = synth.gaussian((12, 16), 0.02, "bf16", 21, 2)
    dy = synth.gaussian((8, 12), 1e-3, "bf16", 21, 3)
    rx, rw = O.seed_ring(2, x, "bf16", O.E4M3), O.seed_ring(2, w, "bf16", O.E4M3)
    fwd = O.linear_forward(x, w, None, rx, rw)
    rg = O.seed_ring(2, dy, "bf16", O.E5M2)
    bwd = O.linear_backward(dy, fwd["qx"], fwd["qw"], rg)
    assert bwd["dx"].shape == (8, 16) and bwd["dw"].shape == (12, 16) and bwd["db"].shape == (12,)
    # dX against the dequantised product computed directly
    tg, t4 = torch_decode(O.E5M2), torch_decode(O.E4M3)
    G = tg[bwd["qg"]["codes"]] * float(bwd["qg"]["scale_inv"])
    W = t4[fwd["qw"]["codes"]] * float(fwd["qw"]["scale_inv"])
    X = t4[fwd["qx"]["codes"]] * float(fwd["qx"]["scale_inv"])
    dx = O.bf16_bits_to_f64(bwd["dx"])
    dw = O.bf16_bits_to_f64(bwd["dw"])
    assert np.allclose(dx, G @ W, rtol=1e-2, atol=1e-9)
    assert np.allclose(dw, G.T @ X, rtol=1e-2, atol=1e-9)
    del g


# ------------------------------------------------------- current scaling ----
def _golden_input(vals, dtype):
    f = np.array(vals, dtype=np.float32)
    if dtype == O.BF16:
        bits = (f.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
        assert np.array_equal(O.widen_to_f32(bits, dtype).view(np.uint32), f.view(np.uint32)), "not exact in bf16"
        return bits
    if dtype == O.F16:
        h = f.astype(np.float16)
        assert np.array_equal(h.astype(np.float32), f), "not exact in fp16"
        return h
    return f


def test_dynamic_golden_worked():
    n = 0
    for line in open(os.path.join(GOLDEN, "dynamic_worked.txt")):
        line = line.split("#")[0].strip()
        if not line:
            continue
        case, fmt, dtype, vals, sinv, am, codes = line.split()
        x = _golden_input([float(v) for v in vals.split(",")], dtype)[None, :]
        r = O.quantize_dynamic(x, dtype, fmt)
        assert r["scale_inv"] == np.float32(float(sinv)), case
        assert r["amax"] == np.float32(float(am)), case
        assert r["codes"][0].tolist() == [int(c, 16) for c in codes.split(",")], case
        assert r["ring"] is None
        n += 1
    assert n == 8


@pytest.mark.parametrize("fmt,top", [(O.E4M3, 0x7E), (O.E5M2, 0x7B)])
@pytest.mark.parametrize("dtype", O.DTYPES)
def test_dynamic_scale_is_nearest_quotient_and_hits_format_max(fmt, top, dtype):
    """The scale is the fp32 nearest of the exact quotient fmt_max / amax(x)
    (checked with exact fractions), scale_inv its fp32 reciprocal, and the
    element(s) of largest magnitude land on the format's largest code while
    no code exceeds it."""
    for seed, sigma in ((1, 1.0), (2, 3e-3), (3, 7e2)):
        x = synth.gaussian((37, 29), sigma, dtype, 90, seed)
        xf = O.widen_to_f32(x, dtype)
        a = float(np.max(np.abs(xf)))
        r = O.quantize_dynamic(x, dtype, fmt)
        s = np.float32(float(Fraction(O.FMT_MAX[fmt]) / Fraction(a)))
        assert r["amax"] == np.float32(a)
        assert r["scale_inv"] == np.float32(float(Fraction(1) / Fraction(float(s))))
        mag = r["codes"] & 0x7F
        assert mag.max() == top
        assert np.all(mag[np.abs(xf) == np.float32(a)] == top)
        # the scaled tensor spans the format: the scale is not the reciprocal
        # of the quotient, nor measured from anything but this tensor
        assert np.array_equal(r["codes"], O.quantize(x, dtype, fmt, scale=s)["codes"])


def test_dynamic_depends_on_this_tensor_only():
    """Two tensors that differ by a power-of-two factor get the same codes;
    a tensor with one element raised gets a smaller scale for all the rest."""
    x = synth.gaussian((16, 24), 1.0, O.F32, 91, 0)
    r1 = O.quantize_dynamic(x, O.F32, O.E4M3)
    r2 = O.quantize_dynamic(x * np.float32(2.0 ** -20), O.F32, O.E4M3)
    assert np.array_equal(r1["codes"], r2["codes"])
    assert r2["scale_inv"] == r1["scale_inv"] * np.float32(2.0 ** -20)
    y = x.copy()
    y[3, 5] = np.float32(4 * np.max(np.abs(x)))
    r3 = O.quantize_dynamic(y, O.F32, O.E4M3)
    assert r3["scale_inv"] > r1["scale_inv"]
    assert r3["codes"][3, 5] == 0x7E


def test_dynamic_equals_delayed_with_a_ring_seeded_from_the_same_tensor():
    for dtype in O.DTYPES:
        x = synth.gaussian((19, 40), 0.5, dtype, 92, 1)
        r = O.quantize_dynamic(x, dtype, O.E5M2)
        d = O.quantize(x, dtype, O.E5M2, ring=O.seed_ring(4, x, dtype, O.E5M2))
        assert np.array_equal(r["codes"], d["codes"])
        assert r["scale_inv"] == d["scale_inv"] and r["amax"] == d["amax"]


# --------------------------------------------- fp8 bias, FP8-out GEMM ----
@pytest.mark.parametrize("fmt", O.FORMATS)
def test_dequant_bias_matches_torch_widen_times_scale(fmt):
    """fl32(dec(code) * s) for every code and several scales, against torch's
    own fp8 -> fp32 cast followed by an fp32 multiply."""
    codes = np.arange(256, dtype=np.uint8)
    ref_dec = torch.from_numpy(codes).view(TORCH_FP8[fmt]).to(torch.float32)
    for s in (1.0, 0.5, 3.0e-3, 771.25):
        got = O.dequant_bias(codes, fmt, s)
        ref = (ref_dec * torch.tensor(np.float32(s))).numpy()
        assert np.array_equal(got.view(np.uint32)[~np.isnan(ref)], ref.view(np.uint32)[~np.isnan(ref)])
        assert np.array_equal(np.isnan(got), np.isnan(ref))


def _mm_golden_rows():
    for line in open(os.path.join(GOLDEN, "mm_fp8_out_worked.txt")):
        line = line.split("#")[0].strip()
        if line:
            yield line.split()


def _mm_golden_case(f):
    case, fmt_c, bcodes, sa, sb, bias, scale = f[:7]
    a = np.array([[0x38, 0x40]], np.uint8)
    b = np.array([[int(c, 16) for c in row.split(",")] for row in bcodes.split(";")], np.uint8)
    bias_v = None
    if bias.startswith("f32:"):
        bias_v = np.array([float(v) for v in bias[4:].split(",")], np.float32).astype(np.float64)
    elif bias.startswith("e4m3:"):
        codes, bs = bias[5:].split("@")
        bias_v = O.dequant_bias(np.array([int(c, 16) for c in codes.split(",")], np.uint8), O.E4M3,
                                float(bs)).astype(np.float64)
    kind, val = scale.split(":")
    kw = {"scale": float(val)} if kind == "explicit" else {"ring": O.Ring.new(2, float(val))}
    return case, a, b, float(sa), float(sb), bias_v, fmt_c, kw


def test_mm_quantized_golden_worked():
    n = 0
    for f in _mm_golden_rows():
        case, a, b, sa, sb, bias_v, fmt_c, kw = _mm_golden_case(f)
        codes, amax, sinv, ring_after = f[7:11]
        r = O.mm_quantized(a, O.E4M3, b, O.E4M3, fmt_c, sa, sb, bias_v, **kw)
        assert r["codes"][0, 0].tolist() == [int(c, 16) for c in codes.split(",")], case
        assert r["amax"] == np.float32(float(amax)), case
        assert r["scale_inv"] == np.float32(float(sinv)), case
        if ring_after != "-":
            sc, idx, hist = ring_after.split(",")
            assert r["ring"].scale == np.float32(float(sc)) and r["ring"].idx == int(idx), case
            assert r["ring"].hist.tolist() == [float(h) for h in hist.split(":")], case
        else:
            assert r["ring"] is None
        n += 1
    assert n == 6


def test_mm_quantized_is_quantize_of_the_exact_gemm():
    """Small-integer codes make every y exact (the integer-GEMM pin); then the
    output codes must be a quantize of those exact values, batch and all."""
    g = synth.rng(93)
    vals = np.arange(-6, 7)
    enc = {v: int(O.encode(np.array([v], np.float32), O.E4M3)[0]) for v in vals}
    a = np.vectorize(enc.get)(g.choice(vals, (2, 9, 32))).astype(np.uint8)
    b = np.vectorize(enc.get)(g.choice(vals, (2, 7, 32))).astype(np.uint8)
    ia, ib = O.decode_table(O.E4M3)[a], O.decode_table(O.E4M3)[b]
    y = np.einsum("bik,bjk->bij", ia, ib) * 0.25 + np.arange(7)[None, None, :]
    ring = O.Ring.new(3, 2.0)
    r = O.mm_quantized(a, O.E4M3, b, O.E4M3, O.E5M2, 0.5, 0.5, np.arange(7, dtype=np.float64), ring=ring)
    q = O.quantize(y.reshape(-1, 7).astype(np.float32), O.F32, O.E5M2, ring=ring)
    assert np.array_equal(r["codes"].reshape(-1, 7), q["codes"])
    assert r["amax"] == np.float32(np.abs(y).max()) and r["ring"].words().tolist() == q["ring"].words().tolist()
