"""Plain CPU oracle for FP8 per-tensor scaled quantize, the delayed-scaling amax
history fold and the per-tensor-scaled fp8 GEMM with fused bias.

TEST INFRASTRUCTURE ONLY.  This module is the correctness authority that the
HIP library is checked against.  Only the test suite, the package smoke check
and the benchmark's CPU-baseline leg may import it; the product path never
calls it and shares no code, table or constant generator with it.

Everything here is deliberately slow and obvious: numpy + the Python standard
library, float64 wherever the method leaves the precision open, no blocking,
fusion or reordering beyond what each definition states.

Sources (the AstrAI commit-log pages; "log:<path>" below means the Gitea
commit history page of that path in the ViperEkura/AstrAI repository):

* log:tests/extension -- the commit that moves the amax/history update into the
  quantize kernel's last block; the commit that fuses the bias into the GEMM
  epilogue ahead of a single bf16 rounding; the commit adding batched (3-D)
  operands with stride-0 broadcast; the commit that snapshots the scales before
  the ring is finalised; the commit templating quantize on bf16/fp16/fp32 and
  asking for fp32-domain amax references.
* log:csrc/kernels/fp8/quantize.cuh -- the commit introducing the tiled
  transposed/dual quantize layouts.
* log:csrc/kernels/fp8_mm.cu -- commit 69f35c46e0 (amax must come from the
  raw input, not the scaled fp8 values; E4M3's largest value is 448) and
  commit 5244f1a8fc (TE-style delayed scaling with per-tensor A/B scales).

Readings taken where the pages are silent (all listed in the design notes):
scaled value = one fp32 multiply of the exactly widened input; encoding is
saturating round-to-nearest-even with ties to the even code; NaN keeps its
sign as S.1111.111 (E4M3) / S.11111.11 (E5M2 quiet NaN); +-inf saturate; amax
ignores NaN; next scale = fmt_max / max(history), or 1.0 whenever that
maximum is 0 or non-finite or the quotient is not a finite positive number.

Parity pins for every function live in tests/test_oracle_pins.py.
"""
from __future__ import annotations

import dataclasses
import numpy as np

E4M3 = "e4m3"
E5M2 = "e5m2"
FORMATS = (E4M3, E5M2)

# Largest finite magnitude of each format (log:fp8_mm.cu, commit 69f35c46e0,
# names ~448 for E4M3; OCP E5M2's is 57344).
FMT_MAX = {E4M3: 448.0, E5M2: 57344.0}

BF16, F16, F32 = "bf16", "f16", "f32"
DTYPES = (BF16, F16, F32)


# --------------------------------------------------------------------------
# O1: decode -- the 256 codes of each OCP fp8 format, closed form.
# --------------------------------------------------------------------------
def decode_code(code: int, fmt: str) -> float:
    """Value of one fp8 code (OCP FP8 formats E4M3FN and E5M2).

    E4M3: 1 sign, 4 exponent bits (bias 7), 3 mantissa bits; exponent 0 is
    subnormal; S.1111.111 is NaN; there is no infinity.
    E5M2: 1 sign, 5 exponent bits (bias 15), 2 mantissa bits; exponent 0 is
    subnormal; exponent 31 is inf (mantissa 0) or NaN.
    """
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    if fmt == E4M3:
        e, m = (code >> 3) & 0xF, code & 0x7
        if e == 0xF and m == 0x7:
            return float("nan")
        if e == 0:
            return sign * m * 2.0 ** -9          # m/8 * 2^(1-7)
        return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    if fmt == E5M2:
        e, m = (code >> 2) & 0x1F, code & 0x3
        if e == 0x1F:
            return sign * float("inf") if m == 0 else float("nan")
        if e == 0:
            return sign * m * 2.0 ** -16         # m/4 * 2^(1-15)
        return sign * (1.0 + m / 4.0) * 2.0 ** (e - 15)
    raise ValueError(f"unknown fp8 format {fmt!r}")


def decode_table(fmt: str) -> np.ndarray:
    """float64[256]: value of every code (NaN where the code is NaN)."""
    return np.array([decode_code(c, fmt) for c in range(256)], dtype=np.float64)


def _positive_grid(fmt: str):
    """Finite non-negative values of the format, ascending, with their codes."""
    tab = decode_table(fmt)
    codes = [c for c in range(0x80) if np.isfinite(tab[c])]
    vals = np.array([tab[c] for c in codes], dtype=np.float64)
    order = np.argsort(vals, kind="stable")
    return vals[order], np.array(codes, dtype=np.int64)[order]


# --------------------------------------------------------------------------
# Inputs: exact widening of bf16 / fp16 / fp32 storage to fp32
# (log:tests/extension, commit templating quantize on the three input types).
# --------------------------------------------------------------------------
def widen_to_f32(x: np.ndarray, dtype: str) -> np.ndarray:
    """Exact fp32 value of each stored element.

    bf16 is carried as its uint16 bit pattern (numpy has no bf16); its fp32
    value is those 16 bits in the top half of an fp32 word.
    """
    if dtype == BF16:
        bits = np.asarray(x, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return bits.view(np.float32)
    if dtype == F16:
        return np.asarray(x, dtype=np.float16).astype(np.float32)
    if dtype == F32:
        return np.asarray(x, dtype=np.float32)
    raise ValueError(f"unknown input dtype {dtype!r}")


# --------------------------------------------------------------------------
# O2: encode -- saturating round-to-nearest-even of an fp32 value.
# --------------------------------------------------------------------------
def encode(v: np.ndarray, fmt: str) -> np.ndarray:
    """fp8 code of each fp32 value: nearest finite value, ties to the even
    code, magnitudes at or above fmt_max (and +-inf) saturate to +-fmt_max,
    NaN -> the format's NaN code carrying the input's sign, sign of zero kept.
    """
    v = np.asarray(v, dtype=np.float32)
    grid, codes = _positive_grid(fmt)
    fmax = FMT_MAX[fmt]
    max_code = int(codes[-1])
    nan_code = 0x7F
    with np.errstate(invalid="ignore"):
        a = np.abs(v.astype(np.float64))
    sign = np.signbit(v).astype(np.uint8) << np.uint8(7)

    out = np.zeros(v.shape, dtype=np.uint8)
    nan = np.isnan(a)
    sat = ~nan & (a >= fmax)
    mid = ~nan & ~sat

    am = a[mid]
    hi = np.searchsorted(grid, am, side="left")       # grid[hi] >= am
    hi = np.minimum(hi, len(grid) - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo = am - grid[lo]                               # exact in float64
    d_hi = grid[hi] - am
    c_lo, c_hi = codes[lo], codes[hi]
    take_hi = (d_hi < d_lo) | ((d_hi == d_lo) & ((c_hi & 1) == 0))
    pick = np.where(take_hi, c_hi, c_lo)
    pick = np.where(am == grid[hi], c_hi, pick)        # exact hit (incl. zero)
    out[mid] = pick.astype(np.uint8)
    out[sat] = max_code
    out[nan] = nan_code
    return out | sign


# --------------------------------------------------------------------------
# O3/O4: scaled value and raw amax.
# --------------------------------------------------------------------------
def scaled_values(x_f32: np.ndarray, scale) -> np.ndarray:
    """fl32(x * s): one IEEE fp32 multiply (round to nearest even, no flush)."""
    return np.asarray(x_f32, dtype=np.float32) * np.float32(scale)


def amax(x_f32: np.ndarray) -> np.float32:
    """max |x| over the raw (unscaled) input, NaN ignored, 0 for no elements
    (log:fp8_mm.cu, commit 69f35c46e0)."""
    a = np.abs(np.asarray(x_f32, dtype=np.float32)).ravel()
    a = a[~np.isnan(a)]
    return np.float32(a.max()) if a.size else np.float32(0.0)


# --------------------------------------------------------------------------
# O6/O7: scale inverse and the history fold.
# --------------------------------------------------------------------------
def scale_inv(scale) -> np.float32:
    """fl32(1 / s) for the scale a quantize call used."""
    return np.float32(1.0) / np.float32(scale)


def next_scale(hist: np.ndarray, fmt: str) -> np.float32:
    """Scale published from an amax history window: fmt_max / max(window)."""
    m = np.float32(np.max(np.asarray(hist, dtype=np.float32)))
    if not (np.isfinite(m) and m > 0):
        return np.float32(1.0)
    with np.errstate(over="ignore"):
        s = np.float32(FMT_MAX[fmt]) / m
    if not (np.isfinite(s) and s > 0):
        return np.float32(1.0)
    return np.float32(s)


@dataclasses.dataclass
class Ring:
    """Device ring state, as plain values: history window, current scale and
    the slot the next amax goes to (log:tests/extension, the commits that pack
    history, scale and counter into one buffer and fold in-kernel)."""
    hist: np.ndarray          # float32[H]
    scale: np.float32
    idx: int

    @staticmethod
    def new(hist_len: int, scale0=1.0) -> "Ring":
        return Ring(np.zeros(hist_len, np.float32), np.float32(scale0), 0)

    def copy(self) -> "Ring":
        return Ring(self.hist.copy(), np.float32(self.scale), int(self.idx))

    def words(self) -> np.ndarray:
        """The (H+4) 32-bit words of the device buffer at rest:
        hist | scale | idx | ticket (0) | amax accumulator (0)."""
        h = len(self.hist)
        w = np.zeros(h + 4, dtype=np.uint32)
        w[:h] = self.hist.astype(np.float32).view(np.uint32)
        w[h] = np.array([self.scale], np.float32).view(np.uint32)[0]
        w[h + 1] = self.idx
        return w

    @staticmethod
    def from_words(w: np.ndarray) -> "Ring":
        w = np.asarray(w, dtype=np.uint32)
        h = len(w) - 4
        return Ring(w[:h].view(np.float32).copy(),
                    w[h:h + 1].view(np.float32)[0], int(w[h + 1]))


def fold(ring: Ring, amax_value, fmt: str) -> Ring:
    """Write amax into the current history slot, advance the slot modulo H,
    and publish fmt_max / max(window) as the next scale."""
    r = ring.copy()
    r.hist[r.idx] = np.float32(amax_value)
    r.idx = (r.idx + 1) % len(r.hist)
    r.scale = next_scale(r.hist, fmt)
    return r


# --------------------------------------------------------------------------
# O5/O8: one quantize call (row / transposed / dual layout).
# --------------------------------------------------------------------------
def quantize(x: np.ndarray, dtype: str, fmt: str, scale=None, ring: Ring | None = None):
    """Quantize a [rows, cols] tensor.

    Exactly one of `scale` (explicit per-tensor scale) or `ring` (delayed
    scaling: use ring.scale, then fold this call's raw amax) is given.
    Returns a dict: codes (row layout [rows, cols]), codes_t (= codes.T),
    amax, scale_inv (1/scale actually used) and ring (the folded ring, or None).
    """
    if (scale is None) == (ring is None):
        raise ValueError("give exactly one of scale / ring")
    xf = widen_to_f32(x, dtype)
    s = np.float32(ring.scale if ring is not None else scale)
    codes = encode(scaled_values(xf, s), fmt)
    a = amax(xf)
    new_ring = fold(ring, a, fmt) if ring is not None else None
    return {"codes": codes, "codes_t": np.ascontiguousarray(codes.T), "amax": a,
            "scale_inv": scale_inv(s), "ring": new_ring}


def quantize_dynamic(x: np.ndarray, dtype: str, fmt: str):
    """Current (dynamic) scaling: no history ring; the scale is measured from
    the tensor being quantized and used by the same call (log:tests/extension,
    the commit merging the delayed and dynamic recipes behind one `dynamic`
    flag, and the commit skipping scale-meta allocation on the dynamic path,
    whose scales are measured inline).  The pages give no formula of their own
    for it; the reading taken is the delayed rule over a window that holds
    only this tensor's amax: s = fmt_max / amax(x), 1.0 when amax is 0 or not
    finite or the quotient is not a finite positive number.  Returns the same
    dict as quantize (ring None)."""
    s = next_scale(np.array([amax(widen_to_f32(x, dtype))], dtype=np.float32), fmt)
    return quantize(x, dtype, fmt, scale=s)


# --------------------------------------------------------------------------
# bf16 rounding from float64 and the GEMM (O9-O11).
# --------------------------------------------------------------------------
def bf16_bits_from_f64(y: np.ndarray) -> np.ndarray:
    """Round float64 values once, to nearest even, to bf16; return the bits.

    bf16 keeps 8 significant bits over fp32's exponent range; below 2^-126
    its spacing is 2^-133.  Magnitudes at or above the midpoint between the
    largest bf16 (2^128 - 2^120) and 2^128 round to infinity.
    """
    y = np.asarray(y, dtype=np.float64)
    out = np.empty(y.shape, dtype=np.float64)
    fin = np.isfinite(y)
    yf = y[fin]
    _, e = np.frexp(np.abs(yf))                 # |y| = f * 2^e, f in [0.5, 1)
    e = e - 1                                   # floor(log2|y|) for y != 0
    e = np.maximum(e, -126)
    q = np.ldexp(1.0, (e - 7).astype(np.int64))  # spacing at that binade
    r = np.rint(yf / q) * q                     # y/q is exact: power-of-2 scaling
    r = np.where(np.abs(r) >= 2.0 ** 128, np.copysign(np.inf, yf), r)
    out[fin] = r
    out[~fin] = y[~fin]
    f32 = out.astype(np.float32)                # exact: r is a bf16 value
    return (f32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    return widen_to_f32(bits, BF16).astype(np.float64)


def ulp_bf16(x: np.ndarray) -> np.ndarray:
    """Spacing of bf16 at |x|: 2^(max(floor(log2|x|), -126) - 7); 2^-133 at 0."""
    x = np.abs(np.asarray(x, dtype=np.float64))
    out = np.full(x.shape, 2.0 ** -133)
    nz = x > 0
    _, e = np.frexp(x[nz])
    out[nz] = np.ldexp(1.0, (np.maximum(e - 1, -126) - 7).astype(np.int64))
    return out


def _as_batched(t: np.ndarray) -> np.ndarray:
    return t[None] if t.ndim == 2 else t


def mm_exact_f64(a_codes, fmt_a, b_codes, fmt_b, a_scale_inv=1.0, b_scale_inv=1.0, bias=None):
    """Pre-rounding GEMM value and the tolerance's sum of magnitudes.

    y[b,i,j] = sum_k dec(A[b,i,k]) * dec(B[b,j,k]) * sa_inv * sb_inv + bias[j]
    (NT operands: A is [M,K], B is [N,K], both K-contiguous).  The sum runs in
    float64; for E4M3 x E4M3 every partial sum is an exact float64 (codes are
    multiples of 2^-9 below 2^9), so the result does not depend on order.
    Returns (y, abs_sum) with abs_sum[b,i,j] = sum_k |a_ik * b_jk| in the
    dequantised (scaled) domain.
    """
    A = _as_batched(np.asarray(a_codes, dtype=np.uint8))
    B = _as_batched(np.asarray(b_codes, dtype=np.uint8))
    da = decode_table(fmt_a)[A]
    db = decode_table(fmt_b)[B]
    sab = float(np.float64(np.float32(a_scale_inv)) * np.float64(np.float32(b_scale_inv)))
    acc = np.matmul(da, np.swapaxes(db, -1, -2))
    mag = np.matmul(np.abs(da), np.swapaxes(np.abs(db), -1, -2))
    y = acc * sab
    if bias is not None:
        y = y + np.asarray(bias, dtype=np.float64)[None, None, :]
    return y, mag * abs(sab)


def mm(a_codes, fmt_a, b_codes, fmt_b, a_scale_inv=1.0, b_scale_inv=1.0, bias=None):
    """bf16 bits of the GEMM rounded once from float64, plus the abs-sum
    needed by `within_tolerance`.  `bias` is given as exact values (float64),
    e.g. from widen_to_f32 of bf16 bits."""
    y, mag = mm_exact_f64(a_codes, fmt_a, b_codes, fmt_b, a_scale_inv, b_scale_inv, bias)
    return bf16_bits_from_f64(y), mag


def within_tolerance(gpu_bits, ref_bits, abs_sum, rel=1e-5):
    """Acceptance bound of a GEMM output element:
    |gpu - ref| <= ulp_bf16(|ref|) + rel * sum_k |a_ik * b_jk|."""
    g = bf16_bits_to_f64(np.asarray(gpu_bits, dtype=np.uint16))
    r = bf16_bits_to_f64(np.asarray(ref_bits, dtype=np.uint16))
    bound = ulp_bf16(r) + rel * np.asarray(abs_sum, dtype=np.float64)
    with np.errstate(invalid="ignore"):
        ok = np.abs(g - r) <= bound
    return ok | ((g == r) & ~np.isnan(g))


# --------------------------------------------------------------------------
# O14/O15: fp8-stored bias and the quantizing (FP8-out) GEMM epilogue.
# --------------------------------------------------------------------------
def dequant_bias(codes: np.ndarray, fmt: str, bias_scale) -> np.ndarray:
    """An fp8-stored bias as the epilogue uses it: fl32(dec(code) * s_b), one
    fp32 multiply of the code's exact value by the bias scale, applied after
    the operand scaling and before any output quantization (log:tests/extension,
    the commit giving the bias a bias_scale slot: no scale = a bf16 bias, a
    scale = fp8 storage dequantized in the epilogue)."""
    return scaled_values(decode_table(fmt)[np.asarray(codes, dtype=np.uint8)].astype(np.float32), bias_scale)


def mm_quantized(a_codes, fmt_a, b_codes, fmt_b, fmt_c, a_scale_inv=1.0, b_scale_inv=1.0, bias=None,
                 scale=None, ring: Ring | None = None):
    """FP8-in / FP8-out GEMM (log:tests/extension, the commit adding the
    FP8-in/FP8-out GEMM op; the output quantization comes after the bias, per
    the bias_scale commit).  The pre-quantization output is the GEMM's value
    y (mm_exact_f64) held in fp32, fl32(y); it is then quantized exactly as a
    quantize call quantizes an fp32 tensor: codes enc(fl32(fl32(y) * s_c)),
    amax over fl32(y) (NaN ignored, every batch together), s_c explicit or the
    ring's current scale, and one fold of that amax into the ring.  Returns
    the quantize dict (codes shaped like y) plus y and abs_sum for the
    tolerance."""
    y, mag = mm_exact_f64(a_codes, fmt_a, b_codes, fmt_b, a_scale_inv, b_scale_inv, bias)
    with np.errstate(over="ignore"):
        y32 = y.astype(np.float32)
    q = quantize(y32.reshape(-1, y32.shape[-1]), F32, fmt_c, scale=scale, ring=ring)
    out = {k: q[k] for k in ("amax", "scale_inv", "ring")}
    out["codes"] = q["codes"].reshape(y.shape)
    out["y"], out["abs"] = y, mag
    return out


def grad_bias(dy_bits: np.ndarray, dtype: str = BF16):
    """Bias gradient: sum of the bf16 (or fp16) upstream gradient over every
    leading dimension, summed in float64 and rounded once to bf16
    (log:tests/extension, the commit reducing grad_b over leading dims; grads
    are bf16).  Returns (bits, abs_sum) for the same tolerance form as the GEMM."""
    v = widen_to_f32(dy_bits, dtype).astype(np.float64)
    v = v.reshape(-1, v.shape[-1])
    return bf16_bits_from_f64(v.sum(axis=0)), np.abs(v).sum(axis=0)


# --------------------------------------------------------------------------
# O12: the delayed-scaling step, as the caller drives it.
# --------------------------------------------------------------------------
def seed_ring(hist_len: int, x_first: np.ndarray, dtype: str, fmt: str) -> Ring:
    """A zeroed ring whose scale is fmt_max / amax of the first tensor seen
    (1.0 when that amax is 0), i.e. what a fold of that amax into a zeroed
    window publishes."""
    return Ring.new(hist_len, next_scale(np.array([amax(widen_to_f32(x_first, dtype))]), fmt))


def linear_forward(x, w, bias_bits, ring_x: Ring, ring_w: Ring):
    """Forward of one fp8 linear layer under delayed scaling: quantize x and W
    to E4M3 with their rings (scales snapshotted before the fold), then
    Y = Xq Wq^T * sx_inv * sw_inv + b rounded once to bf16."""
    qx = quantize(x, BF16, E4M3, ring=ring_x)
    qw = quantize(w, BF16, E4M3, ring=ring_w)
    bias = None if bias_bits is None else widen_to_f32(bias_bits, BF16).astype(np.float64)
    y, mag = mm(qx["codes"], E4M3, qw["codes"], E4M3, qx["scale_inv"], qw["scale_inv"], bias)
    return {"qx": qx, "qw": qw, "y": y[0], "y_abs": mag[0]}


def linear_backward(dy, qx, qw, ring_g: Ring):
    """Backward under delayed scaling: dY -> E5M2 with its own ring; dX = dY W
    and dW = dY^T X as NT GEMMs on the transposed codes, reusing the forward's
    x / W scales; grad_b over leading dims."""
    qg = quantize(dy, BF16, E5M2, ring=ring_g)
    dx, dx_mag = mm(qg["codes"], E5M2, qw["codes_t"], E4M3, qg["scale_inv"], qw["scale_inv"])
    dw, dw_mag = mm(qg["codes_t"], E5M2, qx["codes_t"], E4M3, qg["scale_inv"], qx["scale_inv"])
    db, db_mag = grad_bias(dy)
    return {"qg": qg, "dx": dx[0], "dx_abs": dx_mag[0], "dw": dw[0], "dw_abs": dw_mag[0],
            "db": db, "db_abs": db_mag}
