"""fp8mi: FP8 per-tensor scaled quantize, delayed-scaling amax history fold
and per-tensor-scaled fp8 GEMM on MI355X (gfx950).

Thin Python binding over the C ABI in include/fp8mi.h (libfp8mi.so).  The
functions carry the ABI's names and only marshal arguments: shapes, strides
and device pointers of torch tensors, and torch's current HIP stream.  Every
step of the computation runs in the library's HIP kernels; when the library
is missing, every call raises.
"""
from __future__ import annotations

import torch

from ._lib import lib

__all__ = ["E4M3", "E5M2", "F32", "F16", "BF16", "Fp8Error", "fp8_quantize", "fp8_quantize_dual", "fp8_quantize_dual_bias_grad",
           "fp8_quantize_dual_bias_grad_noalloc", "NOALLOC_SCRATCH_BYTES", "stream_reference",
           "fp8_quantize_dynamic", "DYNAMIC_WORKSPACE_BYTES", "fp8_amax_fold", "fp8_mm", "fp8_mm_ex", "FP8_E4M3", "FP8_E5M2", "fp8_bias_grad", "fp8_bias_grad_workspace_bytes", "fp8_ring_seed", "new_ring", "ring_words", "version"]

E4M3, E5M2 = 0, 1
F32, F16, BF16 = 0, 1, 2
FP8_E4M3, FP8_E5M2 = 3, 4  # fp8 storage types (fp8 bias / fp8 GEMM output of fp8_mm_ex)

_FMT = {"e4m3": E4M3, "e5m2": E5M2, E4M3: E4M3, E5M2: E5M2}
_DT = {torch.float32: F32, torch.float16: F16, torch.bfloat16: BF16}
RING_SCRATCH_WORDS = 1024  # FP8MI_RING_SCRATCH_WORDS
DYNAMIC_WORKSPACE_BYTES = 4096  # FP8MI_DYNAMIC_WORKSPACE_BYTES
NOALLOC_SCRATCH_BYTES = 8 * 1024 * 1024  # FP8MI_NOALLOC_SCRATCH_BYTES
LAYOUT_ROW, LAYOUT_T, LAYOUT_DUAL = 0, 1, 2


def ring_words_for(hist_len: int) -> int:
    """FP8MI_RING_WORDS(hist_len)."""
    return hist_len + 4 + RING_SCRATCH_WORDS


class Fp8Error(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"fp8mi status {status}: {detail}")
        self.status = status


def _check(status: int) -> None:
    if status != 0:
        L = lib()
        raise Fp8Error(status, f"{L.fp8mi_status_string(status).decode()} -- {L.fp8mi_last_error().decode()}")


def _fmt(f) -> int:
    try:
        return _FMT[f]
    except KeyError:
        raise ValueError(f"unknown fp8 format {f!r}") from None


def _ptr(t):
    return None if t is None else t.data_ptr()


_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)
_raw_device = getattr(torch._C, "_cuda_getDevice", None)


def _current_device() -> int:
    """torch's current HIP device (the raw getter skips the lazy-init check,
    done already by the time a device tensor exists)."""
    return _raw_device() if _raw_device is not None else torch.cuda.current_device()


def _stream(t: torch.Tensor):
    """Handle of torch's current HIP stream on t's device (the raw getter
    skips building a Stream object: a few microseconds per call)."""
    if _raw_stream is not None:
        return _raw_stream(t.get_device())
    return torch.cuda.current_stream(t.device).cuda_stream


def _as_codes(t: torch.Tensor, name: str = "codes") -> torch.Tensor:
    if t.element_size() != 1:
        raise ValueError(f"{name} must hold 1-byte fp8 codes, got {t.dtype}")
    return t.view(torch.uint8) if t.dtype != torch.uint8 else t


# Argument checks.  The library takes raw device pointers and sizes, so the
# binding checks what only the tensors know -- device, dtype, shape -- before
# the call; the library itself checks sizes, strides and alignment.

def _on_device(*ts) -> None:
    """Every tensor argument lives on the current HIP device (the library
    launches there): a host tensor or another device's memory would be read
    as this device's."""
    dev = None
    for t in ts:
        if t is None:
            continue
        d = t.get_device()
        if d < 0:
            raise ValueError("tensor arguments must be HIP device tensors, got a host tensor")
        if dev is None:
            dev = d
        elif d != dev:
            raise ValueError(f"tensor arguments on devices cuda:{dev} and cuda:{d}")
    if dev is not None and dev != _current_device():
        raise ValueError(f"tensors on cuda:{dev} but the current device is cuda:{_current_device()}")


def _dt(t: torch.Tensor, name: str) -> int:
    try:
        return _DT[t.dtype]
    except KeyError:
        raise ValueError(f"{name} must be float32, float16 or bfloat16, got {t.dtype}") from None


def _scalar(t, name: str) -> None:
    """A device fp32 scalar argument (its first element is read or written)."""
    if t is not None and (t.dtype != torch.float32 or t.numel() < 1):
        raise ValueError(f"{name} must be a float32 tensor of at least one element")


def _matrix_out(t: torch.Tensor, shape, name: str) -> None:
    """A 2-D output of exactly `shape` with unit stride along its rows."""
    if t.shape != shape:
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if shape[1] > 1 and t.stride(1) != 1:
        raise ValueError(f"{name} needs unit stride along its rows")


def _vector(t: torch.Tensor, n: int, name: str) -> None:
    """A contiguous 1-D tensor of n elements."""
    if t.dim() != 1 or t.numel() != n or (n > 1 and t.stride(0) != 1):
        raise ValueError(f"{name} must be a contiguous 1-D tensor of {n} elements, got {tuple(t.shape)}")


def _quant_checks(x, name, out_row, out_t, scale, scale_inv_out, amax_out):
    rows, cols = x.shape
    if out_row is not None:
        _matrix_out(out_row, (rows, cols), "out" if out_t is None else "out_row")
    if out_t is not None:
        _matrix_out(out_t, (cols, rows), "out" if out_row is None else "out_t")
    _scalar(scale, "scale")
    _scalar(scale_inv_out, "scale_inv_out")
    _scalar(amax_out, "amax_out")
    return _dt(x, name)


def _ring_args(ring):
    if ring is None:
        return None, 0
    if ring.dim() != 1 or ring.dtype not in (torch.int32, torch.uint32) or not ring.is_contiguous():
        raise ValueError("ring must be a contiguous 1-D int32 tensor of hist_len + 4 + 1024 words")
    h = ring.numel() - 4 - RING_SCRATCH_WORDS
    if h < 1:
        raise ValueError(f"ring of {ring.numel()} words is too short")
    return ring.data_ptr(), h


def version() -> str:
    return lib().fp8mi_version().decode()


def new_ring(hist_len: int, scale0: float = 1.0, device=None) -> torch.Tensor:
    """A zeroed ring (history 0, slot 0, ticket and scratch 0) holding scale0
    as its current scale: FP8MI_RING_WORDS(hist_len) int32 words on `device`."""
    w = torch.zeros(ring_words_for(hist_len), dtype=torch.int32)
    w[hist_len] = torch.tensor([scale0], dtype=torch.float32).view(torch.int32)[0]
    return w.to(device if device is not None else "cuda")


def ring_words(ring: torch.Tensor):
    """Host copy of a ring: dict of hist (fp32), scale, idx, ticket and
    whether the scratch region is all zero (as it is between calls)."""
    w = ring.detach().to("cpu")
    h = w.numel() - 4 - RING_SCRATCH_WORDS
    f = w.view(torch.float32)
    return {"hist": f[:h].clone(), "scale": float(f[h]), "idx": int(w[h + 1]),
            "ticket": int(w[h + 2]), "scratch_clear": bool((w[h + 3:] == 0).all())}


def fp8_quantize(x: torch.Tensor, fmt, transposed: bool = False, out: torch.Tensor | None = None,
                 scale: torch.Tensor | None = None, ring: torch.Tensor | None = None,
                 scale_inv_out: torch.Tensor | None = None, amax_out: torch.Tensor | None = None) -> torch.Tensor:
    """Quantize a 2-D bf16/fp16/fp32 tensor (unit column stride; any row
    stride and base offset) to fp8 codes (uint8) in row or transposed layout.
    Exactly one of `scale` (device fp32 scalar) or `ring` is given."""
    if x.dim() != 2 or (x.shape[1] > 1 and x.stride(1) != 1):
        raise ValueError("x must be 2-D with unit column stride")
    rows, cols = x.shape
    f = _fmt(fmt)
    if out is None:
        out = torch.empty((cols, rows) if transposed else (rows, cols), dtype=torch.uint8, device=x.device)
    out = _as_codes(out, "out")
    dt = _quant_checks(x, "x", None if transposed else out, out if transposed else None, scale, scale_inv_out,
                       amax_out)
    ld_x = x.stride(0) if rows > 1 else cols
    ld_out = out.stride(0) if out.shape[0] > 1 else out.shape[1]
    rp, h = _ring_args(ring)
    _on_device(x, out, scale, ring, scale_inv_out, amax_out)
    _check(lib().fp8_quantize(_ptr(x), dt, rows, cols, ld_x, f, int(bool(transposed)), _ptr(out),
                              ld_out, _ptr(scale), rp, h, _ptr(scale_inv_out), _ptr(amax_out), _stream(x)))
    return out


def fp8_quantize_dual(x: torch.Tensor, fmt, out_row: torch.Tensor | None = None, out_t: torch.Tensor | None = None,
                      scale: torch.Tensor | None = None, ring: torch.Tensor | None = None,
                      scale_inv_out: torch.Tensor | None = None, amax_out: torch.Tensor | None = None):
    """Both layouts from one read; returns (codes [rows, cols], codes_t [cols, rows])."""
    if x.dim() != 2 or (x.shape[1] > 1 and x.stride(1) != 1):
        raise ValueError("x must be 2-D with unit column stride")
    rows, cols = x.shape
    f = _fmt(fmt)
    if out_row is None:
        out_row = torch.empty((rows, cols), dtype=torch.uint8, device=x.device)
    if out_t is None:
        out_t = torch.empty((cols, rows), dtype=torch.uint8, device=x.device)
    out_row, out_t = _as_codes(out_row, "out_row"), _as_codes(out_t, "out_t")
    dt = _quant_checks(x, "x", out_row, out_t, scale, scale_inv_out, amax_out)
    ld_x = x.stride(0) if rows > 1 else cols
    ld_r = out_row.stride(0) if out_row.shape[0] > 1 else out_row.shape[1]
    ld_t = out_t.stride(0) if out_t.shape[0] > 1 else out_t.shape[1]
    rp, h = _ring_args(ring)
    _on_device(x, out_row, out_t, scale, ring, scale_inv_out, amax_out)
    _check(lib().fp8_quantize_dual(_ptr(x), dt, rows, cols, ld_x, f, _ptr(out_row), ld_r, _ptr(out_t),
                                   ld_t, _ptr(scale), rp, h, _ptr(scale_inv_out), _ptr(amax_out), _stream(x)))
    return out_row, out_t


def fp8_quantize_dual_bias_grad(dy: torch.Tensor, fmt, out_row: torch.Tensor | None = None,
                                out_t: torch.Tensor | None = None, scale: torch.Tensor | None = None,
                                ring: torch.Tensor | None = None, scale_inv_out: torch.Tensor | None = None,
                                amax_out: torch.Tensor | None = None, bias_grad_out: torch.Tensor | None = None,
                                workspace: torch.Tensor | None = None):
    """fp8_quantize_dual of a 2-D bf16/fp16 gradient plus its bias gradient
    from the same read; returns (codes, codes_t, bias_grad bf16 [cols])."""
    if dy.dim() != 2 or (dy.shape[1] > 1 and dy.stride(1) != 1):
        raise ValueError("dy must be 2-D with unit column stride")
    rows, cols = dy.shape
    f = _fmt(fmt)
    if out_row is None:
        out_row = torch.empty((rows, cols), dtype=torch.uint8, device=dy.device)
    if out_t is None:
        out_t = torch.empty((cols, rows), dtype=torch.uint8, device=dy.device)
    if bias_grad_out is None:
        bias_grad_out = torch.empty(cols, dtype=torch.bfloat16, device=dy.device)
    need = fp8_bias_grad_workspace_bytes(rows, cols)
    if workspace is None:
        workspace = torch.empty(max(need, 8), dtype=torch.uint8, device=dy.device)
    out_row, out_t = _as_codes(out_row, "out_row"), _as_codes(out_t, "out_t")
    dt = _quant_checks(dy, "dy", out_row, out_t, scale, scale_inv_out, amax_out)
    _vector(bias_grad_out, cols, "bias_grad_out")
    if bias_grad_out.dtype != torch.bfloat16:
        raise ValueError("bias_grad_out must be bfloat16")
    ld_x = dy.stride(0) if rows > 1 else cols
    ld_r = out_row.stride(0) if out_row.shape[0] > 1 else out_row.shape[1]
    ld_t = out_t.stride(0) if out_t.shape[0] > 1 else out_t.shape[1]
    rp, h = _ring_args(ring)
    _on_device(dy, out_row, out_t, scale, ring, scale_inv_out, amax_out, bias_grad_out, workspace)
    _check(lib().fp8_quantize_dual_bias_grad(_ptr(dy), dt, rows, cols, ld_x, f, _ptr(out_row), ld_r,
                                             _ptr(out_t), ld_t, _ptr(scale), rp, h, _ptr(scale_inv_out),
                                             _ptr(amax_out), _ptr(bias_grad_out), _ptr(workspace),
                                             workspace.numel() * workspace.element_size(), _stream(dy)))
    return out_row, out_t, bias_grad_out


def fp8_quantize_dual_bias_grad_noalloc(dy: torch.Tensor, fmt, out_row: torch.Tensor, out_t: torch.Tensor,
                                        bias_grad_out: torch.Tensor, scale: torch.Tensor | None = None,
                                        ring: torch.Tensor | None = None, scale_inv_out: torch.Tensor | None = None,
                                        amax_out: torch.Tensor | None = None):
    """fp8_quantize_dual_bias_grad with the library's own scratch instead of a
    workspace: every output is the caller's (nothing is allocated here or in
    the library).  Returns (codes, codes_t, bias_grad)."""
    if dy.dim() != 2 or (dy.shape[1] > 1 and dy.stride(1) != 1):
        raise ValueError("dy must be 2-D with unit column stride")
    rows, cols = dy.shape
    f = _fmt(fmt)
    out_row, out_t = _as_codes(out_row, "out_row"), _as_codes(out_t, "out_t")
    dt = _quant_checks(dy, "dy", out_row, out_t, scale, scale_inv_out, amax_out)
    _vector(bias_grad_out, cols, "bias_grad_out")
    if bias_grad_out.dtype != torch.bfloat16:
        raise ValueError("bias_grad_out must be bfloat16")
    ld_x = dy.stride(0) if rows > 1 else cols
    ld_r = out_row.stride(0) if out_row.shape[0] > 1 else out_row.shape[1]
    ld_t = out_t.stride(0) if out_t.shape[0] > 1 else out_t.shape[1]
    rp, h = _ring_args(ring)
    _on_device(dy, out_row, out_t, scale, ring, scale_inv_out, amax_out, bias_grad_out)
    _check(lib().fp8_quantize_dual_bias_grad_noalloc(_ptr(dy), dt, rows, cols, ld_x, f, _ptr(out_row), ld_r,
                                                     _ptr(out_t), ld_t, _ptr(scale), rp, h, _ptr(scale_inv_out),
                                                     _ptr(amax_out), _ptr(bias_grad_out), _stream(dy)))
    return out_row, out_t, bias_grad_out


def stream_reference(src: torch.Tensor, dst: torch.Tensor) -> torch.Tensor:
    """Measurement aid: fp8mi_stream_reference over two contiguous device
    tensors (dst of src's byte size or its half) -- the HBM traffic of a
    quantize moving the same bytes, with no arithmetic."""
    for t, name in ((src, "src"), (dst, "dst")):
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    _on_device(src, dst)
    _check(lib().fp8mi_stream_reference(src.data_ptr(), src.numel() * src.element_size(), dst.data_ptr(),
                                        dst.numel() * dst.element_size(), _stream(src)))
    return dst


def fp8_quantize_dynamic(x: torch.Tensor, fmt, layout: int = LAYOUT_ROW, out_row: torch.Tensor | None = None,
                         out_t: torch.Tensor | None = None, scale_inv_out: torch.Tensor | None = None,
                         amax_out: torch.Tensor | None = None, workspace: torch.Tensor | None = None):
    """Current scaling: quantize a 2-D bf16/fp16/fp32 tensor with
    s = fmt_max / amax(x) measured in the same call (no ring).  layout 0 row,
    1 transposed, 2 both; returns (codes or None, codes_t or None)."""
    if x.dim() != 2 or (x.shape[1] > 1 and x.stride(1) != 1):
        raise ValueError("x must be 2-D with unit column stride")
    if layout not in (LAYOUT_ROW, LAYOUT_T, LAYOUT_DUAL):
        raise ValueError(f"layout must be 0, 1 or 2, got {layout!r}")
    rows, cols = x.shape
    f = _fmt(fmt)
    if layout != LAYOUT_T and out_row is None:
        out_row = torch.empty((rows, cols), dtype=torch.uint8, device=x.device)
    if layout != LAYOUT_ROW and out_t is None:
        out_t = torch.empty((cols, rows), dtype=torch.uint8, device=x.device)
    if workspace is None:
        workspace = torch.empty(DYNAMIC_WORKSPACE_BYTES, dtype=torch.uint8, device=x.device)
    out_row = None if out_row is None else _as_codes(out_row, "out_row")
    out_t = None if out_t is None else _as_codes(out_t, "out_t")
    dt = _quant_checks(x, "x", out_row if layout != LAYOUT_T else None, out_t if layout != LAYOUT_ROW else None,
                       None, scale_inv_out, amax_out)
    _on_device(x, out_row, out_t, scale_inv_out, amax_out, workspace)
    ld_x = x.stride(0) if rows > 1 else cols
    ld_r = 0 if out_row is None else (out_row.stride(0) if out_row.shape[0] > 1 else out_row.shape[1])
    ld_t = 0 if out_t is None else (out_t.stride(0) if out_t.shape[0] > 1 else out_t.shape[1])
    _check(lib().fp8_quantize_dynamic(_ptr(x), dt, rows, cols, ld_x, f, layout, _ptr(out_row), ld_r,
                                      _ptr(out_t), ld_t, _ptr(scale_inv_out), _ptr(amax_out), _ptr(workspace),
                                      workspace.numel() * workspace.element_size(), _stream(x)))
    return out_row, out_t


def fp8_amax_fold(ring: torch.Tensor, amax: torch.Tensor, fmt) -> None:
    """Fold a device fp32 amax into the ring (the fold a ring-mode quantize
    performs in its last workgroup)."""
    rp, h = _ring_args(ring)
    _scalar(amax, "amax")
    _on_device(ring, amax)
    _check(lib().fp8_amax_fold(rp, h, _ptr(amax), _fmt(fmt), _stream(ring)))


def fp8_mm(a: torch.Tensor, b: torch.Tensor, fmt_a=E4M3, fmt_b=E4M3, a_scale_inv: torch.Tensor | None = None,
           b_scale_inv: torch.Tensor | None = None, bias: torch.Tensor | None = None,
           out: torch.Tensor | None = None) -> torch.Tensor:
    """C = bf16(A B^T * sa * sb + bias) for fp8 codes A [(batch,) M, K] and
    B [(batch,) N, K]; a size-1 (or stride-0) batch dimension broadcasts.
    An operand that is a transposed view (unit stride along its rows, e.g.
    codes_t.t()) is read K-major through fp8_mm_ex's layout tags."""
    return _mm_call(a, b, fmt_a, fmt_b, a_scale_inv, b_scale_inv, bias, None, None, out, None, ex=False)


def fp8_mm_ex(a: torch.Tensor, b: torch.Tensor, fmt_a=E4M3, fmt_b=E4M3, a_scale_inv: torch.Tensor | None = None,
              b_scale_inv: torch.Tensor | None = None, bias: torch.Tensor | None = None,
              bias_fmt=None, bias_scale: torch.Tensor | None = None, out: torch.Tensor | None = None,
              out_fmt=None, out_scale: torch.Tensor | None = None, out_ring: torch.Tensor | None = None,
              out_scale_inv: torch.Tensor | None = None, out_amax: torch.Tensor | None = None) -> torch.Tensor:
    """fp8_mm with an fp8-stored bias (codes `bias` of format `bias_fmt`,
    dequantized by `bias_scale`) and/or a quantizing epilogue: with `out_fmt`
    (E4M3 / E5M2) the output is fp8 codes quantized with `out_scale` or the
    ring `out_ring` (which then folds the output's amax); `out_scale_inv` and
    `out_amax` receive 1/s and amax."""
    return _mm_call(a, b, fmt_a, fmt_b, a_scale_inv, b_scale_inv, bias, bias_fmt, bias_scale, out, out_fmt,
                    out_scale, out_ring, out_scale_inv, out_amax)


def _operand(t: torch.Tensor, name: str):
    """(batch, rows, K, batch stride, leading dimension, K-major) of a
    [rows, K] or [batch, rows, K] operand.  An operand that is a transposed
    view of [K, rows] storage (unit stride along its rows) is K-major: the
    library reads it through the FP8MI_A_KM / FP8MI_B_KM layout tags."""
    if t.dim() == 3:
        batch, rows, K = t.shape
        sb, sr, sk = t.stride()
    elif t.dim() == 2:
        batch, (rows, K), sb = 1, t.shape, 0
        sr, sk = t.stride()
    else:
        raise ValueError(f"operand {name} must be [rows, K] or [batch, rows, K], got {tuple(t.shape)}")
    if batch == 1:
        sb = 0
    if K <= 1 or sk == 1:
        return batch, rows, K, sb, (sr if rows > 1 else K), False
    if rows <= 1 or sr == 1:
        ld = sk
        # the library reads K full rows of ld bytes (the last row's padding included)
        last = t.storage_offset() + (batch - 1) * sb + K * ld
        if last > t.untyped_storage().nbytes():
            raise ValueError(f"K-major operand {name} must span {K} full rows of {ld} bytes in its storage")
        return batch, rows, K, sb, ld, True
    raise ValueError(f"operand {name} needs unit stride along K or along its rows")


def _operand_ld(t: torch.Tensor, name: str):
    """Leading dimension of an operand and whether it is K-major."""
    return _operand(t, name)[4:]


def _mm_call(a, b, fmt_a, fmt_b, a_scale_inv, b_scale_inv, bias, bias_fmt, bias_scale, out, out_fmt,
             out_scale=None, out_ring=None, out_scale_inv=None, out_amax=None, ex=True):
    a, b = _as_codes(a, "a"), _as_codes(b, "b")
    ba, M, K, sa, lda, a_km = _operand(a, "a")
    bb, N, Kb, sb, ldb, b_km = _operand(b, "b")
    if K != Kb:
        raise ValueError(f"K mismatch: {tuple(a.shape)} vs {tuple(b.shape)}")
    batch = ba if ba > 1 else bb
    if ba not in (1, batch) or bb not in (1, batch):
        raise ValueError("batch sizes must match or be 1")
    layout = (1 if a_km else 0) | (2 if b_km else 0)
    c_dt = BF16 if out_fmt is None else FP8_E4M3 + _fmt(out_fmt)
    batched = a.dim() == 3 or b.dim() == 3
    if out is None:
        out = torch.empty((batch, M, N) if batched else (M, N), dtype=torch.bfloat16 if c_dt == BF16 else torch.uint8,
                          device=a.device)
    if c_dt != BF16:
        out = _as_codes(out, "out")
    elif out.dtype != torch.bfloat16:
        raise ValueError(f"out must be bfloat16, got {out.dtype}")
    if out.dim() == 3:
        cshape, (sc, ldc, scn) = tuple(out.shape), out.stride()
    else:
        cshape, (ldc, scn) = (1,) + tuple(out.shape), out.stride()
        sc = M * ldc
    if cshape != (batch, M, N):
        raise ValueError(f"out has shape {tuple(out.shape)}, expected {(batch, M, N) if batch > 1 else (M, N)}")
    if N > 1 and scn != 1:
        raise ValueError("out needs unit stride along N")
    if M <= 1:
        ldc = N
    if batch <= 1:
        sc = M * ldc
    if bias is None:
        bias_dt = 0
    elif bias_fmt is not None:
        bias, bias_dt = _as_codes(bias, "bias"), FP8_E4M3 + _fmt(bias_fmt)
    else:
        bias_dt = _dt(bias, "bias")
    if bias is not None:
        _vector(bias, N, "bias")
    _scalar(a_scale_inv, "a_scale_inv")
    _scalar(b_scale_inv, "b_scale_inv")
    if ex:
        for t, name in ((bias_scale, "bias_scale"), (out_scale, "out_scale"), (out_scale_inv, "out_scale_inv"),
                        (out_amax, "out_amax")):
            _scalar(t, name)
        _on_device(a, b, a_scale_inv, b_scale_inv, bias, bias_scale, out, out_scale, out_ring, out_scale_inv,
                   out_amax)
    else:
        _on_device(a, b, a_scale_inv, b_scale_inv, bias, out)
    L = lib()
    if not ex and layout == 0:
        _check(L.fp8_mm(a.data_ptr(), _fmt(fmt_a), lda, sa, b.data_ptr(), _fmt(fmt_b), ldb, sb, M, N, K, batch,
                        _ptr(a_scale_inv), _ptr(b_scale_inv), _ptr(bias), bias_dt, out.data_ptr(), ldc, sc,
                        _stream(a)))
        return out
    rp, h = _ring_args(out_ring)
    _check(L.fp8_mm_ex(a.data_ptr(), _fmt(fmt_a), lda, sa, b.data_ptr(), _fmt(fmt_b), ldb, sb, M, N, K, batch,
                       layout, _ptr(a_scale_inv), _ptr(b_scale_inv), _ptr(bias), bias_dt, _ptr(bias_scale),
                       out.data_ptr(), c_dt, ldc, sc, _ptr(out_scale), rp, h, _ptr(out_scale_inv), _ptr(out_amax),
                       _stream(a)))
    return out


def fp8_bias_grad_workspace_bytes(rows: int, cols: int) -> int:
    """Device workspace fp8_bias_grad needs for a [rows, cols] gradient."""
    return int(lib().fp8_bias_grad_workspace_bytes(rows, cols))


def fp8_bias_grad(dy: torch.Tensor, out: torch.Tensor | None = None,
                  workspace: torch.Tensor | None = None) -> torch.Tensor:
    """Bias gradient: sum of a bf16/fp16 gradient over every leading
    dimension (fp64 accumulation in a fixed order, one bf16 rounding) ->
    bf16 [cols].  `workspace` (any dtype, device) is scratch of at least
    fp8_bias_grad_workspace_bytes(rows, cols) bytes; one is allocated from
    torch's caching allocator when it is not given."""
    if dy.dim() < 1 or (dy.shape[-1] > 1 and dy.stride(-1) != 1):
        raise ValueError("dy needs unit stride along its last dimension")
    cols = dy.shape[-1]
    d2 = dy.reshape(-1, cols)
    rows = d2.shape[0]
    ld = d2.stride(0) if rows > 1 else cols
    if out is None:
        out = torch.empty(cols, dtype=torch.bfloat16, device=dy.device)
    need = fp8_bias_grad_workspace_bytes(rows, cols)
    if workspace is None:
        workspace = torch.empty(max(need, 8), dtype=torch.uint8, device=dy.device)
    dt = _dt(dy, "dy")
    _vector(out, cols, "out")
    if out.dtype != torch.bfloat16:
        raise ValueError("out must be bfloat16")
    _on_device(d2, out, workspace)
    nbytes = workspace.numel() * workspace.element_size()
    _check(lib().fp8_bias_grad(_ptr(d2), dt, rows, cols, ld, _ptr(out), _ptr(workspace), nbytes,
                               _stream(dy)))
    return out


def fp8_ring_seed(ring: torch.Tensor, amax: torch.Tensor, fmt) -> None:
    """Reset a ring and publish the scale a fold of `amax` into an empty
    window gives (fmt_max / amax, or 1.0)."""
    rp, h = _ring_args(ring)
    _scalar(amax, "amax")
    _on_device(ring, amax)
    _check(lib().fp8_ring_seed(rp, h, _ptr(amax), _fmt(fmt), _stream(ring)))
