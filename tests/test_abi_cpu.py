"""The C-ABI library loads, exports every symbol include/fp8mi.h declares,
and rejects invalid arguments with the documented status before touching the
GPU (these calls never reach a HIP API, so they run without a device)."""
import ctypes as C
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp8mi.h")

fp8mi = pytest.importorskip("fp8_tensor_scaled_quantize_amd")
from fp8_tensor_scaled_quantize_amd import _lib  # noqa: E402

OK, NULL, ENUM, SHAPE, STRIDE, UNSUP, HIP, ARG = range(8)
FAKE = 0x10000  # never dereferenced: every call below fails validation first


def declared_functions():
    text = open(HEADER).read()
    return re.findall(r"FP8MI_API\s+[\w\s\*]+?\b(\w+)\s*\(", text)


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.skip("libfp8mi.so not built")
    return _lib.lib()


def test_header_declares_the_abi():
    names = declared_functions()
    assert set(names) == {"fp8_quantize", "fp8_quantize_dual", "fp8_amax_fold", "fp8_mm",
                          "fp8mi_status_string", "fp8mi_last_error", "fp8mi_version", "fp8mi_stream_reference"} | set(
        n for n in names if n.startswith("fp8_"))


def test_every_declared_symbol_is_exported(L):
    for name in declared_functions():
        assert hasattr(L, name), name
        assert name in _lib.SIGNATURES, f"binding lacks {name}"


def _ctype(decl: str):
    """ctypes type of one C parameter / return declaration of the header."""
    decl = " ".join(decl.replace("const ", "").split())
    if "*" in decl:
        return C.c_char_p if decl.startswith("char") else C.c_void_p
    base = decl.split()[0]
    return {"int": C.c_int, "int32_t": C.c_int32, "int64_t": C.c_int64, "size_t": C.c_size_t,
            "fp8mi_status": C.c_int}[base]


def test_binding_signatures_match_the_header():
    """Every declaration's return type and parameter types equal the ctypes
    signature the binding installs (a mismatch would pass arguments in the
    wrong registers or widths without any error)."""
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    decls = re.findall(r"FP8MI_API\s+([\w\s\*]+?)\b(\w+)\s*\(([^)]*)\)", text)
    assert len(decls) == len(_lib.SIGNATURES)
    for ret, name, params in decls:
        res, args = _lib.SIGNATURES[name]
        assert _ctype(ret) == res, name
        plist = [p.strip() for p in params.split(",") if p.strip() and p.strip() != "void"]
        assert [_ctype(p) for p in plist] == list(args), name


def test_error_text_is_per_thread(L):
    """fp8mi_last_error is thread-local: rejected calls in four threads each
    see their own text, and the calling thread sees none of them."""
    import threading
    texts = {}

    def worker(t):
        st = L.fp8_quantize(FAKE, 2, 4, 4, 4, 7 + t, 0, FAKE, 4, FAKE, None, 0, None, None, None)
        texts[t] = (st, L.fp8mi_last_error().decode())

    ths = [threading.Thread(target=worker, args=(t,)) for t in range(4)]
    for th in ths:
        th.start()
    for th in ths:
        th.join(timeout=30)
    for t in range(4):
        st, text = texts[t]
        assert st == ENUM and f"fmt {7 + t} " in text, (t, text)
    main = L.fp8mi_last_error().decode()
    assert all(f"fmt {7 + t} " not in main for t in range(4))


def test_version_and_status_strings(L):
    assert L.fp8mi_version().decode().startswith("fp8mi")
    for s in range(8):
        assert L.fp8mi_status_string(s).decode()
    assert L.fp8mi_status_string(99) == b"unknown status"


def q(L, x=FAKE, dt=2, rows=4, cols=4, ld=4, fmt=0, tr=0, out=FAKE, ld_out=4, scale=FAKE, ring=None, H=0,
      sinv=None, amax=None):
    return L.fp8_quantize(x, dt, rows, cols, ld, fmt, tr, out, ld_out, scale, ring, H, sinv, amax, None)


@pytest.mark.parametrize("kw,status", [
    (dict(dt=3), ENUM), (dict(dt=-1), ENUM), (dict(fmt=2), ENUM), (dict(tr=2), ENUM),
    (dict(rows=-1), SHAPE), (dict(cols=-5), SHAPE), (dict(ld=3), SHAPE),
    (dict(x=None), NULL), (dict(out=None), NULL),
    (dict(ld_out=3), SHAPE), (dict(tr=1, rows=8, ld_out=7), SHAPE),
    (dict(scale=None), ARG), (dict(ring=FAKE, H=4), ARG),
    (dict(scale=None, ring=FAKE, H=0), SHAPE), (dict(scale=None, ring=FAKE, H=5000), SHAPE),
    (dict(x=FAKE + 1), ARG), (dict(scale=FAKE + 2), ARG), (dict(amax=FAKE + 1), ARG),
    # extents beyond 2^62 bytes
    (dict(ld=1 << 61), SHAPE), (dict(ld_out=1 << 62), SHAPE), (dict(tr=1, ld_out=1 << 62), SHAPE),
])
def test_quantize_rejects(L, kw, status):
    assert q(L, **kw) == status
    assert L.fp8mi_last_error()


def test_quantize_dual_rejects(L):
    f = L.fp8_quantize_dual
    assert f(FAKE, 2, 4, 4, 4, 0, None, 4, FAKE, 4, FAKE, None, 0, None, None, None) == NULL
    assert f(FAKE, 2, 4, 4, 4, 0, FAKE, 4, None, 4, FAKE, None, 0, None, None, None) == NULL
    assert f(FAKE, 2, 4, 8, 8, 0, FAKE, 8, FAKE, 3, FAKE, None, 0, None, None, None) == SHAPE
    assert f(FAKE, 2, 4, 4, 4, 1, FAKE, 4, FAKE, 4, None, None, 0, None, None, None) == ARG


def test_amax_fold_rejects(L):
    assert L.fp8_amax_fold(None, 4, FAKE, 0, None) == NULL
    assert L.fp8_amax_fold(FAKE, 4, None, 0, None) == NULL
    assert L.fp8_amax_fold(FAKE, 4, FAKE, 9, None) == ENUM
    assert L.fp8_amax_fold(FAKE, 0, FAKE, 0, None) == SHAPE


def mm(L, a=FAKE, fa=0, lda=64, sa=0, b=FAKE, fb=0, ldb=64, sb=0, M=32, N=32, K=64, batch=1, sai=None, sbi=None,
       bias=None, bdt=2, c=FAKE, ldc=32, sc=0):
    return L.fp8_mm(a, fa, lda, sa, b, fb, ldb, sb, M, N, K, batch, sai, sbi, bias, bdt, c, ldc, sc, None)


@pytest.mark.parametrize("kw,status", [
    (dict(fa=2), ENUM), (dict(fb=-1), ENUM), (dict(bias=FAKE, bdt=5), ENUM),
    (dict(M=-1), SHAPE), (dict(K=-16), SHAPE), (dict(batch=-1), SHAPE),
    (dict(c=None), NULL), (dict(a=None), NULL), (dict(b=None), NULL),
    (dict(ldc=31), SHAPE), (dict(lda=48), SHAPE), (dict(ldb=32), SHAPE),
    (dict(batch=2, sc=32 * 31), STRIDE), (dict(sa=-64), STRIDE),
    (dict(c=FAKE + 1), ARG), (dict(bias=FAKE + 2, bdt=0), ARG),
    (dict(K=40, lda=64, ldb=64), UNSUP), (dict(lda=72, K=64), UNSUP), (dict(a=FAKE + 8), UNSUP),
    (dict(batch=2, sa=8, sc=32 * 32), UNSUP), (dict(batch=70000, sc=32 * 32), UNSUP),
])
def test_mm_rejects(L, kw, status):
    assert mm(L, **kw) == status


def test_mm_empty_is_noop(L):
    # no pointer is touched for an empty problem
    assert mm(L, M=0, a=None, b=None, c=None) == OK
    assert mm(L, N=0, a=None, b=None, c=None) == OK
    assert mm(L, batch=0, a=None, b=None, c=None) == OK


def test_binding_raises_without_gpu_on_bad_args():
    import torch
    x = torch.zeros(4, 4, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        fp8mi.fp8_quantize(x.t()[:, :3].t() if False else x.unsqueeze(0), fp8mi.E4M3, scale=None)
    with pytest.raises(ValueError):
        fp8mi.fp8_quantize(x, "e9m9", scale=None)


def test_binding_checks_tensor_arguments():
    """The binding refuses, before any library call, what only the tensors
    know: host tensors, wrong output shapes, non-code operands, wrong dtypes
    and bias lengths (host-side logic only: CPU tensors, nothing launched)."""
    import torch
    x = torch.zeros(4, 8, dtype=torch.bfloat16)
    one = torch.ones(1)
    codes = torch.zeros(4, 8, dtype=torch.uint8)
    with pytest.raises(ValueError, match="device"):                       # host tensors
        fp8mi.fp8_quantize(x, fp8mi.E4M3, scale=one)
    with pytest.raises(ValueError, match="shape"):                        # out of the wrong shape
        fp8mi.fp8_quantize(x, fp8mi.E4M3, out=torch.zeros(2, 8, dtype=torch.uint8), scale=one)
    with pytest.raises(ValueError, match="shape"):                        # transposed out is [cols, rows]
        fp8mi.fp8_quantize(x, fp8mi.E4M3, True, out=torch.zeros(4, 8, dtype=torch.uint8), scale=one)
    with pytest.raises(ValueError, match="shape"):
        fp8mi.fp8_quantize_dual(x, fp8mi.E4M3, out_t=torch.zeros(4, 8, dtype=torch.uint8), scale=one)
    with pytest.raises(ValueError, match="float32"):                      # scale of the wrong dtype
        fp8mi.fp8_quantize(x, fp8mi.E4M3, scale=torch.ones(1, dtype=torch.float64))
    with pytest.raises(ValueError, match="float32, float16 or bfloat16"):  # integer input
        fp8mi.fp8_quantize(x.to(torch.int16), fp8mi.E4M3, scale=one)
    with pytest.raises(ValueError, match="1-byte"):                       # bf16 passed as fp8 codes
        fp8mi.fp8_mm(x, codes)
    with pytest.raises(ValueError, match="shape"):                        # 2-D out for a batch of 3
        fp8mi.fp8_mm(codes.expand(3, 4, 8), codes, out=torch.zeros(4, 4, dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="bfloat16"):
        fp8mi.fp8_mm(codes, codes, out=torch.zeros(4, 4))
    with pytest.raises(ValueError, match="bias"):                         # bias of the wrong length
        fp8mi.fp8_mm(codes, codes, bias=torch.zeros(5))
    with pytest.raises(ValueError, match="device"):                       # valid shapes, host tensors
        fp8mi.fp8_mm(codes, codes, bias=torch.zeros(4))
    with pytest.raises(ValueError, match="bias_grad_out"):
        fp8mi.fp8_quantize_dual_bias_grad(x, fp8mi.E5M2, scale=one, bias_grad_out=torch.zeros(7, dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="out"):
        fp8mi.fp8_bias_grad(x, out=torch.zeros(8))


def test_bias_grad_workspace_bytes(L):
    f = L.fp8_bias_grad_workspace_bytes
    assert f(0, 16) == 0 and f(16, 0) == 0 and f(-1, 4) == 0
    assert f(1, 7) == 7 * 8                                 # one chunk of fp64 column sums
    assert f(128, 7) == 7 * 8 and f(129, 7) == 2 * 7 * 8    # 128-row chunks
    assert f(8192, 6912) == 64 * 6912 * 8


def test_bias_grad_rejects(L):
    f = L.fp8_bias_grad
    W = L.fp8_bias_grad_workspace_bytes(4, 4)
    assert f(FAKE, 0, 4, 4, 4, FAKE, FAKE, W, None) == UNSUP          # fp32 gradient
    assert f(FAKE, 9, 4, 4, 4, FAKE, FAKE, W, None) == ENUM
    assert f(FAKE, 2, -1, 4, 4, FAKE, FAKE, W, None) == SHAPE
    assert f(FAKE, 2, 4, 4, 3, FAKE, FAKE, W, None) == SHAPE
    assert f(None, 2, 4, 4, 4, FAKE, FAKE, W, None) == NULL
    assert f(FAKE, 2, 4, 4, 4, None, FAKE, W, None) == NULL
    assert f(FAKE + 1, 2, 4, 4, 4, FAKE, FAKE, W, None) == ARG
    assert f(FAKE, 2, 4, 4, 4, FAKE, None, W, None) == NULL          # workspace missing
    assert f(FAKE, 2, 4, 4, 4, FAKE, FAKE, W - 1, None) == ARG       # workspace too small
    assert f(FAKE, 2, 4, 4, 4, FAKE, FAKE + 4, W, None) == ARG       # workspace misaligned
    assert f(FAKE, 2, 4, 4, 1 << 61, FAKE, FAKE, W, None) == SHAPE  # rows x ld beyond 2^62 bytes
    assert f(None, 2, 4, 0, 4, None, None, 0, None) == OK            # no columns: no-op


def test_fused_dual_bias_grad_rejects(L):
    f = L.fp8_quantize_dual_bias_grad
    W = L.fp8_bias_grad_workspace_bytes(4, 4)
    ring, H = FAKE, 4

    def call(x=FAKE, dt=2, rows=4, cols=4, ld=4, fmt=0, o_row=FAKE, o_t=FAKE, scale=None, ring=ring, h=H,
             db=FAKE, ws=FAKE, wsb=W):
        return f(x, dt, rows, cols, ld, fmt, o_row, 4, o_t, 4, scale, ring, h, None, None, db, ws, wsb, None)

    assert call(dt=0) == UNSUP          # fp32 gradient
    assert call(dt=9) == ENUM
    assert call(db=None) == NULL        # bias gradient output missing
    assert call(ws=None) == NULL        # workspace missing
    assert call(wsb=W - 1) == ARG       # workspace too small
    assert call(db=FAKE + 1) == ARG     # misaligned bias gradient output
    assert call(fmt=5) == ENUM          # then the dual quantize's own checks
    assert call(o_t=None) == NULL
    assert call(rows=-1) == SHAPE


def test_noalloc_dual_bias_grad_rejects(L):
    """The allocation-free fused call checks everything the workspace form
    does, and rejects a gradient whose column sums exceed the library's
    scratch (FP8MI_NOALLOC_SCRATCH_BYTES) -- all before any HIP call."""
    f = L.fp8_quantize_dual_bias_grad_noalloc
    ring, H = FAKE, 4

    def call(x=FAKE, dt=2, rows=4, cols=4, ld=None, fmt=0, o_row=FAKE, o_t=FAKE, scale=None, ring=ring, h=H,
             db=FAKE):
        ld = cols if ld is None else ld
        return f(x, dt, rows, cols, ld, fmt, o_row, cols, o_t, rows, scale, ring, h, None, None, db, None)

    assert call(dt=0) == UNSUP          # fp32 gradient
    assert call(dt=9) == ENUM
    assert call(db=None) == NULL
    assert call(db=FAKE + 1) == ARG
    assert call(fmt=5) == ENUM
    assert call(o_t=None) == NULL
    assert call(rows=-1) == SHAPE
    assert call(scale=FAKE) == ARG      # both scale and ring
    cap = 8 * 1024 * 1024
    header = open(os.path.join(ROOT, "include", "fp8mi.h")).read()
    assert re.search(r"#define FP8MI_NOALLOC_SCRATCH_BYTES\s+\(8 \* 1024 \* 1024\)", header)
    # ceil(rows / 128) * cols * 8 bytes: 2 tiles x 524288 columns fit exactly, one more column does not
    assert L.fp8_bias_grad_workspace_bytes(256, 524288) == cap
    assert call(rows=256, cols=524289) == UNSUP
    assert b"scratch" in L.fp8mi_last_error()


def test_stream_reference_rejects(L):
    f = L.fp8mi_stream_reference
    assert f(FAKE, 40, FAKE * 4, 20, None) == ARG      # src bytes not a multiple of 16
    assert f(FAKE, 48, FAKE * 4, 16, None) == ARG      # dst neither src's size nor its half
    assert f(None, 48, FAKE * 4, 48, None) == NULL
    assert f(FAKE + 8, 48, FAKE * 4, 48, None) == ARG  # misaligned
    assert f(FAKE, 64, FAKE + 32, 64, None) == ARG     # overlapping
    assert f(None, 0, None, 0, None) == OK             # nothing to move


def test_ring_seed_rejects(L):
    f = L.fp8_ring_seed
    assert f(None, 4, FAKE, 0, None) == NULL
    assert f(FAKE, 4, None, 0, None) == NULL
    assert f(FAKE, 4, FAKE, 3, None) == ENUM
    assert f(FAKE, 0, FAKE, 0, None) == SHAPE
    assert f(FAKE + 2, 4, FAKE, 0, None) == ARG


def test_quantize_dynamic_rejects(L):
    f = L.fp8_quantize_dynamic
    W = 4096  # FP8MI_DYNAMIC_WORKSPACE_BYTES
    header = open(os.path.join(ROOT, "include", "fp8mi.h")).read()
    assert re.search(r"#define FP8MI_DYNAMIC_WORKSPACE_BYTES\s+4096\b", header)

    def call(x=FAKE, dt=2, rows=4, cols=4, ld=4, fmt=0, layout=0, o_row=FAKE, ld_r=4, o_t=FAKE, ld_t=4,
             sinv=None, amax=None, ws=FAKE, wsb=W):
        return f(x, dt, rows, cols, ld, fmt, layout, o_row, ld_r, o_t, ld_t, sinv, amax, ws, wsb, None)

    assert call(layout=3) == ENUM
    assert call(layout=-1) == ENUM
    assert call(dt=7) == ENUM
    assert call(fmt=2) == ENUM
    assert call(rows=-1) == SHAPE
    assert call(ld=3) == SHAPE
    assert call(x=None) == NULL
    assert call(x=FAKE + 1) == ARG          # bf16 input not 2-byte aligned
    assert call(o_row=None) == NULL          # row layout needs out_row
    assert call(layout=1, o_t=None) == NULL  # transposed layout needs out_t
    assert call(layout=2, o_row=None) == NULL
    assert call(layout=1, ld_t=3) == SHAPE
    assert call(ld_r=3) == SHAPE
    assert call(sinv=FAKE + 2) == ARG
    assert call(amax=FAKE + 1) == ARG
    assert call(ws=None) == NULL             # workspace missing, even for an empty tensor
    assert call(ws=None, rows=0) == NULL
    assert call(wsb=W - 4) == ARG            # workspace too small
    assert call(ws=FAKE + 2) == ARG          # workspace not 4-byte aligned


def test_mm_ex_rejects(L):
    f = L.fp8_mm_ex

    def call(a=FAKE, fa=0, lda=32, sa=0, b=FAKE, fb=0, ldb=32, sb=0, M=4, N=4, K=32, batch=1, lay=0, bias=None,
             bdt=0, bsc=None, c=FAKE, cdt=2, ldc=4, sc=16, cscale=None, cring=None, h=0, sinv=None, amax=None):
        return f(a, fa, lda, sa, b, fb, ldb, sb, M, N, K, batch, lay, None, None, bias, bdt, bsc, c, cdt, ldc, sc,
                 cscale, cring, h, sinv, amax, None)

    assert call(fa=2) == ENUM
    assert call(cdt=0) == ENUM                        # fp32 output is not offered
    assert call(cdt=5) == ENUM
    assert call(bias=FAKE, bdt=9) == ENUM
    assert call(bias=FAKE, bdt=3) == NULL             # fp8 bias without its scale
    assert call(bias=FAKE, bdt=2, bsc=FAKE) == ARG    # a scale with a raw bias
    assert call(bsc=FAKE) == ARG                      # a scale without a bias
    assert call(cscale=FAKE) == ARG                   # output scale with a bf16 output
    assert call(amax=FAKE) == ARG
    assert call(cdt=3) == ARG                         # fp8 output: neither scale nor ring
    assert call(cdt=3, cscale=FAKE, cring=FAKE, h=4) == ARG   # ... or both
    assert call(cdt=4, cring=FAKE, h=0) == SHAPE      # ring with a bad history length
    assert call(cdt=3, cscale=FAKE + 2) == ARG        # misaligned fp32 scalar
    assert call(cdt=3, cscale=FAKE, M=-1) == SHAPE
    assert call(cdt=3, cscale=FAKE, c=None) == NULL
    assert call(cdt=3, cscale=FAKE, ldc=3) == SHAPE
    assert call(cdt=3, cscale=FAKE, K=24, lda=24, ldb=24) == UNSUP
    # layout tags
    assert call(lay=4) == ENUM
    assert call(lay=-1) == ENUM
    # an fp8 output takes K-major operands under the same rules as bf16
    assert call(lay=1, cdt=3, cscale=FAKE, M=64, lda=48) == SHAPE
    assert call(lay=1, cdt=3, cscale=FAKE, M=64, lda=72) == UNSUP
    assert call(lay=1, M=64, lda=48) == SHAPE         # K-major A: lda must cover M
    assert call(lay=2, N=64, ldb=48) == SHAPE
    assert call(lay=1, M=64, lda=72) == UNSUP         # lda % 16
    # extents beyond 2^62 bytes and grids beyond the launch limits are refused
    big = 1 << 61
    assert call(lda=big) == SHAPE                     # M x lda
    assert call(ldc=big) == SHAPE                     # M x ldc x 2 bytes
    assert call(batch=4, sa=big) == SHAPE             # batch x stride_a
    assert call(lay=1, M=64, lda=big - big % 16) == SHAPE   # K-major A: K x lda
    assert call(M=1 << 20, N=1 << 24, ldc=1 << 24) == UNSUP  # 2^32 tiles of 64 x 64
    assert call(M=1 << 16, N=1 << 25, ldc=1 << 25) == UNSUP  # 2^29 tiles of 64 x 64
    # the plain fp8_mm refuses an fp8 bias type (it has no bias scale)
    assert L.fp8_mm(FAKE, 0, 32, 0, FAKE, 0, 32, 0, 4, 4, 32, 1, None, None, FAKE, 3, FAKE, 4, 16, None) == ENUM


def test_binding_maps_transposed_views_to_layout_tags():
    """The binding reads an operand that is a transposed view (unit stride
    along its rows) K-major, with the storage's row length as leading
    dimension, and refuses a K-major view whose storage lacks the K full rows
    the library reads; host-side logic only (CPU tensors, no library call)."""
    import torch
    from fp8_tensor_scaled_quantize_amd import _operand_ld
    a = torch.zeros((64, 96), dtype=torch.uint8)                      # [M, K] row-major
    assert _operand_ld(a.unsqueeze(0), "a") == (96, False)
    at = torch.zeros((96, 80), dtype=torch.uint8)                     # [K, M + pad] storage
    v = at[:, :64].t()                                                 # [M, K] view, unit stride along M
    assert _operand_ld(v.unsqueeze(0), "a") == (80, True)
    b3 = torch.zeros((3, 96, 48), dtype=torch.uint8).transpose(1, 2)  # batched K-major view
    assert _operand_ld(b3, "b") == (48, True)
    with pytest.raises(ValueError):
        _operand_ld(torch.zeros((64, 96), dtype=torch.uint8)[:, ::2].unsqueeze(0), "a")  # no unit stride
    flat = torch.zeros(96 * 80 - 8, dtype=torch.uint8)                # last row short of its padding
    short = torch.as_strided(flat, (64, 96), (1, 80))
    with pytest.raises(ValueError):
        _operand_ld(short.unsqueeze(0), "a")
