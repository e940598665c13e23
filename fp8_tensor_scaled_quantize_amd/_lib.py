"""ctypes loader of libfp8mi.so; the argument types mirror include/fp8mi.h."""
from __future__ import annotations

import ctypes as C
import os

_LIB = None
LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfp8mi.so")

_P, _I, _I64, _I32 = C.c_void_p, C.c_int, C.c_int64, C.c_int32

SIGNATURES = {
    "fp8_quantize": (C.c_int, [_P, _I, _I64, _I64, _I64, _I, _I, _P, _I64, _P, _P, _I32, _P, _P, _P]),
    "fp8_quantize_dual": (C.c_int, [_P, _I, _I64, _I64, _I64, _I, _P, _I64, _P, _I64, _P, _P, _I32, _P, _P, _P]),
    "fp8_quantize_dual_bias_grad": (C.c_int, [_P, _I, _I64, _I64, _I64, _I, _P, _I64, _P, _I64, _P, _P, _I32, _P,
                                              _P, _P, _P, C.c_size_t, _P]),
    "fp8_quantize_dual_bias_grad_noalloc": (C.c_int, [_P, _I, _I64, _I64, _I64, _I, _P, _I64, _P, _I64, _P, _P,
                                                      _I32, _P, _P, _P, _P]),
    "fp8_quantize_dynamic": (C.c_int, [_P, _I, _I64, _I64, _I64, _I, _I, _P, _I64, _P, _I64, _P, _P, _P,
                                       C.c_size_t, _P]),
    "fp8_amax_fold": (C.c_int, [_P, _I32, _P, _I, _P]),
    "fp8_mm": (C.c_int, [_P, _I, _I64, _I64, _P, _I, _I64, _I64, _I64, _I64, _I64, _I64, _P, _P, _P, _I, _P,
                         _I64, _I64, _P]),
    "fp8_mm_ex": (C.c_int, [_P, _I, _I64, _I64, _P, _I, _I64, _I64, _I64, _I64, _I64, _I64, _I, _P, _P, _P, _I, _P,
                            _P, _I, _I64, _I64, _P, _P, _I32, _P, _P, _P]),
    "fp8_bias_grad": (C.c_int, [_P, _I, _I64, _I64, _I64, _P, _P, C.c_size_t, _P]),
    "fp8_bias_grad_workspace_bytes": (C.c_size_t, [_I64, _I64]),
    "fp8_ring_seed": (C.c_int, [_P, _I32, _P, _I, _P]),
    "fp8mi_stream_reference": (C.c_int, [_P, _I64, _P, _I64, _P]),
    "fp8mi_status_string": (C.c_char_p, [_I]),
    "fp8mi_last_error": (C.c_char_p, []),
    "fp8mi_version": (C.c_char_p, []),
}


def lib():
    """The loaded library; raises if it has not been built (no fallback)."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m fp8_tensor_scaled_quantize_amd.build` (or __graft_entry__.build())")
        h = C.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(h, name)
            f.restype, f.argtypes = res, args
        _LIB = h
    return _LIB
