"""libfp8mi driven from C: tests/c_abi_demo.c uses only the HIP runtime and
include/fp8mi.h (no Python, no torch) to quantize X with a ring, quantize W
into both layouts at an explicit scale, multiply the codes, fold X's amax once
more through fp8_amax_fold, and make one rejected call.

* CPU: the program compiles and links as strict C11 (-Wall -Wextra -pedantic
  -Werror) against the header and the library -- the header is plain C.
* GPU: its outputs match the oracle: codes, scale snapshots, amaxes and ring
  words bit-exact; the GEMM within the stated bound plus the fp8-MFMA group
  term; the rejected call returns FP8MI_ERR_ENUM with an error text.
X bf16 [96, 256] N(0,1), W bf16 [80, 256] N(0,0.02), a 4-entry ring starting
at scale 112, W's scale fmt_max / amax(W).
"""
import os
import shutil
import subprocess

import numpy as np
import pytest

import oracle as O
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "c_abi_demo.c")
PKG = os.path.join(ROOT, "fp8_tensor_scaled_quantize_amd")
LIB = os.path.join(PKG, "libfp8mi.so")
ROCM = "/opt/rocm"
H, RING_SCRATCH = 4, 1024
ROWS, COLS, N = 96, 256, 80


def compile_demo(out_dir) -> str:
    if shutil.which("gcc") is None or not os.path.isdir(os.path.join(ROCM, "include", "hip")):
        pytest.skip("gcc or the HIP headers are not available")
    if not os.path.exists(LIB):
        pytest.skip("libfp8mi.so not built")
    exe = os.path.join(str(out_dir), "c_abi_demo")
    cmd = ["gcc", "-std=c11", "-O1", "-Wall", "-Wextra", "-pedantic", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-isystem", f"{ROCM}/include", f"-I{ROOT}/include", SRC, f"-L{PKG}", "-lfp8mi", f"-L{ROCM}/lib", "-lamdhip64",
           f"-Wl,-rpath,{PKG}", "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return exe


def test_c_program_compiles_against_the_abi(tmp_path):
    assert os.access(compile_demo(tmp_path), os.X_OK)


@pytest.mark.gpu
def test_c_program_matches_the_oracle(tmp_path):
    exe = compile_demo(tmp_path)
    x = synth.gaussian((ROWS, COLS), 1.0, "bf16", 9500, 0)
    w = synth.gaussian((N, COLS), 0.02, "bf16", 9500, 1)
    s0 = np.float32(112.0)
    sw = np.float32(O.FMT_MAX[O.E4M3] / O.amax(O.widen_to_f32(w, "bf16")))
    src, dst = tmp_path / "in.bin", tmp_path / "out.bin"
    with open(src, "wb") as f:
        f.write(np.array([ROWS, COLS, N], np.int64).tobytes() + np.array([s0, sw], np.float32).tobytes())
        f.write(np.ascontiguousarray(x).astype(np.uint16).tobytes() + np.ascontiguousarray(w).astype(np.uint16).tobytes())
    r = subprocess.run([exe, str(src), str(dst)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    raw = open(dst, "rb").read()
    bad, bad_len = np.frombuffer(raw[:8], np.int32)
    sx, ax, swi, aw = np.frombuffer(raw[8:24], np.float32)
    off = 24
    ring = np.frombuffer(raw[off:off + 4 * (H + 4 + RING_SCRATCH)], np.uint32)
    off += 4 * (H + 4 + RING_SCRATCH)
    codes = np.frombuffer(raw[off:off + ROWS * COLS + 2 * N * COLS], np.uint8)
    off += ROWS * COLS + 2 * N * COLS
    y = np.frombuffer(raw[off:], np.uint16).reshape(ROWS, N)
    xq = codes[:ROWS * COLS].reshape(ROWS, COLS)
    wq = codes[ROWS * COLS:ROWS * COLS + N * COLS].reshape(N, COLS)
    wqt = codes[ROWS * COLS + N * COLS:].reshape(COLS, N)

    qx = O.quantize(x, "bf16", O.E4M3, ring=O.Ring.new(H, s0))
    ring_ref = O.fold(qx["ring"], qx["amax"], O.E4M3)
    qw = O.quantize(w, "bf16", O.E4M3, scale=sw)
    assert bad == 2 and bad_len > 0                              # FP8MI_ERR_ENUM with a message
    assert np.array_equal(xq, qx["codes"])
    assert np.array_equal(wq, qw["codes"]) and np.array_equal(wqt, qw["codes_t"])
    for got, want in ((sx, qx["scale_inv"]), (ax, qx["amax"]), (swi, qw["scale_inv"]), (aw, qw["amax"])):
        assert np.float32(got).view(np.uint32) == np.float32(want).view(np.uint32)
    assert np.array_equal(ring[:H + 4], ring_ref.words()) and not ring[H + 4:].any()
    from tests.gpu_util import check
    check(y, qx["codes"], O.E4M3, qw["codes"], O.E4M3, qx["scale_inv"], qw["scale_inv"], None, tag="c demo")
