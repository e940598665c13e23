"""The library's tuning overrides (FP8MI_MM_TILE, FP8MI_Q_BPC,
FP8MI_AMAX_BPC) are read once per process: a child process with malformed or
out-of-range values (which the library ignores) and ones with a valid forced
GEMM tile (128 x 128, the deep-pipeline 64 x 64, and 256 x 256 where the
default is the mixed grid of 256 x 256 tiles and a 128 x 256 band) must
produce, bit for bit, what this process produces with the defaults -- a persistent-grid dual quantize (bf16 8192x6912, E5M2, ring), a
current-scaling quantize (bf16 8192x1536), a 2048x1536x6912 GEMM with bias
and an 8192x6912x1536 GEMM with bias -- bf16 out with A row-major and
K-major, and E4M3 out with its ring (the result does not depend on the tile
shape: every output's K sum runs in the same MFMA order)."""
import os
import subprocess
import sys

import pytest
import torch

pytestmark = pytest.mark.gpu

fp8mi = pytest.importorskip("fp8_tensor_scaled_quantize_amd")
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r'''
import sys, torch
sys.path.insert(0, sys.argv[1])
import fp8_tensor_scaled_quantize_amd as fp8mi
import synth
dev = torch.device("cuda:0")
dy = synth.device_gaussian((8192, 6912), 1e-3, torch.bfloat16, 9800)
x = synth.device_gaussian((8192, 1536), 1.0, torch.bfloat16, 9801)
ring = fp8mi.new_ring(16, 1.0, dev)
q, qt = fp8mi.fp8_quantize_dual(dy, fp8mi.E5M2, ring=ring)
d, _ = fp8mi.fp8_quantize_dynamic(x, fp8mi.E4M3)
s = torch.full((1,), 4096.0, device=dev)
a = fp8mi.fp8_quantize(dy[:2048].contiguous(), fp8mi.E4M3, scale=s)          # [2048, 6912]
b = fp8mi.fp8_quantize(dy[4096:5632].contiguous(), fp8mi.E4M3, scale=s)      # [1536, 6912]
bias = synth.device_gaussian((1536,), 0.1, torch.bfloat16, 9802)
y = fp8mi.fp8_mm(a, b, fp8mi.E4M3, fp8mi.E4M3, None, None, bias)
# 8192 x 6912 x 1536: four rounds of 256 x 256 tiles by default
a2 = fp8mi.fp8_quantize(x, fp8mi.E4M3, scale=s)                          # [8192, 1536]
b2 = fp8mi.fp8_quantize(dy.t().contiguous()[:, :1536].contiguous(), fp8mi.E4M3, scale=s)  # [6912, 1536]
bias2 = synth.device_gaussian((6912,), 0.1, torch.bfloat16, 9803)
y2 = fp8mi.fp8_mm(a2, b2, fp8mi.E4M3, fp8mi.E4M3, None, None, bias2)
# the same shape through the quantizing epilogue (ring) and with A given K-major
ring_y = fp8mi.new_ring(16, 1.0, dev)
q2 = fp8mi.fp8_mm_ex(a2, b2, fp8mi.E4M3, fp8mi.E4M3, None, None, bias2, out_fmt=fp8mi.E4M3, out_ring=ring_y)
y2k = fp8mi.fp8_mm(a2.t().contiguous().t(), b2, fp8mi.E4M3, fp8mi.E4M3, None, None, bias2)
torch.cuda.synchronize()
torch.save({"q": q.cpu(), "qt": qt.cpu(), "ring": ring.cpu(), "d": d.cpu(), "y": y.cpu().view(torch.int16),
            "y2": y2.cpu().view(torch.int16), "q2": q2.cpu(), "ring_y": ring_y.cpu(),
            "y2k": y2k.cpu().view(torch.int16)}, sys.argv[2])
'''


def run_child(tmp_path, tag, env_extra):
    out = tmp_path / f"{tag}.pt"
    env = {k: v for k, v in os.environ.items() if not k.startswith("FP8MI_")}
    env.update(env_extra)
    r = subprocess.run([sys.executable, "-c", CHILD, ROOT, str(out)], env=env, capture_output=True, text=True,
                       timeout=180)
    assert r.returncode == 0, r.stderr[-2000:]
    return torch.load(out, weights_only=True)


def test_invalid_overrides_are_ignored_and_a_forced_tile_changes_nothing(tmp_path):
    ref = run_child(tmp_path, "default", {})
    bad = run_child(tmp_path, "bad", {"FP8MI_MM_TILE": "abc", "FP8MI_Q_BPC": "0", "FP8MI_AMAX_BPC": "-3"})
    tile = run_child(tmp_path, "tile1", {"FP8MI_MM_TILE": "1", "FP8MI_Q_BPC": "2"})
    deep64 = run_child(tmp_path, "tile6", {"FP8MI_MM_TILE": "6"})
    # 8192 x 6912 x 1536 takes the mixed grid by default (768 tiles of 256 x
    # 256 + a 128 x 256 band); forced tile 0 runs it as four rounds of 256 x 256
    big = run_child(tmp_path, "tile0", {"FP8MI_MM_TILE": "0"})
    for other, tag in ((bad, "invalid overrides"), (tile, "forced tile 1, 2 workgroups per CU"),
                       (deep64, "forced deep-pipeline 64x64"), (big, "forced 256x256 (no band)")):
        for k in ref:
            assert torch.equal(other[k], ref[k]), (tag, k)
