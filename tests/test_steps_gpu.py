"""Delayed-scaling steps through the library against the oracle.

* tiny config: X bf16 [64,256] N(0,1) fresh each step, W [256,256] N(0,0.02),
  bias [256] N(0,0.1); E4M3 row-layout quantize, 4-entry history; one seeded
  step and 3 delayed steps.  Codes, scale snapshots and ring words bit-exact,
  Y within the GEMM bound.
* checkpoint / resume: a ring is a plain device buffer; 4 + (copy, restore) +
  4 steps equal 8 straight steps, bit for bit.
* full training step: x bf16 [4,2048,1536] N(0,1) and dY [8192,6912]
  N(0,1e-3) fresh each step, W [6912,1536] N(0,0.02) and bias [6912] N(0,0.1)
  fixed; E4M3 x/W, E5M2 dY, 16-entry histories, 32 steps.  Ring words and
  scale snapshots bit-exact every step; codes bit-exact on seeded row and
  column samples every step; Y and dX on sampled rows every step, dW on
  sampled rows at steps 0, 1, 15, 31; the bias gradient in full every step.
"""
import numpy as np
import pytest
import torch

import oracle as O
import synth
from tests.gpu_util import DEV, as_bits, check, np_bf16_bits, np_codes, ring_from_oracle, ring_state_words

pytestmark = pytest.mark.gpu

fp8mi = pytest.importorskip("fp8_tensor_scaled_quantize_amd")
from fp8_tensor_scaled_quantize_amd.linear import Fp8Linear  # noqa: E402
from tests.test_mm_fp8_out_gpu import check_amax, check_codes, y_band  # noqa: E402


def dev_bf16(bits):
    return synth.to_torch(bits, "bf16").to(DEV)


def f32_words(t):
    return t.cpu().numpy().view(np.uint32)


def tiny_inputs(steps):
    xs = [synth.gaussian((64, 256), 1.0, "bf16", 1, synth.T_X, t) for t in range(steps)]
    w = synth.gaussian((256, 256), 0.02, "bf16", 1, synth.T_W, 0)
    b = synth.gaussian((256,), 0.1, "bf16", 1, synth.T_BIAS, 0)
    return xs, w, b


def test_tiny_delayed_scaling_steps():
    xs, w, b = tiny_inputs(4)
    xs[2] = synth.f32_to_bf16_bits(O.widen_to_f32(xs[2], "bf16") * np.float32(10.0))  # amax jumps 10x
    rx, rw = O.seed_ring(4, xs[0], "bf16", O.E4M3), O.seed_ring(4, w, "bf16", O.E4M3)
    layer = Fp8Linear(dev_bf16(w), dev_bf16(b), hist_len=4)
    layer.seed(dev_bf16(xs[0]))
    torch.cuda.synchronize()
    assert np.array_equal(ring_state_words(layer.ring_x), rx.words())
    assert np.array_equal(ring_state_words(layer.ring_w), rw.words())
    for t in range(4):
        ref = O.linear_forward(xs[t], w, b, rx, rw)
        y = layer.forward(dev_bf16(xs[t]), save_for_backward=False)
        xq, wq = layer.last_codes
        torch.cuda.synchronize()
        assert np.array_equal(np_codes(xq), ref["qx"]["codes"]), t
        assert np.array_equal(np_codes(wq), ref["qw"]["codes"]), t
        si = f32_words(layer.scale_inv)
        assert si[0] == as_bits(ref["qx"]["scale_inv"]) and si[1] == as_bits(ref["qw"]["scale_inv"]), t
        rx, rw = ref["qx"]["ring"], ref["qw"]["ring"]
        assert np.array_equal(ring_state_words(layer.ring_x), rx.words()), t
        assert np.array_equal(ring_state_words(layer.ring_w), rw.words()), t
        bias = O.widen_to_f32(b, "bf16").astype(np.float64)
        check(np_bf16_bits(y), ref["qx"]["codes"], O.E4M3, ref["qw"]["codes"], O.E4M3,
              ref["qx"]["scale_inv"], ref["qw"]["scale_inv"], bias, tag=f"tiny step {t}")
    # the step after the jump quantized with the stale (delayed) scale and the
    # GEMM dequantised with that same snapshot: no leak of the scale ratio
    assert rx.scale < np.float32(448.0) / O.amax(O.widen_to_f32(xs[1], "bf16"))


def test_checkpoint_resume_rings():
    xs, w, b = tiny_inputs(8)
    straight = Fp8Linear(dev_bf16(w), dev_bf16(b), hist_len=3)
    straight.seed(dev_bf16(xs[0]))
    ys = [straight.forward(dev_bf16(x), save_for_backward=False).clone() for x in xs]

    first = Fp8Linear(dev_bf16(w), dev_bf16(b), hist_len=3)
    first.seed(dev_bf16(xs[0]))
    ys2 = [first.forward(dev_bf16(x), save_for_backward=False).clone() for x in xs[:4]]
    saved = [first.ring_x.cpu().clone(), first.ring_w.cpu().clone()]       # checkpoint = byte copy
    resumed = Fp8Linear(dev_bf16(w), dev_bf16(b), hist_len=3)
    resumed.ring_x.copy_(saved[0].to(DEV))
    resumed.ring_w.copy_(saved[1].to(DEV))
    ys2 += [resumed.forward(dev_bf16(x), save_for_backward=False).clone() for x in xs[4:]]
    torch.cuda.synchronize()
    for a, c in zip(ys, ys2):
        assert torch.equal(a, c)
    assert torch.equal(straight.ring_x, resumed.ring_x) and torch.equal(straight.ring_w, resumed.ring_w)


@pytest.mark.timeout(900)
def test_full_training_step_32_steps():
    M, K, N, H, STEPS = 8192, 1536, 6912, 16, 32
    w = synth.gaussian((N, K), 0.02, "bf16", 5, synth.T_W, 0)
    b = synth.gaussian((N,), 0.1, "bf16", 5, synth.T_BIAS, 0)
    wf, bias = O.widen_to_f32(w, "bf16"), O.widen_to_f32(b, "bf16").astype(np.float64)
    layer = Fp8Linear(dev_bf16(w), dev_bf16(b), hist_len=H)

    def x_of(t):
        return synth.gaussian((M, K), 1.0, "bf16", 5, synth.T_X, t)

    def dy_of(t):
        return synth.gaussian((M, N), 1e-3, "bf16", 5, synth.T_DY, t)

    x0, dy0 = x_of(0), dy_of(0)
    rx = O.seed_ring(H, x0, "bf16", O.E4M3)
    rw = O.seed_ring(H, w, "bf16", O.E4M3)
    rg = O.seed_ring(H, dy0, "bf16", O.E5M2)
    layer.seed(dev_bf16(x0).view(4, 2048, K), dev_bf16(dy0))
    w_codes = {}

    for t in range(STEPS):
        x = x0 if t == 0 else x_of(t)
        dy = dy0 if t == 0 else dy_of(t)
        y = layer.forward(dev_bf16(x).view(4, 2048, K))
        dx, dw, db = layer.backward(dev_bf16(dy))
        torch.cuda.synchronize()
        xf, gf = O.widen_to_f32(x, "bf16"), O.widen_to_f32(dy, "bf16")
        sx, sw, sg = rx.scale, rw.scale, rg.scale
        rx = O.fold(rx, O.amax(xf), O.E4M3)
        rw = O.fold(rw, O.amax(wf), O.E4M3)
        rg = O.fold(rg, O.amax(gf), O.E5M2)
        for ring, ref in ((layer.ring_x, rx), (layer.ring_w, rw), (layer.ring_g, rg)):
            assert np.array_equal(ring_state_words(ring), ref.words()), t
        si = f32_words(layer.scale_inv)
        assert list(si) == [as_bits(O.scale_inv(s)) for s in (sx, sw, sg)], t

        # codes on seeded samples of rows (row layout) and columns (transposed layout)
        rs = np.sort(synth.rng(6, t, 0).choice(M, 48, replace=False))
        cs_k = np.sort(synth.rng(6, t, 1).choice(K, 24, replace=False))
        cs_n = np.sort(synth.rng(6, t, 2).choice(N, 24, replace=False))
        xq_rows = O.encode(O.scaled_values(xf[rs], sx), O.E4M3)
        gq_rows = O.encode(O.scaled_values(gf[rs], sg), O.E5M2)
        xq, wq = layer.last_codes
        gq, gq_t = layer.last_grad_codes
        xq_t_dev, wq_t_dev, _ = layer._saved
        assert np.array_equal(np_codes(xq[rs]), xq_rows), t
        assert np.array_equal(np_codes(gq[rs]), gq_rows), t
        assert np.array_equal(np_codes(xq_t_dev[cs_k]), O.encode(O.scaled_values(xf[:, cs_k], sx), O.E4M3).T), t
        assert np.array_equal(np_codes(gq_t[cs_n]), O.encode(O.scaled_values(gf[:, cs_n], sg), O.E5M2).T), t
        key = as_bits(sw)
        if key not in w_codes:
            w_codes[key] = O.encode(O.scaled_values(wf, sw), O.E4M3)
            assert np.array_equal(np_codes(wq), w_codes[key]), t
            assert np.array_equal(np_codes(wq_t_dev), w_codes[key].T), t
        wc = w_codes[key]

        # GEMMs on sampled rows: each sampled output row is exact in the oracle
        y2 = np_bf16_bits(y.reshape(M, N))
        check(y2[rs], xq_rows, O.E4M3, wc, O.E4M3, O.scale_inv(sx), O.scale_inv(sw), bias, tag=f"Y step {t}")
        check(np_bf16_bits(dx.reshape(M, K))[rs], gq_rows, O.E5M2, np.ascontiguousarray(wc.T), O.E4M3,
              O.scale_inv(sg), O.scale_inv(sw), None, tag=f"dX step {t}")
        if t in (0, 1, 15, 31):
            xq_t_full = np.ascontiguousarray(O.encode(O.scaled_values(xf, sx), O.E4M3).T)
            ns = np.sort(synth.rng(6, t, 3).choice(N, 24, replace=False))
            gq_t_rows = np.ascontiguousarray(O.encode(O.scaled_values(gf[:, ns], sg), O.E5M2).T)
            check(np_bf16_bits(dw)[ns], gq_t_rows, O.E5M2, xq_t_full, O.E4M3, O.scale_inv(sg), O.scale_inv(sx),
                  None, tag=f"dW step {t}")
        # bias gradient: full
        db_ref, db_mag = O.grad_bias(dy)
        db_gpu = np_bf16_bits(db)
        assert O.within_tolerance(db_gpu, db_ref, db_mag).all(), t
        assert (db_gpu == db_ref).mean() > 0.999, t


def test_tiny_dynamic_scaling_steps():
    """The layer under the dynamic recipe: every step's scales come from that
    step's own tensors (an amax jump is followed at once), codes and scale
    snapshots bit-exact, Y / dX / dW within the GEMM bound, db exact."""
    xs, w, b = tiny_inputs(4)
    xs[2] = synth.f32_to_bf16_bits(O.widen_to_f32(xs[2], "bf16") * np.float32(10.0))
    dys = [synth.gaussian((64, 256), 1e-3, "bf16", 1, synth.T_DY, t) for t in range(4)]
    layer = Fp8Linear(dev_bf16(w), dev_bf16(b), dynamic=True)
    assert layer.ring_x is None
    layer.seed(dev_bf16(xs[0]))  # no-op under dynamic scaling
    bias = O.widen_to_f32(b, "bf16").astype(np.float64)
    qw = O.quantize_dynamic(w, "bf16", O.E4M3)
    for t in range(4):
        qx = O.quantize_dynamic(xs[t], "bf16", O.E4M3)
        qg = O.quantize_dynamic(dys[t], "bf16", O.E5M2)
        y = layer.forward(dev_bf16(xs[t]))
        dx, dw, db = layer.backward(dev_bf16(dys[t]))
        torch.cuda.synchronize()
        xq, wq = layer.last_codes
        gq, gq_t = layer.last_grad_codes
        assert np.array_equal(np_codes(xq), qx["codes"]), t
        assert np.array_equal(np_codes(wq), qw["codes"]), t
        assert np.array_equal(np_codes(gq), qg["codes"]) and np.array_equal(np_codes(gq_t), qg["codes_t"]), t
        si = f32_words(layer.scale_inv)
        assert list(si) == [as_bits(qx["scale_inv"]), as_bits(qw["scale_inv"]), as_bits(qg["scale_inv"])], t
        check(np_bf16_bits(y), qx["codes"], O.E4M3, qw["codes"], O.E4M3, qx["scale_inv"], qw["scale_inv"], bias,
              tag=f"dyn Y {t}")
        check(np_bf16_bits(dx), qg["codes"], O.E5M2, qw["codes_t"], O.E4M3, qg["scale_inv"], qw["scale_inv"], None,
              tag=f"dyn dX {t}")
        check(np_bf16_bits(dw), qg["codes_t"], O.E5M2, qx["codes_t"], O.E4M3, qg["scale_inv"], qx["scale_inv"],
              None, tag=f"dyn dW {t}")
        assert np.array_equal(np_bf16_bits(db), O.grad_bias(dys[t])[0]), t
    # the step with the 10x amax used a 10x smaller scale at once (no delay)
    assert O.quantize_dynamic(xs[2], "bf16", O.E4M3)["scale_inv"] > O.quantize_dynamic(xs[1], "bf16",
                                                                                        O.E4M3)["scale_inv"]


def test_full_shape_dynamic_step():
    """Two dynamic steps at the training shape (x [4,2048,1536], W
    [6912,1536], dY [8192,6912]): scale snapshots exact, codes and GEMM rows
    on seeded samples."""
    M, K, N = 8192, 1536, 6912
    w = synth.gaussian((N, K), 0.02, "bf16", 7, synth.T_W, 0)
    b = synth.gaussian((N,), 0.1, "bf16", 7, synth.T_BIAS, 0)
    wf, bias = O.widen_to_f32(w, "bf16"), O.widen_to_f32(b, "bf16").astype(np.float64)
    layer = Fp8Linear(dev_bf16(w), dev_bf16(b), dynamic=True)
    sw = O.next_scale(np.array([O.amax(wf)]), O.E4M3)
    wc = O.encode(O.scaled_values(wf, sw), O.E4M3)
    for t in range(2):
        x = synth.gaussian((M, K), 1.0, "bf16", 7, synth.T_X, t)
        dy = synth.gaussian((M, N), 1e-3 * (1 + 9 * t), "bf16", 7, synth.T_DY, t)
        y = layer.forward(dev_bf16(x).view(4, 2048, K))
        dx, dw, db = layer.backward(dev_bf16(dy))
        torch.cuda.synchronize()
        xf, gf = O.widen_to_f32(x, "bf16"), O.widen_to_f32(dy, "bf16")
        sx = O.next_scale(np.array([O.amax(xf)]), O.E4M3)
        sg = O.next_scale(np.array([O.amax(gf)]), O.E5M2)
        si = f32_words(layer.scale_inv)
        assert list(si) == [as_bits(O.scale_inv(s)) for s in (sx, sw, sg)], t
        rs = np.sort(synth.rng(8, t, 0).choice(M, 32, replace=False))
        xq_rows = O.encode(O.scaled_values(xf[rs], sx), O.E4M3)
        gq_rows = O.encode(O.scaled_values(gf[rs], sg), O.E5M2)
        xq, wq = layer.last_codes
        gq, _ = layer.last_grad_codes
        assert np.array_equal(np_codes(xq[rs]), xq_rows), t
        assert np.array_equal(np_codes(gq[rs]), gq_rows), t
        assert np.array_equal(np_codes(wq), wc), t
        check(np_bf16_bits(y.reshape(M, N))[rs], xq_rows, O.E4M3, wc, O.E4M3, O.scale_inv(sx), O.scale_inv(sw),
              bias, tag=f"dyn Y {t}")
        check(np_bf16_bits(dx.reshape(M, K))[rs], gq_rows, O.E5M2, np.ascontiguousarray(wc.T), O.E4M3,
              O.scale_inv(sg), O.scale_inv(sw), None, tag=f"dyn dX {t}")
        db_ref, db_mag = O.grad_bias(dy)
        assert np.array_equal(np_bf16_bits(db), db_ref), t


def test_prequantized_weight_and_fp8_bias():
    """w8 / b8, w8 / bf16 bias and the amax_w = 0 contract against an explicit
    quantization reference: a layer over pre-quantized E4M3 weight codes skips
    the weight quantize (its amax reads 0) and gives the outputs of the same
    codes pushed through the oracle; an E5M2-stored bias is dequantized by its
    scale in the epilogue."""
    xs, w, b = tiny_inputs(2)
    qw = O.quantize_dynamic(w, "bf16", O.E4M3)
    bf = O.widen_to_f32(b, "bf16")
    s_b = np.float32(O.FMT_MAX[O.E5M2]) / O.amax(bf)
    b8 = O.encode(O.scaled_values(bf, s_b), O.E5M2)
    sbi = O.scale_inv(s_b)
    for bias_kind in ("b8", "bf16"):
        if bias_kind == "b8":
            layer = Fp8Linear.from_fp8_weight(torch.from_numpy(qw["codes"]).to(DEV),
                                              torch.tensor([qw["scale_inv"]], dtype=torch.float32, device=DEV),
                                              torch.from_numpy(b8).to(DEV), codes_t=torch.from_numpy(qw["codes_t"]).to(DEV),
                                              bias_fmt=fp8mi.E5M2,
                                              bias_scale=torch.tensor([sbi], dtype=torch.float32, device=DEV))
            bias = O.dequant_bias(b8, O.E5M2, sbi).astype(np.float64)
        else:
            layer = Fp8Linear.from_fp8_weight(torch.from_numpy(qw["codes"]).to(DEV),
                                              torch.tensor([qw["scale_inv"]], dtype=torch.float32, device=DEV), dev_bf16(b),
                                              codes_t=torch.from_numpy(qw["codes_t"]).to(DEV))
            bias = bf.astype(np.float64)
        rx = O.seed_ring(4, xs[0], "bf16", O.E4M3)
        layer.seed(dev_bf16(xs[0]))
        for t in range(2):
            ref_x = O.quantize(xs[t], "bf16", O.E4M3, ring=rx)
            y = layer.forward(dev_bf16(xs[t]))
            dx, dw, db = layer.backward(dev_bf16(synth.gaussian((64, 256), 1e-3, "bf16", 1, synth.T_DY, t)))
            torch.cuda.synchronize()
            amax = f32_words(layer.amax)
            assert amax[1] == 0 and amax[0] == as_bits(ref_x["amax"]), (bias_kind, t)   # amax_w = 0
            xq, wq = layer.last_codes
            assert np.array_equal(np_codes(xq), ref_x["codes"]) and np.array_equal(np_codes(wq), qw["codes"])
            check(np_bf16_bits(y), ref_x["codes"], O.E4M3, qw["codes"], O.E4M3, ref_x["scale_inv"], qw["scale_inv"],
                  bias, tag=f"w8 {bias_kind} step {t}")
            rx = ref_x["ring"]


def test_fp8_out_layer_chain():
    """Inference chaining: layer 1 returns E4M3 codes of Y from its quantizing
    epilogue (output ring), layer 2 consumes them as x with their scale_inv --
    no quantize between the layers -- against the oracle's mm_quantized then mm."""
    x = synth.gaussian((64, 256), 1.0, "bf16", 3, synth.T_X, 0)
    w1 = synth.gaussian((256, 256), 0.05, "bf16", 3, synth.T_W, 1)
    w2 = synth.gaussian((128, 256), 0.05, "bf16", 3, synth.T_W, 2)
    b2 = synth.gaussian((128,), 0.1, "bf16", 3, synth.T_BIAS, 2)
    l1 = Fp8Linear(dev_bf16(w1), None, hist_len=4, dynamic=True)
    l2 = Fp8Linear(dev_bf16(w2), dev_bf16(b2), hist_len=4, dynamic=True)
    ry0 = O.Ring.new(4, 8.0)
    l1.ring_y.copy_(ring_from_oracle(ry0))
    y1, y1_sinv = l1.forward(dev_bf16(x), save_for_backward=False, out_fp8=True)
    y2 = l2.forward(y1, save_for_backward=False, x_scale_inv=y1_sinv)
    torch.cuda.synchronize()
    qx = O.quantize_dynamic(x, "bf16", O.E4M3)
    q1 = O.quantize_dynamic(w1, "bf16", O.E4M3)
    q2 = O.quantize_dynamic(w2, "bf16", O.E4M3)
    ref1 = O.mm_quantized(qx["codes"], O.E4M3, q1["codes"], O.E4M3, O.E4M3, qx["scale_inv"], q1["scale_inv"],
                          ring=ry0)
    got1 = np_codes(y1)
    # layer 1's codes: inside the band of the codes of y -+ the GEMM bound on y
    y, tol = y_band(qx["codes"], O.E4M3, q1["codes"], O.E4M3, qx["scale_inv"], q1["scale_inv"], None)
    check_codes(got1, y[0], tol[0], O.E4M3, ry0.scale, "chain layer 1")
    # its ring: the history holds the device's amax (within the band around
    # max |y|), and the ring words are the oracle's fold of that amax
    amax1 = np.float32(l1.ring_y.cpu().numpy().view(np.float32)[0])
    check_amax(float(amax1), y[0], tol[0], "chain layer 1")
    assert np.array_equal(ring_state_words(l1.ring_y), O.fold(ry0, amax1, O.E4M3).words())
    # the device's codes feed layer 2; its output must match the oracle on those codes
    assert f32_words(y1_sinv)[0] == as_bits(ref1["scale_inv"])
    check(np_bf16_bits(y2), got1, O.E4M3, q2["codes"], O.E4M3, ref1["scale_inv"], q2["scale_inv"],
          O.widen_to_f32(b2, "bf16").astype(np.float64), tag="chain layer 2")
