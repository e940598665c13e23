"""Helpers for the GPU parity tests: moving synth arrays to the device (with
optional misaligned bases and padded leading dimensions) and back."""
import numpy as np
import torch

import oracle as O

DEV = torch.device("cuda:0")
TORCH_DT = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}
SENTINEL = 0xA5


def to_device(x: np.ndarray, dtype: str, misalign: int = 0, ld: int | None = None) -> torch.Tensor:
    """2-D device tensor with the storage values of x.  misalign > 0 places
    the first element `misalign` elements past an allocation start; ld pads
    rows to a larger leading dimension."""
    rows, cols = x.shape
    ld = cols if ld is None else ld
    n = misalign + (rows - 1) * ld + cols if rows > 0 else misalign
    buf = torch.zeros(max(n, 1) + 16, dtype=TORCH_DT[dtype], device=DEV)
    if dtype == "bf16":
        src = torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16)
    else:
        src = torch.from_numpy(np.ascontiguousarray(x))
    view = torch.as_strided(buf, (rows, cols), (ld, 1), misalign)
    if rows and cols:
        view.copy_(src.to(DEV))
    return view


def codes_out(rows: int, cols: int, ld: int | None = None, misalign: int = 0) -> torch.Tensor:
    """uint8 output view filled with a sentinel (so untouched bytes show)."""
    ld = cols if ld is None else ld
    n = misalign + max(rows - 1, 0) * ld + cols
    buf = torch.full((max(n, 1) + 64,), SENTINEL, dtype=torch.uint8, device=DEV)
    return torch.as_strided(buf, (rows, cols), (ld, 1), misalign)


def padding_untouched(view: torch.Tensor) -> bool:
    """Every byte of the underlying buffer outside the view still holds the sentinel."""
    buf = view.untyped_storage()
    full = torch.empty(0, dtype=torch.uint8, device=view.device).set_(buf).cpu().numpy()
    mask = np.ones(full.shape, bool)
    rows, cols = view.shape
    off, ld = view.storage_offset(), view.stride(0)
    for i in range(rows):
        mask[off + i * ld: off + i * ld + cols] = False
    return bool(np.all(full[mask] == SENTINEL))


def scalar(v) -> torch.Tensor:
    return torch.tensor([np.float32(v)], dtype=torch.float32, device=DEV)


def np_codes(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().cpu().numpy()


def np_bf16_bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def f32_bits(t: torch.Tensor) -> int:
    return int(t.cpu().view(torch.int32).numpy().view(np.uint32)[0])


def as_bits(v) -> int:
    return int(np.array([v], np.float32).view(np.uint32)[0])


RING_SCRATCH = 1024


def ring_state_words(ring: torch.Tensor) -> np.ndarray:
    """The H + 4 state words of a device ring (history, scale, slot, ticket,
    reserved) after checking that its scratch region is clear."""
    w = ring.cpu().numpy().view(np.uint32)
    assert not w[-RING_SCRATCH:].any(), "ring scratch not cleared after the call"
    return w[:-RING_SCRATCH]


def ring_to_oracle(ring: torch.Tensor) -> "O.Ring":
    return O.Ring.from_words(ring_state_words(ring))


def ring_from_oracle(r: "O.Ring") -> torch.Tensor:
    w = np.concatenate([r.words(), np.zeros(RING_SCRATCH, np.uint32)])
    return torch.from_numpy(w.view(np.int32).copy()).to(DEV)


# ----------------------------------------------------------------- GEMM checks ----
# The fp8 MFMA's in-group truncation (the kernels' precise-accumulation note):
# products are added in aligned groups of 8 k, each cut toward zero to a grid
# 2^-13 below the group's largest product, so one group can lose up to 7 grid
# steps.  Only the named cancellation test widens the bound by this term.
MFMA_GROUP = 8
MFMA_GROUP_LOSS = 7 * 2.0 ** -12


def mfma_group_term(a, fa, b, fb, sa, sb):
    """7 * 2^-12 * sum_g max|a_ik| max|b_jk| over aligned groups of 8 k."""
    da = np.abs(O.decode_table(fa)[a])
    db = np.abs(O.decode_table(fb)[b])
    K = a.shape[-1]
    if K == 0:
        return np.zeros((a.shape[0], b.shape[0]))
    ga = da.reshape(a.shape[0], K // MFMA_GROUP, MFMA_GROUP).max(-1)
    gb = db.reshape(b.shape[0], K // MFMA_GROUP, MFMA_GROUP).max(-1)
    return MFMA_GROUP_LOSS * (ga @ gb.T) * abs(float(np.float32(sa)) * float(np.float32(sb)))


def check(gpu_bits, a, fa, b, fb, sa, sb, bias, rows=None, tag="", exact=False, hw_group_term=False):
    """Compare (a sample of rows of) the GPU output with the oracle.

    exact: every output equal to the oracle's bit for bit.  Otherwise every
    output must satisfy the stated bound |gpu - ref| <= ulp_bf16(|ref|) +
    1e-5 * sum_k |a_ik b_jk|; the number outside it is printed per call and
    must be 0.  hw_group_term (the named cancellation test only) adds the
    MFMA group term to the bound and returns the count outside the stated one."""
    a3 = a if a.ndim == 3 else a[None]
    b3 = b if b.ndim == 3 else b[None]
    g3 = gpu_bits if gpu_bits.ndim == 3 else gpu_bits[None]
    batch = max(a3.shape[0], b3.shape[0])
    n_all = n_out = 0
    worst = 0.0
    for z in range(batch):
        az = a3[min(z, a3.shape[0] - 1)]
        bz = b3[min(z, b3.shape[0] - 1)]
        rsel = np.arange(az.shape[0]) if rows is None else rows
        ref, mag = O.mm(az[rsel], fa, bz, fb, sa, sb, bias)
        got = g3[z][rsel]
        if exact:
            bad = got != ref[0]
            assert not bad.any(), f"{tag} batch {z}: {bad.sum()} of {bad.size} differ from the exact result"
            continue
        stated = O.within_tolerance(got, ref[0], mag[0])
        g = O.bf16_bits_to_f64(got)
        r = O.bf16_bits_to_f64(ref[0])
        with np.errstate(invalid="ignore", divide="ignore"):
            ratio = np.abs(g - r) / (O.ulp_bf16(r) + 1e-5 * mag[0])
        fin = np.isfinite(ratio)
        if fin.any():
            worst = max(worst, float(ratio[fin].max()))
        if hw_group_term:
            ext = O.within_tolerance(got, ref[0], mag[0] + mfma_group_term(az[rsel], fa, bz, fb, sa, sb) / 1e-5)
            assert ext.all(), f"{tag} batch {z}: {(~ext).sum()} of {ext.size} outside the widened bound"
        n_all += stated.size
        n_out += int((~stated).sum())
    if exact:
        return 0
    print(f"[mm bound] {tag}: {n_out} of {n_all} outside the stated bound, worst |gpu-ref|/bound {worst:.3f}",
          flush=True)
    if not hw_group_term:
        assert n_out == 0, f"{tag}: {n_out} of {n_all} outputs outside 1 bf16 ulp + 1e-5 * sum|ab|"
    return n_out
