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
