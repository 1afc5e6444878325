"""Helpers for the GPU tests: moving storage bits to and from the device and
the elementwise parity bound.  No attention arithmetic lives here."""
from __future__ import annotations

import numpy as np

TOL_ABS = 1e-2
TOL_REL = 1e-2


def torch_dtype(dtype: str):
    import torch
    return torch.bfloat16 if dtype == "bf16" else torch.float16


def to_dev(bits: np.ndarray, dtype: str):
    """uint16 storage bits -> device tensor of the storage type (bit-exact)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch_dtype(dtype)).to("cuda")


def bits_of(t) -> np.ndarray:
    """device tensor (bf16/fp16) -> uint16 storage bits on the host."""
    import torch
    return t.detach().to("cpu").contiguous().view(torch.int16).numpy().view(np.uint16)


def parity(got: np.ndarray, ref: np.ndarray, what: str = "") -> dict:
    """|got - ref| <= 1e-2 + 1e-2 |ref| elementwise (both float64); returns stats."""
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = np.abs(got - ref)
    bound = TOL_ABS + TOL_REL * np.abs(ref)
    frac = float(np.max(err / bound)) if err.size else 0.0
    stats = {"max_abs": float(err.max()) if err.size else 0.0, "worst_frac_of_bound": frac}
    if frac > 1.0:
        idx = np.unravel_index(int(np.argmax(err / bound)), err.shape)
        raise AssertionError(f"{what}: parity bound exceeded at {idx}: got {got[idx]} "
                             f"ref {ref[idx]} ({stats})")
    return stats
