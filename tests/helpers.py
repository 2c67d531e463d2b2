"""Shared test helpers: storage conversions and the tolerance checks.

Tolerances (the layer's stated bar):
  * integer / index outputs and scores: bit-exact;
  * float32 tensors: max |gpu - ref| <= 1e-4;
  * bfloat16 tensors: max |gpu - ref| / max |ref| <= 2e-2.
"""
from __future__ import annotations

import numpy as np
import torch

FP32_ABS_TOL = 1e-4
BF16_REL_TOL = 2e-2


def to_device(arr: np.ndarray, dtype: str, device="cuda") -> torch.Tensor:
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).to(device)


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu", torch.float64).numpy()


def check_close(got, ref, dtype: str, what: str, scale: float | None = None):
    """got/ref float64 arrays; raise AssertionError with the error figure."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    if got.size == 0:
        return 0.0
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    err = float(np.max(np.abs(got - ref)))
    if dtype == "bf16":
        denom = scale if scale is not None else float(np.max(np.abs(ref)))
        rel = err / max(denom, 1e-30)
        assert rel <= BF16_REL_TOL, f"{what}: relative error {rel:.3e} > {BF16_REL_TOL}"
        return rel
    assert err <= FP32_ABS_TOL, f"{what}: max abs error {err:.3e} > {FP32_ABS_TOL}"
    return err
