"""Shared test helpers: uploading seeded inputs and the parity criteria.

Parity bar (the tolerances stated for this method):
* fp32 inputs: max relative error 1e-5, where the relative error of an entry
  is |gpu - oracle| / max(|oracle|, rms(oracle)) -- an unfloored relative
  error is ill-posed on entries of y that cancel to ~0;
* bf16 inputs with fp32 state: |gpu - oracle| <= 1e-3 + 2e-2 |oracle|.
"""

from __future__ import annotations

import numpy as np
import torch

FP32_RTOL = 1e-5
BF16_ATOL, BF16_RTOL = 1e-3, 2e-2


def to_dev(t, device="cuda"):
    """Tensor (ssm_inputs.Tensor) or float32 ndarray -> device tensor in its storage dtype."""
    if t is None:
        return None
    if isinstance(t, np.ndarray):
        return torch.from_numpy(np.ascontiguousarray(t, dtype=np.float32)).to(device)
    if t.bf16 is not None:
        return torch.from_numpy(t.bf16.view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(t.f32)).to(device)


def to_np(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def rel_err_floored(g, r):
    g = np.asarray(g, np.float64)
    r = np.asarray(r, np.float64)
    if r.size == 0:
        return 0.0
    rms = float(np.sqrt(np.mean(r * r)))
    den = np.maximum(np.abs(r), max(rms, 1e-30))
    return float(np.max(np.abs(g - r) / den))


def nmse(g, r):
    g = np.asarray(g, np.float64)
    r = np.asarray(r, np.float64)
    den = float(np.sum(r * r))
    return float(np.sum((g - r) ** 2) / den) if den > 0 else 0.0


def assert_close(g, r, dtype: str, what: str = ""):
    g = np.asarray(g, np.float64)
    r = np.asarray(r, np.float64)
    assert g.shape == r.shape, (what, g.shape, r.shape)
    assert np.isfinite(g).all(), f"{what}: non-finite values from the GPU"
    if dtype == "f32":
        e = rel_err_floored(g, r)
        assert e <= FP32_RTOL, f"{what}: floored relative error {e:.3e} > {FP32_RTOL} (nmse {nmse(g, r):.2e})"
    else:
        bad = np.abs(g - r) > BF16_ATOL + BF16_RTOL * np.abs(r)
        if bad.any():
            i = np.unravel_index(np.argmax(np.abs(g - r) - BF16_RTOL * np.abs(r)), g.shape)
            raise AssertionError(f"{what}: {int(bad.sum())} entries outside 1e-3 + 2e-2|r|; worst at {i}: "
                                 f"gpu {g[i]!r} oracle {r[i]!r}")
