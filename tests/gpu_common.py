"""Helpers for the GPU parity tests: device transfers and the tolerance.

Tolerance for products (fp32 accumulation vs the oracle's fp64 sum over the
same dequantized operands, then a bf16 output): elementwise
|y - ref| <= 1e-3 + 1e-2 * |ref|.
"""
from __future__ import annotations

import numpy as np
import torch

ATOL = 1e-3
RTOL = 1e-2


def device():
    if not torch.cuda.is_available():
        raise RuntimeError("GPU tests need a visible GPU")
    return torch.device("cuda", 0)


def dev_bf16(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device())


def dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(device())


def host_u8(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy()


def host_bf16_f32(t: torch.Tensor) -> np.ndarray:
    b = t.view(torch.int16).cpu().numpy().view(np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def assert_close(y: np.ndarray, ref: np.ndarray, what: str = ""):
    y = np.asarray(y, np.float64)
    ref = np.asarray(ref, np.float64)
    assert y.shape == ref.shape, (y.shape, ref.shape)
    assert np.isfinite(y).all(), f"{what}: non-finite output"
    err = np.abs(y - ref)
    ok = err <= ATOL + RTOL * np.abs(ref)
    if not ok.all():
        bad = np.argwhere(~ok)
        i = tuple(bad[0])
        raise AssertionError(f"{what}: {bad.shape[0]} of {y.size} outside tolerance; first {i}: "
                             f"got {y[i]!r} want {ref[i]!r}; max abs err {err.max():.3e}")
    return float(err.max()), float((err / np.maximum(np.abs(ref), 1e-30)).max())
