"""Helpers shared by the GPU parity tests (tensor <-> numpy bit views and the
GEMM tolerance).  Nothing here computes any part of the method."""
from __future__ import annotations

import numpy as np
import torch

DEV = "cuda"

# GEMM outputs: the oracle is the exact product rounded once; the library
# accumulates in fp32 and rounds the fp32 result.  Gate, per element:
#   |y - ref| <= RTOL * |ref| + ATOL_RMS * rms(ref)
# (relative tolerance 1e-2; the absolute term only matters for outputs that
# cancel to near zero).
RTOL = 1e-2
ATOL_RMS = 1e-2


def bits16(t: torch.Tensor) -> np.ndarray:
    """bf16 tensor (any device) -> numpy uint16 bit patterns."""
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def bits8(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().numpy().view(np.uint8)


def f32(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().numpy().astype(np.float32)


def f32_bits(t: torch.Tensor) -> np.ndarray:
    return f32(t).view(np.uint32)


def bf16_values(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def assert_gemm_close(y: np.ndarray, ref: np.ndarray, what: str = "gemm") -> dict:
    """y, ref: float64 arrays of the same shape (already decoded)."""
    assert y.shape == ref.shape, (y.shape, ref.shape)
    assert np.isfinite(ref).all(), "reference has non-finite outputs"
    assert np.isfinite(y).all(), f"{what}: non-finite outputs"
    rms = float(np.sqrt(np.mean(ref * ref))) if ref.size else 0.0
    err = np.abs(y - ref)
    bound = RTOL * np.abs(ref) + ATOL_RMS * rms
    bad = err > bound
    fro = float(np.linalg.norm(y - ref) / max(np.linalg.norm(ref), 1e-300))
    stats = {"max_abs": float(err.max(initial=0.0)), "rms_ref": rms, "fro_rel": fro,
             "n_bad": int(bad.sum())}
    assert not bad.any(), f"{what}: {stats}, first bad at {np.argwhere(bad)[:5].tolist()}"
    return stats
