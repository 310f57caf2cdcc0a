"""Helpers shared by the GPU parity tests (tensor <-> numpy bit views and the
GEMM tolerance).  Nothing here computes any part of the method."""
from __future__ import annotations

import numpy as np
import torch

DEV = "cuda"

# GEMM outputs: the oracle is the exact product rounded once; the library
# accumulates in fp32 and rounds the fp32 result.  Three gates, all asserted:
#   per element          |y - ref| <= RTOL * |ref| + ATOL_RMS * rms(ref)
#   typical outputs      |y - ref| <= RTOL * |ref|  wherever |ref| >= rms(ref)
#   whole matrix         ||y - ref||_F <= RTOL * ||ref||_F
# (relative tolerance 1e-2; the absolute term only matters for outputs that
# cancel to near zero, where the matrix core's grouped accumulation can lose
# up to about 2^-12.6 of the sum of |products| -- a few thousandths of rms).
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
    """y, ref: float64 arrays of the same shape (already decoded).  Where the
    reference is not finite (NaN or +-inf operands), y must have a NaN at
    exactly the same places and the same signed infinities; every finite
    element passes the three gates above."""
    assert y.shape == ref.shape, (y.shape, ref.shape)
    nan_ref, nan_y = np.isnan(ref), np.isnan(y)
    assert np.array_equal(nan_ref, nan_y), \
        f"{what}: NaN positions differ, first at {np.argwhere(nan_ref != nan_y)[:5].tolist()}"
    inf_ref = np.isinf(ref)
    assert np.array_equal(inf_ref, np.isinf(y)) and np.array_equal(ref[inf_ref], y[inf_ref]), \
        f"{what}: infinities differ"
    fin = np.isfinite(ref)
    y, ref = y[fin], ref[fin]
    rms = float(np.sqrt(np.mean(ref * ref))) if ref.size else 0.0
    err = np.abs(y - ref)
    bound = RTOL * np.abs(ref) + ATOL_RMS * rms
    bad = err > bound
    typical = np.abs(ref) >= rms
    rel_typ = float((err[typical] / np.abs(ref[typical])).max(initial=0.0))
    fro = float(np.linalg.norm(y - ref) / max(np.linalg.norm(ref), 1e-300))
    stats = {"max_abs": float(err.max(initial=0.0)), "rms_ref": rms, "fro_rel": fro,
             "max_rel_typical": rel_typ, "n_bad": int(bad.sum()), "n_nonfinite": int((~fin).sum())}
    assert not bad.any(), f"{what}: {stats}, first bad at {np.argwhere(bad)[:5].tolist()}"
    assert rel_typ <= RTOL, f"{what}: relative error above 1e-2 on |ref| >= rms: {stats}"
    assert fro <= RTOL, f"{what}: Frobenius relative error above 1e-2: {stats}"
    return stats
