"""Seeded synthetic inputs for the delayed-scaling FP8 linear workloads.

This module only draws random numbers: it holds none of the method's
arithmetic and is shared by the tests, the benchmark and the smoke check so
that the oracle and the GPU library see identical bits.  Every tensor is drawn
on the CPU with a fixed ``torch.Generator`` seed in fp32 and rounded to bf16
by torch (round to nearest even).

Shapes and distributions follow the toy transformer of "CPU Overhead of
te.Linear FP8 Layers" (hidden 2048, batch 8, seq 1024, mlp_ratio 4, inputs
drawn with torch.rand, i.e. U(0, 1)); the pages give no weight init, so
weights and biases are N(0, 0.02); gradients are N(0, 1e-3).

Seeds: activation of iteration i = 100 + i, weight = 2, bias = 3, gradient = 4,
outlier positions = 5.
"""
from __future__ import annotations

import torch

HIDDEN = 2048
BATCH = 8
SEQ = 1024
TOKENS = BATCH * SEQ          # GEMM M of every toy-block linear
MLP_RATIO = 4

SEED_X = 100
SEED_W = 2
SEED_BIAS = 3
SEED_DY = 4
SEED_OUTLIER = 5


def _gen(seed: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    return g


def normal_bf16(shape, std: float, seed: int) -> torch.Tensor:
    x = torch.randn(*shape, generator=_gen(seed), dtype=torch.float32)
    return (x * std).to(torch.bfloat16)


def uniform_bf16(shape, seed: int) -> torch.Tensor:
    return torch.rand(*shape, generator=_gen(seed), dtype=torch.float32).to(torch.bfloat16)


def with_outliers_bf16(shape, seed: int, frac: float = 1e-3, factor: float = 1e3,
                       outlier_seed: int = SEED_OUTLIER) -> torch.Tensor:
    """N(0, 1) with a seeded random fraction `frac` of entries times `factor`."""
    x = torch.randn(*shape, generator=_gen(seed), dtype=torch.float32)
    n = x.numel()
    k = int(round(n * frac))
    idx = torch.randperm(n, generator=_gen(outlier_seed))[:k]
    x.view(-1)[idx] *= factor
    return x.to(torch.bfloat16)


# ---- the workloads --------------------------------------------------------

def tiny_forward(iteration: int):
    """Single FP8 linear, tiny: X [128, 256] ~N(0,1) (fresh per iteration),
    W [512, 256] ~N(0, 0.02), bias [512] ~N(0, 0.02)."""
    x = normal_bf16((128, 256), 1.0, SEED_X + iteration)
    w = normal_bf16((512, 256), 0.02, SEED_W)
    b = normal_bf16((512,), 0.02, SEED_BIAS)
    return x, w, b


def cast_only(rows: int = 4096, cols: int = 4096):
    """Memory-bound cast workload: N(0, 1) with 0.1% outliers times 1e3."""
    return with_outliers_bf16((rows, cols), SEED_X)


def mlp_forward(iteration: int, m: int = TOKENS, n: int = MLP_RATIO * HIDDEN, k: int = HIDDEN):
    """Toy-block MLP up-projection: X [8192, 2048] ~U(0,1), W [8192, 2048]
    ~N(0, 0.02), bias [8192] ~N(0, 0.02)."""
    x = uniform_bf16((m, k), SEED_X + iteration)
    w = normal_bf16((n, k), 0.02, SEED_W)
    b = normal_bf16((n,), 0.02, SEED_BIAS)
    return x, w, b


def mlp_grad(m: int = TOKENS, n: int = MLP_RATIO * HIDDEN):
    """Output gradient dY [8192, 8192] ~N(0, 1e-3)."""
    return normal_bf16((m, n), 1e-3, SEED_DY)


def toy_block_linears(hidden: int = HIDDEN, mlp_ratio: int = MLP_RATIO):
    """(in_features, out_features, has_bias) of the six linears of one toy
    block: timestep modulation, self-attention qkv, cross-attention q and kv,
    and the two MLP layers."""
    h, m = hidden, int(hidden * mlp_ratio)
    return [(h, 6 * h, True), (h, 3 * h, False), (h, h, False), (h, 2 * h, False),
            (h, m, True), (m, h, True)]


def random_fp8_codes(shape, seed: int, fmt: int) -> torch.Tensor:
    """Uniformly random finite FP8 bytes of format fmt (0 = E4M3, 1 = E5M2):
    the NaN codes (and for E5M2 the infinities) are replaced by zero."""
    c = torch.randint(0, 256, shape, generator=_gen(seed), dtype=torch.int32).to(torch.uint8)
    if fmt == 0:
        c[(c & 0x7F) == 0x7F] = 0
    else:
        c[(c & 0x7C) == 0x7C] = 0
    return c
