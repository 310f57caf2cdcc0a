"""GPU parity of the dynamic-scaling cast (fp8_cast_transpose_dynamic), the
comparator of delayed scaling: amax, scale, scale-inverse, codes and
transpose bit-exact against the oracle, through the C ABI."""
import numpy as np
import pytest
import torch

import delayed_scaling_linear_amd as dsl
import oracle
from tests.gpu_util import DEV, bits8, bits16, f32_bits


pytestmark = pytest.mark.gpu


def _check(x_cpu, fmt, margin=0, fallback=1.0, ld_pad=0):
    rows, cols = x_cpu.shape
    if ld_pad:
        wide = torch.zeros(rows, cols + ld_pad, dtype=x_cpu.dtype)
        wide[:, :cols] = x_cpu
        x_dev = wide.to(DEV)[:, :cols]
    else:
        x_dev = x_cpu.to(DEV)
    out = dsl.Float8Tensor.empty(rows, cols, fmt, device=DEV)
    scale = torch.tensor([fallback], dtype=torch.float32, device=DEV)
    amax = torch.full((1,), -1.0, dtype=torch.float32, device=DEV)
    dsl.fp8_cast_transpose_dynamic(x_dev, scale, out, amax, margin=margin)
    torch.cuda.synchronize()
    src = bits16(x_cpu) if x_cpu.dtype == torch.bfloat16 else x_cpu.numpy()
    oq, oqt, oamax, oscale, osinv = oracle.dynamic_cast(src, fmt, margin=margin,
                                                        fallback_scale=fallback)
    assert f32_bits(amax)[0] == np.float32(oamax).view(np.uint32)
    assert f32_bits(scale)[0] == np.float32(oscale).view(np.uint32)
    assert f32_bits(out.scale_inv)[0] == np.float32(osinv).view(np.uint32)
    np.testing.assert_array_equal(bits8(out.data), oq)
    np.testing.assert_array_equal(bits8(out.data_t), oqt)
    return float(scale[0])


@pytest.mark.parametrize("shape,src", [((16, 16), "bf16"), ((400, 272), "bf16"),
                                       ((272, 400), "fp32"), ((1024, 2048), "bf16")])
@pytest.mark.parametrize("fmt", [oracle.E4M3, oracle.E5M2])
@pytest.mark.parametrize("margin", [0, 3])
def test_dynamic_shapes(shape, src, fmt, margin):
    g = torch.Generator().manual_seed(shape[0] + 17 * margin + fmt)
    x = torch.randn(*shape, generator=g) * 0.02
    x = x.to(torch.bfloat16) if src == "bf16" else x
    _check(x, fmt, margin)


def test_dynamic_strided_rows():
    g = torch.Generator().manual_seed(5)
    x = (torch.randn(256, 320, generator=g) * 7).to(torch.bfloat16)
    _check(x, oracle.E4M3, ld_pad=64)


def test_dynamic_guards():
    assert _check(torch.zeros(64, 64, dtype=torch.bfloat16), oracle.E4M3, fallback=7.0) == 7.0
    x = torch.ones(64, 64)
    x[3, 3] = float("nan")
    assert _check(x.to(torch.bfloat16), oracle.E5M2, fallback=3.0) == 3.0
    x = torch.ones(64, 64)
    x[0, 0] = float("inf")
    assert _check(x, oracle.E4M3, fallback=2.0) == 2.0


def test_dynamic_full_size_workloads():
    import workloads
    x, _, _ = workloads.mlp_forward(0)
    _check(x, oracle.E4M3)
    _check(workloads.mlp_grad(), oracle.E5M2)


def test_dynamic_noop():
    x = torch.ones(64, 64, dtype=torch.bfloat16, device=DEV)
    out = dsl.Float8Tensor.empty(64, 64, 0, device=DEV)
    out.data.fill_(0xAA)
    scale = torch.tensor([5.0], device=DEV)
    amax = torch.tensor([-1.0], device=DEV)
    flag = torch.ones(1, dtype=torch.int32, device=DEV)
    dsl.fp8_cast_transpose_dynamic(x, scale, out, amax, noop_flag=flag)
    torch.cuda.synchronize()
    assert float(scale[0]) == 5.0 and float(amax[0]) == -1.0 and (out.data == 0xAA).all()


@pytest.mark.parametrize("shape", [(0, 32), (48, 0)])
def test_dynamic_empty_keeps_scale(shape):
    """An empty tensor has amax 0: the guard keeps the scale, and the
    scale-inverse snapshot is still written."""
    x = torch.empty(*shape, dtype=torch.bfloat16, device=DEV)
    out = dsl.Float8Tensor.empty(*shape, 1, device=DEV)
    scale = torch.tensor([4.0], device=DEV)
    amax = torch.tensor([-1.0], device=DEV)
    dsl.fp8_cast_transpose_dynamic(x, scale, out, amax)
    torch.cuda.synchronize()
    assert float(amax[0]) == 0.0 and float(scale[0]) == 4.0
    assert float(out.scale_inv[0]) == 0.25
