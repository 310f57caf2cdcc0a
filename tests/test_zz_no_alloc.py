"""The no-allocation variant of the dbias cast,
fp8_cast_transpose_amax_dbias_noalloc, called through the C ABI, against the
workspace entry point it varies (fp8_cast_transpose_amax_dbias): the same
kernels, so codes, transpose, amax, scale-inverse and dbias must agree bit
for bit.  Two calls in a row on the one per-GPU scratch array, the second
with a smaller, ragged source, so stale sums of the first call would show."""
import ctypes

import numpy as np
import pytest
import torch

import delayed_scaling_linear_amd as dsl
import workloads
from tests.gpu_util import DEV, bits8, f32_bits

pytestmark = pytest.mark.gpu


def _noalloc(x, scale, out, amax, dbias):
    """The raw C-ABI call (no workspace argument)."""
    d = out.desc()
    rc = dsl.lib().fp8_cast_transpose_amax_dbias_noalloc(
        x.data_ptr(), dsl.DTYPE_BF16, x.shape[0], x.shape[1], x.stride(0), scale.data_ptr(),
        ctypes.byref(d), amax.data_ptr(), dbias.data_ptr(), None,
        torch.cuda.current_stream().cuda_stream)
    assert rc == 0, dsl.fp8_status_string(rc)


def _run(x, scale_v, fmt, noalloc):
    rows, cols = x.shape
    out = dsl.Float8Tensor.empty(rows, cols, fmt, device=DEV)
    scale = torch.tensor([scale_v], dtype=torch.float32, device=DEV)
    amax = torch.zeros(1, dtype=torch.float32, device=DEV)
    dbias = torch.full((cols,), float("nan"), dtype=torch.float32, device=DEV)
    if noalloc:
        _noalloc(x, scale, out, amax, dbias)
    else:
        ws = torch.empty(dsl.fp8_cast_dbias_workspace_bytes(rows, cols), dtype=torch.uint8,
                         device=DEV)
        dsl.fp8_cast_transpose_amax_dbias(x, scale, out, amax, dbias, ws)
    torch.cuda.synchronize()
    return out, amax, dbias


@pytest.mark.parametrize("order", ["noalloc_first", "workspace_first"])
def test_noalloc_matches_the_workspace_entry_point_on_two_calls(order):
    cases = [((8192, 12288), dsl.E5M2, 2.0e5, 41),     # the toy block's widest output gradient
             ((1040, 400), dsl.E4M3, 37.0, 42)]        # smaller and ragged: partial tiles
    for (rows, cols), fmt, scale, seed in cases:
        x = workloads.normal_bf16((rows, cols), 1e-3, seed).to(DEV)
        x[3, :] = 5.0                                  # a row that dominates the column sums
        runs = [True, False] if order == "noalloc_first" else [False, True]
        res = {na: _run(x, scale, fmt, na) for na in runs}
        (oa, aa, da), (ob, ab, db) = res[True], res[False]
        np.testing.assert_array_equal(bits8(oa.data), bits8(ob.data))
        np.testing.assert_array_equal(bits8(oa.data_t), bits8(ob.data_t))
        assert f32_bits(aa)[0] == f32_bits(ab)[0]
        assert f32_bits(oa.scale_inv)[0] == f32_bits(ob.scale_inv)[0]
        np.testing.assert_array_equal(f32_bits(da), f32_bits(db))
        assert not torch.isnan(da).any()
