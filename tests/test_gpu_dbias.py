"""GPU parity of the cast with the bias gradient fused in
(fp8_cast_transpose_amax_dbias), through the C ABI.

Codes, transpose, amax and scale-inverse must equal the oracle bit for bit,
as for the plain cast.  dbias (fp32 column sums) is compared with the
oracle's exact sum rounded once: a term passes through at most
ceil(rows / 128) + 12 additions (3 within a lane's four rows, 3 in the
butterfly over a wave's eight row groups, 3 over the four waves, at most one
per tile row within a part of the second pass, 3 over its four parts), so by
the standard bound on recursive summation the error is at most
(ceil(rows / 128) + 12) * 2^-24 * sum |x|, plus 2^-24 * sum |x| for the
oracle's own rounding.  Repeated calls must give
identical bits (fixed summation order)."""
import numpy as np
import pytest
import torch

import delayed_scaling_linear_amd as dsl
import oracle
from tests.gpu_util import DEV, bits8, bits16, f32_bits

pytestmark = pytest.mark.gpu


def _run(x_dev, scale, fmt, q=True, qt=True, noop=None, dbias_fill=None):
    rows, cols = x_dev.shape
    out = dsl.Float8Tensor.empty(rows, cols, fmt, data=q, transpose=qt, device=DEV)
    s = torch.tensor([scale], dtype=torch.float32, device=DEV)
    amax = torch.zeros(1, dtype=torch.float32, device=DEV)
    dbias = torch.full((cols,), np.nan if dbias_fill is None else dbias_fill,
                       dtype=torch.float32, device=DEV)
    ws = torch.empty(max(dsl.fp8_cast_dbias_workspace_bytes(rows, cols), 16), dtype=torch.uint8,
                     device=DEV)
    dsl.fp8_cast_transpose_amax_dbias(x_dev, s, out, amax, dbias, ws, noop_flag=noop)
    torch.cuda.synchronize()
    return out, amax, dbias


def _src_np(x_cpu):
    return bits16(x_cpu) if x_cpu.dtype == torch.bfloat16 else x_cpu.numpy()


def _check(x_cpu, scale, fmt, q=True, qt=True):
    x_dev = x_cpu.to(DEV)
    out, amax, dbias = _run(x_dev, scale, fmt, q, qt)
    src = _src_np(x_cpu)
    oq, oqt, oamax, osinv = oracle.cast_transpose_amax(src, scale, fmt, want_q=q, want_qt=qt)
    if q:
        np.testing.assert_array_equal(bits8(out.data), oq)
    if qt:
        np.testing.assert_array_equal(bits8(out.data_t), oqt)
    assert f32_bits(amax)[0] == np.float32(oamax).view(np.uint32)
    assert f32_bits(out.scale_inv)[0] == np.float32(osinv).view(np.uint32)
    ref = oracle.dbias(src).astype(np.float64)
    got = dbias.cpu().numpy().astype(np.float64)
    xv = x_cpu.float().numpy().astype(np.float64)
    finite = np.isfinite(ref)
    np.testing.assert_array_equal(np.isnan(got), np.isnan(ref))
    np.testing.assert_array_equal(np.isinf(got) & ~np.isnan(ref), np.isinf(ref))
    with np.errstate(invalid="ignore"):
        bound = (np.ceil(x_cpu.shape[0] / 128) + 13) * 2.0 ** -24 * np.abs(xv).sum(axis=0)
    err = np.where(finite, np.abs(np.where(finite, got, 0.0) - np.where(finite, ref, 0.0)), 0.0)
    bad = finite & (err > bound)
    assert not bad.any(), (np.nonzero(bad)[0][:5], got[bad][:5], ref[bad][:5], bound[bad][:5])
    # same bits on a second call
    _, _, dbias2 = _run(x_dev, scale, fmt, q, qt)
    assert torch.equal(dbias.view(torch.int32), dbias2.view(torch.int32))
    return dbias


@pytest.mark.parametrize("extra", [16, 48, 64, 80, 112])
def test_dbias_every_column_residue_of_a_tile(extra):
    """Right-edge tiles whose lanes hold one source chunk inside the tensor
    and one outside: the column sums land on their own columns."""
    g = torch.Generator().manual_seed(2000 + extra)
    x = (torch.randn(272, 128 + extra, generator=g) * 3).to(torch.bfloat16)
    _check(x, 0.75, oracle.E5M2)


@pytest.mark.parametrize("shape,src,fmt,q,qt", [
    ((16, 16), "bf16", oracle.E5M2, True, True),
    ((400, 272), "bf16", oracle.E5M2, True, True),        # ragged tiles
    ((272, 400), "fp32", oracle.E4M3, True, True),        # fp32 source
    ((512, 128), "bf16", oracle.E5M2, True, False),       # codes only
    ((128, 640), "bf16", oracle.E5M2, False, True),       # transpose only
    ((5008, 5024), "bf16", oracle.E5M2, True, True),      # one workgroup per tile, ragged
])
def test_dbias_shapes(shape, src, fmt, q, qt):
    g = torch.Generator().manual_seed(shape[0] * 3 + shape[1])
    x = torch.randn(*shape, generator=g) * 1e-3
    x = x.to(torch.bfloat16) if src == "bf16" else x
    _check(x, 2.0e5, fmt, q, qt)


def test_dbias_full_size_gradient():
    """dY [8192, 8192] ~N(0, 1e-3): the gradient cast of the bench step."""
    import workloads
    dy = workloads.mlp_grad()
    _check(dy, 5.0e6, oracle.E5M2)


def test_dbias_special_values():
    x = torch.randn(256, 64) * 0.5
    x[3, 0] = float("inf")                 # column 0: +inf
    x[7, 1] = float("nan")                 # column 1: NaN
    x[5, 2] = float("inf")
    x[9, 2] = float("-inf")                # column 2: inf - inf = NaN
    x[:, 3] = 1.0                          # column 3: exact 256
    dbias = _check(x.to(torch.bfloat16), 1.0, oracle.E5M2)
    v = dbias.cpu().numpy()
    assert v[0] == np.inf and np.isnan(v[1]) and np.isnan(v[2]) and v[3] == 256.0


def test_dbias_empty_rows_and_noop():
    x = torch.zeros(0, 48, dtype=torch.bfloat16, device=DEV)
    _, _, dbias = _run(x, 1.0, oracle.E5M2)
    assert torch.equal(dbias.cpu(), torch.zeros(48))
    x = torch.ones(64, 48, dtype=torch.bfloat16, device=DEV)
    flag = torch.ones(1, dtype=torch.int32, device=DEV)
    out, amax, dbias = _run(x, 1.0, oracle.E5M2, noop=flag, dbias_fill=-7.0)
    assert torch.equal(dbias.cpu(), torch.full((48,), -7.0))
    assert float(amax[0]) == 0.0


def test_dbias_codes_equal_plain_cast():
    g = torch.Generator().manual_seed(9)
    x = (torch.randn(1024, 768, generator=g) * 3).to(torch.bfloat16).to(DEV)
    out_a, amax_a, _ = _run(x, 17.0, oracle.E4M3)
    out_b = dsl.Float8Tensor.empty(1024, 768, oracle.E4M3, device=DEV)
    amax_b = torch.zeros(1, device=DEV)
    dsl.fp8_cast_transpose_amax(x, torch.tensor([17.0], device=DEV), out_b, amax_b)
    torch.cuda.synchronize()
    assert torch.equal(out_a.data, out_b.data) and torch.equal(out_a.data_t, out_b.data_t)
    assert torch.equal(amax_a, amax_b) and torch.equal(out_a.scale_inv, out_b.scale_inv)


def test_dbias_column_slices_equal_the_whole_source():
    """Column sums are taken per 128 x 128 tile and then over tile rows, so a
    column slice (a strided view of the same memory) gives the whole
    source's sums for its columns.  [4096, 8192] against its eight
    [4096, 1024] slices: dbias, codes and transpose bit for bit, with a NaN,
    an inf and an inf - inf column planted; then the whole source against
    the oracle."""
    g = torch.Generator().manual_seed(17)
    x = (torch.randn(4096, 8192, generator=g) * 0.01).to(torch.bfloat16)
    x[5, 3] = float("nan")
    x[77, 1500] = float("inf")
    x[9, 4000] = float("inf")
    x[4000, 4000] = float("-inf")
    x_dev = x.to(DEV)
    print("dbias column slices, [4096, 8192]", flush=True)
    full_out, full_amax, full_db = _run(x_dev, 300.0, oracle.E5M2)
    for j in range(8):
        sl = x_dev[:, 1024 * j:1024 * (j + 1)]
        out, amax, db = _run(sl, 300.0, oracle.E5M2)
        cs = slice(1024 * j, 1024 * (j + 1))
        assert torch.equal(db.view(torch.int32), full_db[cs].view(torch.int32)), f"slice {j}: dbias"
        assert torch.equal(out.data, full_out.data[:, cs]), f"slice {j}: codes"
        assert torch.equal(out.data_t, full_out.data_t[cs, :]), f"slice {j}: transpose"
    v = full_db.cpu().numpy()
    assert np.isnan(v[3]) and v[1500] == np.inf and np.isnan(v[4000])
    _check(x, 300.0, oracle.E5M2)
