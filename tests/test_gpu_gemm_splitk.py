"""GPU parity: the split form of the FP8 products (fp8_linear_{fwd,dgrad,
wgrad}_ws), through the C ABI.

Products whose few output tiles would leave compute units idle over a long
contraction are computed in K parts through the caller's workspace, then
the parts are summed in part order.  Every output is checked against the
oracle's exact product (same tolerance as the unsplit tests), for each role
and output type, ragged shapes and part counts that are not powers of two;
repeated calls give identical bits; a null workspace, or one too short for
any part count that fills the chip, gives the unsplit entry point's bits."""
import numpy as np
import pytest
import torch

import delayed_scaling_linear_amd as dsl
import oracle
import workloads
from tests.gpu_util import DEV, assert_gemm_close, bf16_values, bits16, f32

pytestmark = pytest.mark.gpu


def _cus() -> int:
    return torch.cuda.get_device_properties(0).multi_processor_count


def _parts(M, N, K, cus, ws_bytes=1 << 62):
    """The split rule of the library, restated: 1 for products with 3/4 of a
    256 x 256 tile per CU (or 256^3 outputs) or more than one 128 x 128 tile
    per CU, else the largest P <= 16 with 3/4 CUs <= tiles * P <= CUs,
    K / P >= 4096, K % (128 P) == 0 and P*M*N*4 workspace bytes."""
    tiles = -(-M // 256) * -(-N // 256)
    if M * N >= 256 ** 3 or 4 * tiles >= 3 * cus or K % 128:
        return 1
    if -(-M // 128) * -(-N // 128) > cus:
        return 1
    best = 1
    for p in range(2, 17):
        if K // p < 4096 or tiles * p > cus or p * M * N * 4 > ws_bytes:
            break
        if K % (128 * p) == 0 and 4 * tiles * p >= 3 * cus:
            best = p
    return best


def _ws(nbytes: int) -> torch.Tensor:
    return torch.empty(max(nbytes, 16), dtype=torch.uint8, device=DEV)


def _si(v):
    return torch.tensor([v], dtype=torch.float32, device=DEV)


def _ref(A, fa, B, fb, sa, sb, bias=None, out_kind=oracle.OUT_BF16):
    r = oracle.gemm_nt(A.numpy(), fa, B.numpy(), fb, np.float32(sa), np.float32(sb),
                       bias=None if bias is None else bits16(bias), out_kind=out_kind)
    return bf16_values(r) if out_kind == oracle.OUT_BF16 else r.astype(np.float64)


def _run(role, A, fa, B, fb, sa, sb, bias, out, workspace):
    """The product out[M, N] = dec(A [M, K]) . dec(B [N, K])^T * sa * sb (+ bias)
    through the entry point of `role`, with the operands laid out as that
    role reads them.  Returns the output tensor."""
    M, K = A.shape
    N = B.shape[0]
    Ad, Bd = A.to(DEV).contiguous(), B.to(DEV).contiguous()
    if role == "fwd":
        y = torch.empty(M, N, dtype=torch.bfloat16, device=DEV)
        dsl.fp8_linear_fwd(dsl.Float8Tensor(Ad, None, _si(sa), fa, M, K),
                           dsl.Float8Tensor(Bd, None, _si(sb), fb, N, K),
                           None if bias is None else bias.to(DEV), y, workspace=workspace)
        return y
    if role == "dgrad":
        # dx [M, N] = dy [M, K] . (w_t [N, K])^T: dy.data = A, w.data_t = B
        dx = torch.empty(M, N, dtype=torch.bfloat16, device=DEV)
        dsl.fp8_linear_dgrad(dsl.Float8Tensor(Ad, None, _si(sa), fa, M, K),
                             dsl.Float8Tensor(None, Bd, _si(sb), fb, K, N), dx,
                             workspace=workspace)
        return dx
    # wgrad: dw [M, N] = dy_t [M, K] . (x_t [N, K])^T, dy [K, M], x [K, N]
    dw = torch.empty(M, N, dtype=torch.float32 if out == "fp32" else torch.bfloat16, device=DEV)
    dsl.fp8_linear_wgrad(dsl.Float8Tensor(None, Ad, _si(sa), fa, K, M),
                         dsl.Float8Tensor(None, Bd, _si(sb), fb, K, N), dw, workspace=workspace)
    return dw


def _values(t):
    return bf16_values(bits16(t)) if t.dtype == torch.bfloat16 else f32(t).astype(np.float64)


CASES = [
    # role, M, N, K, out, bias: long contractions over few output tiles (the
    # weight gradient of a 2048 x 2048 linear over 16384 tokens), ragged
    # shapes, and part counts that are not powers of two
    ("wgrad", 2048, 2048, 16384, "fp32", False),  # 64 tiles: 4 parts, fp32 output
    ("fwd", 1000, 2056, 24576, "bf16", True),     # ragged M, N: 36 tiles, 6 parts
    ("dgrad", 520, 1032, 65536, "bf16", False),   # ragged: 15 tiles, 16 parts
    ("wgrad", 776, 1028, 49152, "fp32", False),   # ragged, N % 8 == 4: 20 tiles, 12 parts
]


@pytest.mark.parametrize("role,M,N,K,out,has_bias", CASES)
def test_split_products_against_the_oracle(role, M, N, K, out, has_bias):
    cus = _cus()
    parts = _parts(M, N, K, cus)
    assert parts > 1, "the case must exercise the split form on this device"
    need = dsl.fp8_gemm_workspace_bytes(M, N, K)
    assert need == parts * M * N * 4
    fa, fb = (0, 0) if role == "fwd" else (1, 0)
    A = workloads.random_fp8_codes((M, K), M + K + 11, fa)
    B = workloads.random_fp8_codes((N, K), N + K + 13, fb)
    sa, sb = 1.0 / 41.0, 7.0 / 448.0
    bias = workloads.normal_bf16((N,), 0.5, N + 3) if has_bias else None
    print(f"split {role} {M}x{N}x{K} {out} parts={parts}", flush=True)
    ws = _ws(need)
    y = _run(role, A, fa, B, fb, sa, sb, bias, out, ws)
    torch.cuda.synchronize()
    kind = oracle.OUT_FP32 if out == "fp32" else oracle.OUT_BF16
    ref = _ref(A, fa, B, fb, sa, sb, bias, kind)
    assert_gemm_close(_values(y), ref, f"split {role} {M}x{N}x{K} parts {parts}")
    # the same call again (workspace reused, its old contents left in place):
    # identical bits
    y2 = _run(role, A, fa, B, fb, sa, sb, bias, out, ws)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16) if y.dtype == torch.bfloat16 else y.view(torch.int32),
                       y2.view(torch.int16) if y2.dtype == torch.bfloat16 else y2.view(torch.int32))


def test_null_or_short_workspace_is_the_unsplit_product():
    M, N, K = 1000, 2056, 24576
    cus = _cus()
    A = workloads.random_fp8_codes((M, K), 5, 0)
    B = workloads.random_fp8_codes((N, K), 6, 0)
    bias = workloads.normal_bf16((N,), 0.5, 7)
    sa, sb = 1.0 / 23.0, 3.0 / 448.0
    y_plain = torch.empty(M, N, dtype=torch.bfloat16, device=DEV)
    x8 = dsl.Float8Tensor(A.to(DEV), None, _si(sa), 0, M, K)
    w8 = dsl.Float8Tensor(B.to(DEV), None, _si(sb), 0, N, K)
    dsl.fp8_linear_fwd(x8, w8, bias.to(DEV), y_plain)
    y_null = torch.empty_like(y_plain)
    # the _ws entry point with a NULL workspace (any size)
    d1, d2 = x8.desc(), w8.desc()
    import ctypes
    rc = dsl.lib().fp8_linear_fwd_ws(ctypes.byref(d1), ctypes.byref(d2), bias.to(DEV).data_ptr(),
                                     y_null.data_ptr(), None, 12345, None)
    assert rc == 0
    torch.cuda.synchronize()
    assert torch.equal(y_plain.view(torch.int16), y_null.view(torch.int16))
    # 36 tiles split 6 ways fill the chip; a workspace for 5.5 parts leaves
    # no count that does (5 parts occupy 180 of 256 CUs): unsplit, the plain bits
    assert _parts(M, N, K, cus) == 6 and _parts(M, N, K, cus, 11 * M * N * 2) == 1
    y = torch.empty_like(y_plain)
    dsl.fp8_linear_fwd(x8, w8, bias.to(DEV), y, workspace=_ws(11 * M * N * 2))
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y_plain.view(torch.int16))


def test_workspace_bytes_follow_the_rule():
    cus = _cus()
    for M, N, K in [(1024, 12288, 2048), (1024, 6144, 2048), (1024, 2048, 2048),
                    (1024, 4096, 2048), (1024, 8192, 2048), (1024, 2048, 8192),
                    (2048, 2048, 16384), (1024, 6144, 4096), (512, 520, 6528),
                    (1024, 2048, 32768), (2048, 2048, 32768), (4096, 2048, 16384),
                    (520, 1032, 65536), (776, 1028, 49152), (1000, 2056, 24576),
                    (8192, 8192, 2048), (2048, 2048, 8192), (4096, 2048, 8192),
                    (12288, 2048, 8192), (1000, 2056, 2048), (512, 520, 1152),
                    (256, 256, 128), (64, 64, 4096), (1024, 2048, 1040), (0, 16, 256)]:
        p = _parts(M, N, K, cus) if M > 0 else 1
        want = p * M * N * 4 if p > 1 else 0
        assert dsl.fp8_gemm_workspace_bytes(M, N, K) == want, (M, N, K)


def test_split_products_inside_a_graph_replay():
    """The split forward captured in a HIP graph (workspace from the graph's
    pool, as a framework allocator gives it) replays to the eager bits."""
    M, N, K = 1024, 2048, 32768
    A = workloads.random_fp8_codes((M, K), 21, 0).to(DEV)
    B = workloads.random_fp8_codes((N, K), 22, 0).to(DEV)
    bias = workloads.normal_bf16((N,), 0.5, 23).to(DEV)
    x8 = dsl.Float8Tensor(A, None, _si(1.0 / 19.0), 0, M, K)
    w8 = dsl.Float8Tensor(B, None, _si(2.0 / 448.0), 0, N, K)
    need = dsl.fp8_gemm_workspace_bytes(M, N, K)
    assert need > 0
    ws = _ws(need)
    y_eager = torch.empty(M, N, dtype=torch.bfloat16, device=DEV)
    dsl.fp8_linear_fwd(x8, w8, bias, y_eager, workspace=ws)
    y = torch.empty_like(y_eager)
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        dsl.fp8_linear_fwd(x8, w8, bias, y, workspace=ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        dsl.fp8_linear_fwd(x8, w8, bias, y, workspace=ws)
    for _ in range(3):
        y.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), y_eager.view(torch.int16))
