"""GPU parity: the FP8 GEMM entry points against the oracle (relative
tolerance 1e-2 on identical FP8 operands), through the C ABI."""
import numpy as np
import pytest
import torch

import delayed_scaling_linear_amd as dsl
import oracle
import workloads
from tests.gpu_util import DEV, assert_gemm_close, bf16_values, bits16, f32

pytestmark = pytest.mark.gpu


def _f8(codes: torch.Tensor, fmt: int, sinv: float, transpose_only=False) -> dsl.Float8Tensor:
    rows, cols = codes.shape
    d = codes.to(DEV).contiguous()
    si = torch.tensor([sinv], dtype=torch.float32, device=DEV)
    if transpose_only:
        # `codes` is given as the transpose [cols', rows'] of the logical tensor.
        return dsl.Float8Tensor(None, d, si, fmt, cols, rows)
    return dsl.Float8Tensor(d, None, si, fmt, rows, cols)


def _bias(n, seed):
    return workloads.normal_bf16((n,), 0.5, seed)


def _ref(A, fa, B, fb, sa, sb, bias=None, out_kind=oracle.OUT_BF16):
    r = oracle.gemm_nt(A.numpy(), fa, B.numpy(), fb, sa, sb,
                       bias=None if bias is None else bits16(bias), out_kind=out_kind)
    return bf16_values(r) if out_kind == oracle.OUT_BF16 else r.astype(np.float64)


SHAPES = [(128, 512, 256),       # the tiny forward layer
          (256, 256, 128),
          (200, 264, 272),       # ragged M, N and a K tail
          (16, 8, 16),
          (300, 776, 2064),
          (1, 1024, 48),
          (520, 136, 1024)]


@pytest.mark.parametrize("M,N,K", SHAPES)
@pytest.mark.parametrize("fa,fb", [(0, 0), (1, 0), (0, 1), (1, 1)])
def test_fwd_shapes_formats(M, N, K, fa, fb):
    A = workloads.random_fp8_codes((M, K), M + K + fa, fa)
    B = workloads.random_fp8_codes((N, K), N + K + 7 * fb, fb)
    bias = _bias(N, N)
    sa, sb = 1.0 / 37.0, 3.0 / 448.0
    y = torch.empty(M, N, dtype=torch.bfloat16, device=DEV)
    dsl.fp8_linear_fwd(_f8(A, fa, sa), _f8(B, fb, sb), bias.to(DEV), y)
    torch.cuda.synchronize()
    ref = _ref(A, fa, B, fb, np.float32(sa), np.float32(sb), bias)
    assert_gemm_close(bf16_values(bits16(y)), ref, f"fwd {M}x{N}x{K} {fa}{fb}")


@pytest.mark.parametrize("M,N,K,cfg", [
    (1024, 2048, 8192, "64x128"),      # 128 tiles of 128x128 < 256 CUs: 64x128 tiles
    (520, 1032, 1024, "64x128"),       # ragged M, N: 45 tiles of 128x128, 81 of 64x128
    (1000, 2056, 1040, "64x128"),      # 136 tiles of 128x128, 272 of 64x128; K tail (register-staged)
    (1000, 2056, 1024, "64x128"),      # ragged M, N, whole K stages (direct to LDS)
    (2048, 2048, 256, "64x128"),       # 256 tiles of 128x128, one per CU: 64x128 (direct to LDS)
    (2048, 2048, 272, "128x128"),      # the same with a K tail: 128x128 (register-staged)
    (2000, 2056, 272, "128x128"),      # ragged, 272 tiles, a K tail (register-staged)
    (2000, 2056, 384, "128x128"),      # ragged, whole K stages (direct to LDS)
])
@pytest.mark.parametrize("out", ["bf16", "fp32"])
def test_small_product_tile_shapes(M, N, K, cfg, out):
    """Products below 256^3 outputs run the small kernels: with fewer 128x128
    tiles than CUs they take 64x128 tiles (the direct-to-LDS kernel also with
    exactly one per CU); with whole 128-byte K stages the operand stages go
    straight into LDS, otherwise through registers.  Every output
    of each tile shape and kernel against the oracle, with bias (bf16) or
    without (fp32)."""
    A = workloads.random_fp8_codes((M, K), M + 3, 0)
    B = workloads.random_fp8_codes((N, K), N + 5, 1)
    sa, sb = 1.0 / 29.0, 5.0 / 448.0
    if out == "bf16":
        bias = _bias(N, N + 1)
        y = torch.empty(M, N, dtype=torch.bfloat16, device=DEV)
        dsl.fp8_linear_fwd(_f8(A, 0, sa), _f8(B, 1, sb), bias.to(DEV), y)
        torch.cuda.synchronize()
        ref = _ref(A, 0, B, 1, np.float32(sa), np.float32(sb), bias)
        assert_gemm_close(bf16_values(bits16(y)), ref, f"fwd {M}x{N}x{K} {cfg}")
    else:
        # wgrad form: dw [N', K'] = a [N', M'] . b [K', M']^T through the transposes
        dyt = dsl.Float8Tensor(None, A.to(DEV), torch.tensor([sa], device=DEV), 0, K, M)
        xt = dsl.Float8Tensor(None, B.to(DEV), torch.tensor([sb], device=DEV), 1, K, N)
        dw = torch.empty(M, N, dtype=torch.float32, device=DEV)
        dsl.fp8_linear_wgrad(dyt, xt, dw)
        torch.cuda.synchronize()
        ref = _ref(A, 0, B, 1, np.float32(sa), np.float32(sb), None, oracle.OUT_FP32)
        assert_gemm_close(f32(dw).astype(np.float64), ref, f"wgrad-form {M}x{N}x{K} {cfg}")


def test_fwd_without_bias_and_k_zero():
    A = workloads.random_fp8_codes((64, 128), 1, 0)
    B = workloads.random_fp8_codes((32, 128), 2, 0)
    y = torch.empty(64, 32, dtype=torch.bfloat16, device=DEV)
    dsl.fp8_linear_fwd(_f8(A, 0, 0.5), _f8(B, 0, 0.25), None, y)
    torch.cuda.synchronize()
    assert_gemm_close(bf16_values(bits16(y)), _ref(A, 0, B, 0, 0.5, 0.25), "fwd no bias")
    # K == 0: the output is the bias
    bias = _bias(32, 9)
    A0 = torch.empty(64, 0, dtype=torch.uint8)
    B0 = torch.empty(32, 0, dtype=torch.uint8)
    dsl.fp8_linear_fwd(dsl.Float8Tensor(None, None, torch.ones(1, device=DEV), 0, 64, 0),
                       dsl.Float8Tensor(None, None, torch.ones(1, device=DEV), 0, 32, 0),
                       bias.to(DEV), y)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits16(y), np.broadcast_to(bits16(bias), (64, 32)))
    del A0, B0


def test_exact_cases():
    """All-ones operands give acc = K exactly; an FP8 identity operand gives
    y = dec(A) * sinv_a * sinv_b exactly (power-of-two scale-inverses)."""
    K = 2048
    A = torch.full((256, K), 0x38, dtype=torch.uint8)     # 1.0 in E4M3
    B = torch.full((128, K), 0x3C, dtype=torch.uint8)     # 1.0 in E5M2
    yb = torch.empty(256, 128, dtype=torch.bfloat16, device=DEV)
    dsl.fp8_linear_fwd(_f8(A, 0, 1.0), _f8(B, 1, 1.0), None, yb)
    eye = torch.zeros(256, 256, dtype=torch.uint8)
    eye.fill_diagonal_(0x38)
    A2 = workloads.random_fp8_codes((64, 256), 11, 0)
    y2 = torch.empty(64, 256, dtype=torch.bfloat16, device=DEV)
    dsl.fp8_linear_fwd(_f8(A2, 0, 0.5), _f8(eye, 0, 0.25), None, y2)
    torch.cuda.synchronize()
    assert (bf16_values(bits16(yb)) == K).all()
    want = oracle.fp8_decode(A2.numpy(), 0) * 0.125
    np.testing.assert_array_equal(bf16_values(bits16(y2)), want)


@pytest.mark.parametrize("M,N,K", [(128, 512, 256), (272, 208, 152), (8192, 8192, 2048)])
def test_dgrad_and_wgrad_entry_points(M, N, K):
    """dgrad reads W's transpose, wgrad both transposes; the oracle composes
    the same products from the untransposed codes."""
    dY = workloads.random_fp8_codes((M, N), 3, 1)
    W = workloads.random_fp8_codes((N, K), 4, 0)
    X = workloads.random_fp8_codes((M, K), 5, 0)
    s_dy, s_w, s_x = 1.0 / 4096.0, 1.0 / 300.0, 1.0 / 7.0
    dev = {k: v.to(DEV) for k, v in (("dY", dY), ("W", W), ("X", X))}
    dyT = dsl.Float8Tensor(dev["dY"], dev["dY"].t().contiguous(),
                           torch.tensor([s_dy], device=DEV), 1, M, N)
    wT = dsl.Float8Tensor(None, dev["W"].t().contiguous(), torch.tensor([s_w], device=DEV), 0, N, K)
    xT = dsl.Float8Tensor(None, dev["X"].t().contiguous(), torch.tensor([s_x], device=DEV), 0, M, K)
    dx = torch.empty(M, K, dtype=torch.bfloat16, device=DEV)
    dw = torch.empty(N, K, dtype=torch.float32, device=DEV)
    dwb = torch.empty(N, K, dtype=torch.bfloat16, device=DEV)
    dsl.fp8_linear_dgrad(dyT, wT, dx)
    dsl.fp8_linear_wgrad(dyT, xT, dw)
    dsl.fp8_linear_wgrad(dyT, xT, dwb)
    torch.cuda.synchronize()
    s_dy, s_w, s_x = np.float32(s_dy), np.float32(s_w), np.float32(s_x)
    dYn, Wn, Xn = dY.numpy(), W.numpy(), X.numpy()
    if M * N * K <= 2 ** 27:
        ref_dx = oracle.gemm_nt(dYn, 1, np.ascontiguousarray(Wn.T), 0, s_dy, s_w)
        assert_gemm_close(bf16_values(bits16(dx)), bf16_values(ref_dx), "dgrad")
        ref_dw = oracle.gemm_nt(np.ascontiguousarray(dYn.T), 1, np.ascontiguousarray(Xn.T), 0,
                                s_dy, s_x, out_kind=oracle.OUT_FP32)
        assert_gemm_close(f32(dw).astype(np.float64), ref_dw.astype(np.float64), "wgrad fp32")
        ref_dwb = oracle.gemm_nt(np.ascontiguousarray(dYn.T), 1, np.ascontiguousarray(Xn.T), 0,
                                 s_dy, s_x)
        assert_gemm_close(bf16_values(bits16(dwb)), bf16_values(ref_dwb), "wgrad bf16")
    else:
        rng = np.random.default_rng(1)
        n = 1500
        r, c = rng.integers(0, M, n), rng.integers(0, K, n)
        WT = np.ascontiguousarray(Wn.T)
        ref = oracle.gemm_nt_sampled(dYn, 1, WT, 0, s_dy, s_w, r, c)
        assert_gemm_close(bf16_values(bits16(dx))[r, c], bf16_values(ref), "dgrad sampled")
        rn, ck = rng.integers(0, N, n), rng.integers(0, K, n)
        dYT, XT = np.ascontiguousarray(dYn.T), np.ascontiguousarray(Xn.T)
        ref = oracle.gemm_nt_sampled(dYT, 1, XT, 0, s_dy, s_x, rn, ck, out_kind=oracle.OUT_FP32)
        assert_gemm_close(f32(dw)[rn, ck].astype(np.float64), ref.astype(np.float64), "wgrad sampled")


def test_full_size_forward_sampled():
    """M8192 K2048 N8192 (the toy-block MLP shape), sampled outputs plus
    whole rows and columns, including the corners of the last tile."""
    M, N, K = 8192, 8192, 2048
    A = workloads.random_fp8_codes((M, K), 21, 0)
    B = workloads.random_fp8_codes((N, K), 22, 0)
    bias = _bias(N, 23)
    sa, sb = np.float32(1 / 448.0), np.float32(1 / 3.0)
    y = torch.empty(M, N, dtype=torch.bfloat16, device=DEV)
    dsl.fp8_linear_fwd(_f8(A, 0, float(sa)), _f8(B, 0, float(sb)), bias.to(DEV), y)
    torch.cuda.synchronize()
    rng = np.random.default_rng(2)
    r = np.concatenate([rng.integers(0, M, 3000), np.full(64, M - 1), np.arange(64)])
    c = np.concatenate([rng.integers(0, N, 3000), np.arange(N - 64, N), np.full(64, N - 1)])
    ref = oracle.gemm_nt_sampled(A.numpy(), 0, B.numpy(), 0, sa, sb, r, c, bias=bits16(bias))
    assert_gemm_close(bf16_values(bits16(y))[r, c], bf16_values(ref), "fwd full sampled")


def test_full_size_forward_every_output_on_the_benchmark_inputs():
    """The benchmark's own forward: X [8192, 2048] ~U(0,1) and W [8192, 2048]
    ~N(0,0.02) cast to E4M3 by the oracle with amax-derived scales, bias
    ~N(0,0.02); all 67,108,864 outputs against the oracle's full product."""
    x, w, b = workloads.mlp_forward(0)
    xb, wb = bits16(x), bits16(w)
    sx = np.float32(448.0) / np.float32(np.abs(bf16_values(xb)).max())
    sw = np.float32(448.0) / np.float32(np.abs(bf16_values(wb)).max())
    ox, _, _, six = oracle.cast_transpose_amax(xb, sx, oracle.E4M3, want_qt=False)
    ow, _, _, siw = oracle.cast_transpose_amax(wb, sw, oracle.E4M3, want_qt=False)
    y = torch.empty(8192, 8192, dtype=torch.bfloat16, device=DEV)
    dsl.fp8_linear_fwd(_f8(torch.from_numpy(ox), 0, float(six)),
                       _f8(torch.from_numpy(ow), 0, float(siw)), b.to(DEV), y)
    torch.cuda.synchronize()
    ref = oracle.gemm_nt(ox, 0, ow, 0, six, siw, bias=bits16(b))
    assert_gemm_close(bf16_values(bits16(y)), bf16_values(ref), "fwd 8192x8192x2048, every output")


def test_full_size_backward_every_output_on_the_benchmark_inputs():
    """The benchmark's own backward: dY [8192, 8192] ~N(0,1e-3) cast to E5M2,
    X and W [8192, 2048] cast to E4M3 (codes and transposes by the oracle,
    amax-derived scales); every output of dgrad (dX [8192, 2048] bf16, from
    W's transpose) and of wgrad (dW [8192, 2048] fp32, from both transposes)
    against the oracle's full products (contraction 8192)."""
    x, w, _ = workloads.mlp_forward(0)
    dy = workloads.mlp_grad()
    xb, wb, dyb = bits16(x), bits16(w), bits16(dy)
    amax = lambda b: np.float32(np.abs(bf16_values(b)).max())
    sx, sw, sdy = np.float32(448.0) / amax(xb), np.float32(448.0) / amax(wb), \
        np.float32(57344.0) / amax(dyb)
    _, oxT, _, six = oracle.cast_transpose_amax(xb, sx, oracle.E4M3, want_q=False)
    _, owT, _, siw = oracle.cast_transpose_amax(wb, sw, oracle.E4M3, want_q=False)
    ody, odyT, _, sidy = oracle.cast_transpose_amax(dyb, sdy, oracle.E5M2)
    M, N, K = 8192, 8192, 2048
    dyt = dsl.Float8Tensor(torch.from_numpy(ody).to(DEV), torch.from_numpy(odyT).to(DEV),
                           torch.tensor([float(sidy)], device=DEV), 1, M, N)
    wt = dsl.Float8Tensor(None, torch.from_numpy(owT).to(DEV),
                          torch.tensor([float(siw)], device=DEV), 0, N, K)
    xt = dsl.Float8Tensor(None, torch.from_numpy(oxT).to(DEV),
                          torch.tensor([float(six)], device=DEV), 0, M, K)
    dx = torch.empty(M, K, dtype=torch.bfloat16, device=DEV)
    dw = torch.empty(N, K, dtype=torch.float32, device=DEV)
    dsl.fp8_linear_dgrad(dyt, wt, dx)
    dsl.fp8_linear_wgrad(dyt, xt, dw)
    torch.cuda.synchronize()
    ref_dx = oracle.gemm_nt(ody, 1, owT, 0, sidy, siw)
    assert_gemm_close(bf16_values(bits16(dx)), bf16_values(ref_dx), "dgrad 8192x2048x8192, every output")
    ref_dw = oracle.gemm_nt(odyT, 1, oxT, 0, sidy, six, out_kind=oracle.OUT_FP32)
    assert_gemm_close(f32(dw).astype(np.float64), ref_dw.astype(np.float64),
                      "wgrad 8192x2048x8192 fp32, every output")


@pytest.mark.parametrize("M,N,K", [(4096, 4096, 272),      # large-tile path with a K tail
                                   (4104, 4104, 320),      # ragged M and N on the large-tile path
                                   (8200, 2056, 2064)])    # ragged everything, several tiles per CU
def test_large_path_tails_sampled(M, N, K):
    A = workloads.random_fp8_codes((M, K), M + 1, 0)
    B = workloads.random_fp8_codes((N, K), N + 2, 1)
    bias = _bias(N, K)
    sa, sb = np.float32(1 / 97.0), np.float32(1 / 5.0)
    y = torch.empty(M, N, dtype=torch.bfloat16, device=DEV)
    dsl.fp8_linear_fwd(_f8(A, 0, float(sa)), _f8(B, 1, float(sb)), bias.to(DEV), y)
    torch.cuda.synchronize()
    rng = np.random.default_rng(M)
    # random samples plus the last rows/columns (the ragged edges)
    r = np.concatenate([rng.integers(0, M, 2000), np.full(200, M - 1), rng.integers(M - 8, M, 200)])
    c = np.concatenate([rng.integers(0, N, 2000), rng.integers(0, N, 200), np.full(200, N - 1)])
    ref = oracle.gemm_nt_sampled(A.numpy(), 0, B.numpy(), 1, sa, sb, r, c, bias=bits16(bias))
    assert_gemm_close(bf16_values(bits16(y))[r, c], bf16_values(ref), f"fwd {M}x{N}x{K}")


@pytest.mark.parametrize("M,N,K,fa,fb,out", [
    (4096, 4096, 256, 0, 0, "bf16"),     # two K stages per tile (the minimum)
    (4104, 4104, 384, 1, 0, "bf16"),     # odd stage count, ragged M and N
    (8200, 2056, 2048, 0, 1, "bf16"),    # ragged, several tiles per workgroup
    (4096, 4352, 640, 1, 1, "fp32"),     # fp32 output, five stages
    (8192, 4096, 256, 0, 0, "bf16"),     # two stages per tile, two tiles per workgroup
    (8192, 4096, 256, 1, 0, "fp32"),     # the same with fp32 output
    (8200, 4104, 256, 1, 1, "bf16"),     # two stages, ragged M and N, 2-3 tiles per workgroup
    (4104, 8200, 256, 0, 1, "fp32"),     # the same with fp32 output
    (1024, 12288, 2048, 0, 0, "bf16"),   # under 256^3 outputs, 192 tiles: three quarters per CU
    (1000, 12304, 1024, 1, 0, "fp32"),   # the same, ragged M and N
])
def test_dma_path_rows_and_columns(M, N, K, fa, fb, out):
    """K % 128 == 0 at large M x N: whole output rows and columns at fragment
    and tile boundaries plus random samples, against the oracle."""
    A = workloads.random_fp8_codes((M, K), M + K, fa)
    B = workloads.random_fp8_codes((N, K), N + K + 1, fb)
    bias = _bias(N, K + 1) if out == "bf16" else None
    sa, sb = np.float32(1 / 61.0), np.float32(1 / 9.0)
    if out == "bf16":
        y = torch.empty(M, N, dtype=torch.bfloat16, device=DEV)
        dsl.fp8_linear_fwd(_f8(A, fa, float(sa)), _f8(B, fb, float(sb)), bias.to(DEV), y)
    else:
        y = torch.empty(M, N, dtype=torch.float32, device=DEV)
        # wgrad computes dW = dY^T X from the transposes: A^T is dY, B^T is X.
        dsl.fp8_linear_wgrad(_f8(A, fa, float(sa), transpose_only=True),
                             _f8(B, fb, float(sb), transpose_only=True), y)
    torch.cuda.synchronize()
    rng = np.random.default_rng(K)
    rows = [0, 1, 31, 32, 255, 256, M - 1]
    cols = [0, 127, 128, 255, N - 1]
    r = np.concatenate([np.repeat(rows, N), np.tile(np.arange(M), len(cols)), rng.integers(0, M, 2000)])
    c = np.concatenate([np.tile(np.arange(N), len(rows)), np.repeat(cols, M), rng.integers(0, N, 2000)])
    if out == "bf16":
        ref = oracle.gemm_nt_sampled(A.numpy(), fa, B.numpy(), fb, sa, sb, r, c, bias=bits16(bias))
        assert_gemm_close(bf16_values(bits16(y))[r, c], bf16_values(ref), f"dma {M}x{N}x{K}")
    else:
        ref = oracle.gemm_nt_sampled(A.numpy(), fa, B.numpy(), fb, sa, sb, r, c,
                                     out_kind=oracle.OUT_FP32)
        assert_gemm_close(f32(y)[r, c].astype(np.float64), ref.astype(np.float64), f"dma {M}x{N}x{K}")


def test_dma_path_repeats_bit_identically():
    """The large-tile kernel streams each workgroup's stages across tile
    boundaries and waits on exact counts of memory instructions in flight.
    A wait that released too early would read stale stage data; that shows
    as outputs that change from call to call.  Five calls of the
    8192x8192x2048 forward (four tiles per workgroup) and of an fp32-output
    product with two-stage tiles must give identical bits, and the first
    must match the oracle on sampled outputs."""
    M, N, K = 8192, 8192, 2048
    A = workloads.random_fp8_codes((M, K), 31, 0)
    B = workloads.random_fp8_codes((N, K), 32, 0)
    bias = _bias(N, 33)
    sa, sb = np.float32(1 / 448.0), np.float32(1 / 3.0)
    fa_, fb_ = _f8(A, 0, float(sa)), _f8(B, 0, float(sb))
    bd = bias.to(DEV)
    ys = [torch.empty(M, N, dtype=torch.bfloat16, device=DEV) for _ in range(5)]
    for y in ys:
        dsl.fp8_linear_fwd(fa_, fb_, bd, y)
    torch.cuda.synchronize()
    for y in ys[1:]:
        assert torch.equal(y.view(torch.int16), ys[0].view(torch.int16)), "fwd output changed between calls"
    rng = np.random.default_rng(3)
    r, c = rng.integers(0, M, 1500), rng.integers(0, N, 1500)
    ref = oracle.gemm_nt_sampled(A.numpy(), 0, B.numpy(), 0, sa, sb, r, c, bias=bits16(bias))
    assert_gemm_close(bf16_values(bits16(ys[0]))[r, c], bf16_values(ref), "fwd repeat sampled")

    Mw, Nw, Kw = 4104, 8200, 256           # wgrad-style fp32 output, two stages per tile
    A2 = workloads.random_fp8_codes((Mw, Kw), 34, 1)
    B2 = workloads.random_fp8_codes((Nw, Kw), 35, 0)
    outs = [torch.empty(Mw, Nw, dtype=torch.float32, device=DEV) for _ in range(5)]
    for o in outs:
        dsl.fp8_linear_wgrad(_f8(A2, 1, 0.5, transpose_only=True), _f8(B2, 0, 0.25, transpose_only=True), o)
    torch.cuda.synchronize()
    for o in outs[1:]:
        assert torch.equal(o.view(torch.int32), outs[0].view(torch.int32)), "fp32 output changed between calls"


def _plant_specials(A, fa, B, fb, rng):
    """NaN codes and (E5M2 only) +-inf codes planted in a few operand rows.
    Returns the planted rows of A and of B.  The oracle's exact product then
    has NaN where a NaN meets anything or +inf meets -inf or 0, and +-inf
    where one infinity meets nonzero finite values."""
    M, K = A.shape
    N = B.shape[0]
    ra = [3, M // 2, M - 1]
    rb = [5, N - 2]
    A[ra[0], rng.integers(0, K)] = 0x7F                     # NaN (both formats)
    if fa == 1:
        A[ra[1], rng.integers(0, K)] = 0x7C                 # +inf
        k1, k2 = rng.choice(K, 2, replace=False)
        A[ra[2], k1], A[ra[2], k2] = 0x7C, 0xFC             # +inf and -inf in one row
    else:
        A[ra[1], rng.integers(0, K)] = 0xFF                 # -NaN
    B[rb[0], rng.integers(0, K)] = 0xFF
    if fb == 1:
        B[rb[1], rng.integers(0, K)] = 0xFC                 # -inf
    return ra, rb


@pytest.mark.parametrize("M,N,K", [(200, 264, 272),        # small-tile kernel
                                   (1024, 16384, 272),     # register-staged large-tile kernel
                                   (1024, 16384, 256)])    # direct-to-LDS large-tile kernel
@pytest.mark.parametrize("fa,fb,out", [(1, 0, "bf16"), (0, 1, "fp32"), (1, 1, "bf16")])
def test_nan_and_inf_operands(M, N, K, fa, fb, out):
    """NaN and infinite operand codes (the cast emits 0x7F/0xFF for NaN
    sources; E5M2 has infinities) reach bf16 and fp32 outputs as the exact
    product says: NaN and +-inf at exactly the oracle's places, every finite
    output within tolerance."""
    rng = np.random.default_rng(M + N + K + fa + 2 * fb)
    A = workloads.random_fp8_codes((M, K), M + 3, fa)
    B = workloads.random_fp8_codes((N, K), N + 4, fb)
    ra, rb = _plant_specials(A, fa, B, fb, rng)
    sa, sb = np.float32(1 / 64.0), np.float32(1 / 3.0)
    bias = _bias(N, 40) if out == "bf16" else None
    if out == "bf16":
        y = torch.empty(M, N, dtype=torch.bfloat16, device=DEV)
        dsl.fp8_linear_fwd(_f8(A, fa, float(sa)), _f8(B, fb, float(sb)), bias.to(DEV), y)
    else:
        y = torch.empty(M, N, dtype=torch.float32, device=DEV)
        dsl.fp8_linear_wgrad(_f8(A, fa, float(sa), transpose_only=True),
                             _f8(B, fb, float(sb), transpose_only=True), y)
    torch.cuda.synchronize()
    kind = oracle.OUT_BF16 if out == "bf16" else oracle.OUT_FP32
    got = bf16_values(bits16(y)) if out == "bf16" else f32(y).astype(np.float64)
    # the planted rows and columns whole, plus random samples
    r = np.concatenate([np.repeat(ra, N), np.tile(np.arange(M), len(rb)), rng.integers(0, M, 3000)])
    c = np.concatenate([np.tile(np.arange(N), len(ra)), np.repeat(rb, M), rng.integers(0, N, 3000)])
    ref = oracle.gemm_nt_sampled(A.numpy(), fa, B.numpy(), fb, sa, sb, r, c,
                                 bias=None if bias is None else bits16(bias), out_kind=kind)
    ref = bf16_values(ref) if out == "bf16" else ref.astype(np.float64)
    stats = assert_gemm_close(got[r, c], ref, f"specials {M}x{N}x{K} {fa}{fb} {out}")
    assert stats["n_nonfinite"] >= N + M          # a NaN row and a NaN column at least
    if fa == 1:
        assert np.isinf(ref).any()                # the infinities really were exercised


@pytest.mark.parametrize("M,N", [(1024, 2048), (1000, 2056), (2048, 2048), (2000, 2056)])
@pytest.mark.parametrize("out", ["bf16", "fp32"])
def test_direct_to_lds_small_kernel_equals_register_staged(M, N, out):
    """The two small kernels run the same MFMA sequence, so they agree value
    for value.  K = 2048 takes the direct-to-LDS kernel; the same operands
    with 16 zero columns appended (K = 2064, a K tail) take the
    register-staged one, whose last step adds exact zeros."""
    K = 2048
    A = workloads.random_fp8_codes((M, K), M + 31, 0)
    B = workloads.random_fp8_codes((N, K), N + 37, 1)
    pad = lambda t: torch.cat([t, torch.zeros(t.shape[0], 16, dtype=torch.uint8)], dim=1)
    sa, sb = 1.0 / 13.0, 9.0 / 448.0
    if out == "bf16":
        bias = _bias(N, N + 2).to(DEV)
        y1 = torch.empty(M, N, dtype=torch.bfloat16, device=DEV)
        y2 = torch.empty_like(y1)
        dsl.fp8_linear_fwd(_f8(A, 0, sa), _f8(B, 1, sb), bias, y1)
        dsl.fp8_linear_fwd(_f8(pad(A), 0, sa), _f8(pad(B), 1, sb), bias, y2)
    else:
        si = lambda v: torch.tensor([v], device=DEV)
        y1 = torch.empty(M, N, dtype=torch.float32, device=DEV)
        y2 = torch.empty_like(y1)
        for a, b_, y in ((A, B, y1), (pad(A), pad(B), y2)):
            k = a.shape[1]
            dsl.fp8_linear_wgrad(dsl.Float8Tensor(None, a.to(DEV), si(sa), 0, k, M),
                                 dsl.Float8Tensor(None, b_.to(DEV), si(sb), 1, k, N), y)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)
