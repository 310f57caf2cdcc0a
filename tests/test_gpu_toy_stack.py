"""GPU parity for the toy transformer stack of "CPU Overhead of te.Linear FP8
Layers" (hidden 2048, batch 8, seq 1024, mlp_ratio 4) and HIP-graph capture.

The block (reproduction script of that page): timestep modulation
2048 -> 12288 (+bias) chunked into shift/scale, x = shift * x / scale,
self-attention qkv 2048 -> 6144 (first third added back), cross-attention q
2048 -> 2048 and kv 2048 -> 4096 (first half added back), and an MLP
2048 -> 8192 (+bias) -> 2048 (+bias), all FP8 linears with delayed scaling.
The elementwise glue runs in torch; every linear is checked against the
oracle on the identical bf16 input it received (codes, amax and scale-inverse
bit-exact, outputs sampled within tolerance), and one scale update covers
all 2 x 6 x depth records.
"""
import numpy as np
import pytest
import torch

import delayed_scaling_linear_amd as dsl
import oracle
import workloads
from tests.gpu_util import DEV, assert_gemm_close, bf16_values, bits16, bits8, f32_bits

pytestmark = pytest.mark.gpu

M = workloads.TOKENS


def _linear(x_dev, w_dev, b_dev, st, tx, tw, check, rng):
    """One FP8 linear through the C ABI; if `check`, compare with the oracle."""
    K = x_dev.shape[1]
    N = w_dev.shape[0]
    qx = dsl.Float8Tensor.empty(M, K, 0, transpose=False, device=DEV)
    qw = dsl.Float8Tensor.empty(N, K, 0, device=DEV)
    y = torch.empty(M, N, dtype=torch.bfloat16, device=DEV)
    amax_before = st.amax_cur.clone()
    dsl.fp8_cast_transpose_amax(x_dev, st.scale[tx:tx + 1], qx, st.amax_cur[tx:tx + 1])
    dsl.fp8_cast_transpose_amax(w_dev, st.scale[tw:tw + 1], qw, st.amax_cur[tw:tw + 1])
    dsl.fp8_linear_fwd(qx, qw, b_dev, y)
    if check:
        torch.cuda.synchronize()
        sx, sw = float(st.scale[tx]), float(st.scale[tw])
        ox, _, ax, six = oracle.cast_transpose_amax(bits16(x_dev), sx, 0, want_qt=False,
                                                    amax_in=float(amax_before[tx]))
        ow, owt, aw, siw = oracle.cast_transpose_amax(bits16(w_dev), sw, 0,
                                                      amax_in=float(amax_before[tw]))
        np.testing.assert_array_equal(bits8(qx.data), ox)
        np.testing.assert_array_equal(bits8(qw.data), ow)
        np.testing.assert_array_equal(bits8(qw.data_t), owt)
        assert f32_bits(st.amax_cur)[tx] == np.float32(ax).view(np.uint32)
        assert f32_bits(st.amax_cur)[tw] == np.float32(aw).view(np.uint32)
        assert f32_bits(qx.scale_inv)[0] == six.view(np.uint32)
        r, c = rng.integers(0, M, 400), rng.integers(0, N, 400)
        ref = oracle.gemm_nt_sampled(ox, 0, ow, 0, six, siw, r, c,
                                     bias=None if b_dev is None else bits16(b_dev))
        assert_gemm_close(bf16_values(bits16(y))[r, c], bf16_values(ref), f"linear {N}x{K}")
    return y


def _block_weights(bi):
    ws = []
    for li, (fin, fout, has_bias) in enumerate(workloads.toy_block_linears()):
        seed = 1000 * (bi + 1) + li
        w = workloads.normal_bf16((fout, fin), 0.02, seed).to(DEV)
        b = workloads.normal_bf16((fout,), 0.02, seed + 500).to(DEV) if has_bias else None
        ws.append((w, b))
    return ws


def _block(x, ws, st, base, check, rng):
    """Forward of one toy block; tensor records base + 2*l (input), +1 (weight)."""
    H = workloads.HIDDEN
    lin = lambda l, inp: _linear(inp, ws[l][0], ws[l][1], st, base + 2 * l, base + 2 * l + 1,
                                 check, rng)
    mod = lin(0, x)
    shift, scale = mod[:, :H], mod[:, H:2 * H]
    x = (shift.float() * x.float() / scale.float()).to(torch.bfloat16)
    x = torch.nan_to_num(x, nan=0.0, posinf=0.0, neginf=0.0)   # heavy tails of the ratio
    sa_q = lin(1, x)[:, :H]
    x = x + sa_q
    ca_q = lin(2, x)
    ca_k = lin(3, x)[:, :H]
    x = x + ca_q + ca_k
    h = lin(4, x)
    x = x + lin(5, h.contiguous())
    return x.contiguous()


def test_toy_stack_two_blocks_and_one_update_over_all_records():
    depth = 32
    T = 2 * 6 * depth                                   # 384 records
    st = dsl.DelayedScalingState([0] * T, device=DEV)
    rng = np.random.default_rng(0)
    x = workloads.uniform_bf16((M, workloads.HIDDEN), workloads.SEED_X).to(DEV)
    for bi in range(2):                                 # two blocks at the full shape
        x = _block(x, _block_weights(bi), st, 12 * bi, check=True, rng=rng)
    torch.cuda.synchronize()
    hist = st.amax_history.cpu().numpy().copy()
    cur = st.amax_cur.cpu().numpy().copy()
    scale = st.scale.cpu().numpy().copy()
    sinv = st.scale_inv.cpu().numpy().copy()
    recorded = cur.copy()
    st.update()
    torch.cuda.synchronize()
    oracle.scale_update(hist, cur, scale, sinv, np.zeros(T, np.uint8))
    np.testing.assert_array_equal(f32_bits(st.amax_history), hist.view(np.uint32))
    np.testing.assert_array_equal(f32_bits(st.scale), scale.view(np.uint32))
    np.testing.assert_array_equal(f32_bits(st.scale_inv), sinv.view(np.uint32))
    assert (recorded[:24] > 0).all() and (recorded[24:] == 0).all()
    assert (st.scale[:24].cpu() != 1.0).all() and (st.scale[24:].cpu() == 1.0).all()


def test_graph_capture_replays_match_eager():
    """One delayed-scaling iteration (two casts, the forward GEMM, the scale
    update) captured in a HIP graph and replayed three times, with eager work
    and synchronisations between replays, matches the same iteration run
    eagerly on a separate copy of the state: nothing in the library
    allocates, synchronises or reads device memory on the host."""
    Mg, N, K = 1024, 4096, 2048
    x = workloads.uniform_bf16((Mg, K), 7).to(DEV)
    w = workloads.normal_bf16((N, K), 0.02, 8).to(DEV)
    b = workloads.normal_bf16((N,), 0.02, 9).to(DEV)

    def make():
        st = dsl.DelayedScalingState([0, 0], device=DEV)
        qx = dsl.Float8Tensor.empty(Mg, K, 0, transpose=False, device=DEV)
        qw = dsl.Float8Tensor.empty(N, K, 0, device=DEV)
        y = torch.empty(Mg, N, dtype=torch.bfloat16, device=DEV)
        return st, qx, qw, y

    def iteration(st, qx, qw, y):
        dsl.fp8_cast_transpose_amax(x, st.scale[0:1], qx, st.amax_cur[0:1])
        dsl.fp8_cast_transpose_amax(w, st.scale[1:2], qw, st.amax_cur[1:2])
        dsl.fp8_linear_fwd(qx, qw, b, y)
        st.update()

    g_st, g_qx, g_qw, g_y = make()
    e_st, e_qx, e_qw, e_y = make()
    # Warm up on a side stream (first launches set kernel attributes).
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        w_st, w_qx, w_qw, w_y = make()
        iteration(w_st, w_qx, w_qw, w_y)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        iteration(g_st, g_qx, g_qw, g_y)
    torch.cuda.synchronize()
    # Capture does not execute: the graph's state is still the initial one.
    assert float(g_st.scale[0]) == 1.0 and float(g_st.amax_history.abs().sum()) == 0.0
    for rep in range(3):
        graph.replay()
        iteration(e_st, e_qx, e_qw, e_y)
        torch.cuda.synchronize()
        junk = torch.randn(256, 256, device=DEV) @ torch.randn(256, 256, device=DEV)  # eager work
        torch.cuda.synchronize()
        del junk
        for got, want in ((g_qx.data, e_qx.data), (g_qw.data, e_qw.data), (g_qw.data_t, e_qw.data_t)):
            assert torch.equal(got, want), f"replay {rep}: codes differ"
        assert torch.equal(g_y.view(torch.int16), e_y.view(torch.int16)), f"replay {rep}: Y differs"
        for name in ("amax_history", "amax_cur", "scale", "scale_inv"):
            assert torch.equal(getattr(g_st, name), getattr(e_st, name)), f"replay {rep}: {name}"
    assert float(g_st.scale[0]) != 1.0                  # the state did evolve


class _CachedWeightStack:
    """Toy-block forward whose FP8 weights persist across micro-batches: the
    weight casts take a device no-op flag (0 = cast, 1 = keep the cached
    codes, transpose and scale-inverse), so one captured graph serves both."""

    def __init__(self, blocks):
        H = workloads.HIDDEN
        self.flag = torch.zeros(1, dtype=torch.int32, device=DEV)
        self.st = dsl.DelayedScalingState([0] * (12 * blocks), device=DEV)
        self.blocks = []
        for bi in range(blocks):
            lins = []
            for (w, b), (fin, fout, _) in zip(_block_weights(bi), workloads.toy_block_linears()):
                qw = dsl.Float8Tensor.empty(fout, fin, 0, device=DEV)
                qx = dsl.Float8Tensor.empty(M, fin, 0, device=DEV)
                lins.append((w, b, qw, qx, torch.empty(M, fout, dtype=torch.bfloat16, device=DEV)))
            self.blocks.append(lins)
        self.H = H

    def _lin(self, bi, l, inp):
        w, b, qw, qx, y = self.blocks[bi][l]
        tx, tw = 12 * bi + 2 * l, 12 * bi + 2 * l + 1
        st = self.st
        dsl.fp8_cast_transpose_amax(inp, st.scale[tx:tx + 1], qx, st.amax_cur[tx:tx + 1])
        dsl.fp8_cast_transpose_amax(w, st.scale[tw:tw + 1], qw, st.amax_cur[tw:tw + 1],
                                    noop_flag=self.flag)
        dsl.fp8_linear_fwd(qx, qw, b, y)
        return y

    def _cast_w_gemm(self, bi, l):
        """Weight cast (flag-gated) and GEMM of linear l, its input already cast in qx."""
        w, b, qw, qx, y = self.blocks[bi][l]
        tw = 12 * bi + 2 * l + 1
        dsl.fp8_cast_transpose_amax(w, self.st.scale[tw:tw + 1], qw, self.st.amax_cur[tw:tw + 1],
                                    noop_flag=self.flag)
        dsl.fp8_linear_fwd(qx, qw, b, y)
        return y

    def _cast_in(self, bi, l, inp):
        tx = 12 * bi + 2 * l
        dsl.fp8_cast_transpose_amax(inp, self.st.scale[tx:tx + 1], self.blocks[bi][l][3],
                                    self.st.amax_cur[tx:tx + 1])

    def _produce_in(self, bi, l, op, x, a, b, y):
        tx = 12 * bi + 2 * l
        dsl.fp8_produce_cast_transpose_amax(op, x, a, b, y, self.st.scale[tx:tx + 1],
                                            self.blocks[bi][l][3], self.st.amax_cur[tx:tx + 1])
        return y

    def forward_fused(self, x):
        """forward() with each linear's input produced and cast in one pass
        (modulation, residual adds of one or two terms): no torch glue left
        but the last block's residual add."""
        H = self.H
        nb = len(self.blocks)
        self._cast_in(0, 0, x)
        for bi in range(nb):
            mod = self._cast_w_gemm(bi, 0)
            x = self._produce_in(bi, 1, dsl.PRODUCE_MODULATE, x, mod[:, :H], mod[:, H:2 * H],
                                 torch.empty_like(x))
            sa = self._cast_w_gemm(bi, 1)
            x = self._produce_in(bi, 2, dsl.PRODUCE_ADD, x, sa[:, :H], None, torch.empty_like(x))
            self._cast_in(bi, 3, x)
            ca_q = self._cast_w_gemm(bi, 2)
            ca_k = self._cast_w_gemm(bi, 3)
            x = self._produce_in(bi, 4, dsl.PRODUCE_ADD2, x, ca_q, ca_k[:, :H],
                                 torch.empty_like(x))
            h = self._cast_w_gemm(bi, 4)
            self._cast_in(bi, 5, h)
            o = self._cast_w_gemm(bi, 5)
            if bi + 1 < nb:
                x = self._produce_in(bi + 1, 0, dsl.PRODUCE_ADD, x, o, None, torch.empty_like(x))
            else:
                x = x + o
        self.st.update()
        return x

    def forward(self, x):
        H = self.H
        for bi in range(len(self.blocks)):
            mod = self._lin(bi, 0, x)
            x = torch.nan_to_num((mod[:, :H].float() * x.float() / mod[:, H:2 * H].float())
                                 .to(torch.bfloat16), nan=0.0, posinf=0.0, neginf=0.0)
            x = x + self._lin(bi, 1, x)[:, :H]
            x = x + self._lin(bi, 2, x) + self._lin(bi, 3, x)[:, :H]
            h = self._lin(bi, 4, x)
            x = x + self._lin(bi, 5, h)
        self.st.update()
        return x


def test_cached_weights_and_whole_forward_graph():
    """Two micro-batches of a 2-block forward (weights cast on the first,
    kept on the second by the device flag), eager and as one captured graph
    replayed with the flag flipped on the device: identical bits, and the
    cached FP8 weights are left untouched by the second micro-batch."""
    x1 = workloads.uniform_bf16((M, workloads.HIDDEN), 11).to(DEV)
    x2 = workloads.uniform_bf16((M, workloads.HIDDEN), 12).to(DEV)

    eager = _CachedWeightStack(2)
    eager.flag.fill_(0)
    e1 = eager.forward(x1).clone()
    torch.cuda.synchronize()
    cached = [(qw.data.clone(), qw.data_t.clone(), qw.scale_inv.clone())
              for lins in eager.blocks for (_, _, qw, _, _) in lins]
    eager.flag.fill_(1)
    e2 = eager.forward(x2).clone()
    torch.cuda.synchronize()
    after = [(qw.data, qw.data_t, qw.scale_inv) for lins in eager.blocks for (_, _, qw, _, _) in lins]
    for (d0, t0, s0), (d1, t1, s1) in zip(cached, after):
        assert torch.equal(d0, d1) and torch.equal(t0, t1) and torch.equal(s0, s1)
    # weights amax: recorded on the first micro-batch only
    assert float(eager.st.amax_history[1, 0]) == 0.0 and float(eager.st.amax_history[1, 1]) > 0.0

    g = _CachedWeightStack(2)
    xin = torch.empty_like(x1)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):                 # warm-up launches on a side stream
        w = _CachedWeightStack(1)
        w.forward(x1)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        gout = g.forward(xin)
    for rep, (xv, flag, want) in enumerate(((x1, 0, e1), (x2, 1, e2))):
        xin.copy_(xv)
        g.flag.fill_(flag)
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(gout.view(torch.int16), want.view(torch.int16)), f"micro-batch {rep + 1}"
    for name in ("amax_history", "scale", "scale_inv"):
        assert torch.equal(getattr(g.st, name), getattr(eager.st, name)), name


def test_fused_producers_forward_matches_torch_glue():
    """The 2-block forward with the modulation and the residual adds fused into
    the following casts gives the same bits as the forward with torch glue
    followed by separate casts (same scales, same weights): outputs, and the
    whole delayed-scaling state after the update."""
    x = workloads.uniform_bf16((M, workloads.HIDDEN), 21).to(DEV)
    a, b = _CachedWeightStack(2), _CachedWeightStack(2)
    for _ in range(2):                         # two steps: the second uses updated scales
        ya = a.forward(x)
        yb = b.forward_fused(x)
        torch.cuda.synchronize()
        assert torch.equal(ya.view(torch.int16), yb.view(torch.int16))
    for name in ("amax_history", "scale", "scale_inv"):
        assert torch.equal(getattr(a.st, name), getattr(b.st, name)), name
