"""GPU parity of the toy transformer stack of "CPU Overhead of te.Linear FP8
Layers" (hidden 2048, batch 8 x seq 1024, mlp_ratio 4) run through the
library by bench.ToyStack, against the oracle.

Every probed linear is checked on the identical bf16 (or fp32 weight) tensor
its cast read: codes, transposes, amax and scale-inverse bit-exact, products
sampled within tolerance.  The scale update over all records is checked bit
for bit against the oracle's update of the same state.  Also: cached FP8
weights on a second micro-batch (the device no-op flag of "[PyTorch]
Refactor FP8 workspaces in linear modules"), one captured HIP graph serving
both micro-batches, fused producers against torch glue, a training step
(E5M2 gradient casts with the bias gradient, dgrad from the cached weight
transpose, fp32 wgrad) and the full 32-block forward.
"""
import numpy as np
import pytest
import torch

import delayed_scaling_linear_amd as dsl
import oracle
import workloads
from bench import R_DY, R_W, R_X, ToyStack
from tests.gpu_util import DEV, assert_gemm_close, bf16_values, bits8, bits16, f32, f32_bits

pytestmark = pytest.mark.gpu

M = workloads.TOKENS
H = workloads.HIDDEN


def _src(t: torch.Tensor) -> np.ndarray:
    """A cast source as the oracle takes it: bf16 bits or fp32 values."""
    return bits16(t) if t.dtype == torch.bfloat16 else f32(t)


def _state(st):
    return {n: f32(getattr(st, n)).copy() for n in ("amax_history", "amax_cur", "scale",
                                                     "scale_inv")}


def _update_and_check(stack, want_cur=None):
    """Run the stack's one scale update and compare it, bit for bit, with the
    oracle's update of the same pre-update state; `want_cur` (record ->
    oracle amax) pins the recorded amaxes first."""
    torch.cuda.synchronize()
    st = stack.state
    pre = _state(st)
    if want_cur is not None:
        for r, a in want_cur.items():
            assert pre["amax_cur"][r].view(np.uint32) == np.float32(a).view(np.uint32), f"record {r}"
    stack.state.update()
    torch.cuda.synchronize()
    hist, cur, scale, sinv = (pre["amax_history"].copy(), pre["amax_cur"].copy(),
                              pre["scale"].copy(), pre["scale_inv"].copy())
    oracle.scale_update(hist, cur, scale, sinv, f32(st.fmt).astype(np.uint8))
    np.testing.assert_array_equal(f32_bits(st.amax_history), hist.view(np.uint32))
    np.testing.assert_array_equal(f32_bits(st.scale), scale.view(np.uint32))
    np.testing.assert_array_equal(f32_bits(st.scale_inv), sinv.view(np.uint32))
    assert (f32(st.amax_cur) == 0).all()
    return pre


class ForwardCheck:
    """stack.probe: after the product of linear l of block b, compare its
    input and weight casts with the oracle's casts of the same tensors and
    sampled outputs with the oracle's product of the oracle's codes.

    cached: the weight casts were skipped by the no-op flag, so the weights
    must still hold the codes, transpose and scale-inverse recorded on an
    earlier micro-batch (self.w_codes) and the weight amax must stay 0."""

    def __init__(self, stack, blocks=None, samples=400, seed=0):
        self.stack, self.blocks, self.samples = stack, blocks, samples
        self.rng = np.random.default_rng(seed)
        self.cached = False
        self.w_codes, self.x_codes, self.amax = {}, {}, {}

    def __call__(self, b, l, y):
        if self.blocks is not None and b not in self.blocks:
            return
        torch.cuda.synchronize()
        s = self.stack
        st, train = s.state, s.train
        rx, rw = s.rec(b, l, R_X), s.rec(b, l, R_W)
        scale, cur = f32(st.scale), f32(st.amax_cur)
        qx, qw = s.qx[l][b], s.qw[b][l]
        ox, oxt, ax, six = oracle.cast_transpose_amax(_src(s.last_in[l]), scale[rx], oracle.E4M3,
                                                      want_qt=train)
        np.testing.assert_array_equal(bits8(qx.data), ox, err_msg=f"x codes b{b} l{l}")
        if train:
            np.testing.assert_array_equal(bits8(qx.data_t), oxt, err_msg=f"x^T b{b} l{l}")
        assert cur[rx].view(np.uint32) == np.float32(ax).view(np.uint32), f"x amax b{b} l{l}"
        assert f32_bits(qx.scale_inv)[0] == six.view(np.uint32)
        if self.cached:
            ow, owt, siw = self.w_codes[(b, l)]
            assert cur[rw] == 0.0, f"weight amax recorded on a cached micro-batch b{b} l{l}"
            aw = np.float32(0.0)
        else:
            ow, owt, aw, siw = oracle.cast_transpose_amax(_src(s.w[b][l]), scale[rw],
                                                          oracle.E4M3, want_qt=train)
            assert cur[rw].view(np.uint32) == np.float32(aw).view(np.uint32), f"w amax b{b} l{l}"
            self.w_codes[(b, l)] = (ow, owt, siw)
        np.testing.assert_array_equal(bits8(qw.data), ow, err_msg=f"w codes b{b} l{l}")
        if train:
            np.testing.assert_array_equal(bits8(qw.data_t), owt, err_msg=f"w^T b{b} l{l}")
        assert f32_bits(qw.scale_inv)[0] == np.float32(siw).view(np.uint32)
        self.amax[rx], self.amax[rw] = ax, aw
        self.x_codes[(b, l)] = (ox, oxt, six)
        n = self.samples
        r = self.rng.integers(0, M, n)
        c = self.rng.integers(0, y.shape[1], n)
        bias = s.b16[b][l]
        ref = oracle.gemm_nt_sampled(ox, 0, ow, 0, six, siw, r, c,
                                     bias=None if bias is None else bits16(bias))
        assert_gemm_close(bf16_values(bits16(y))[r, c], bf16_values(ref), f"linear b{b} l{l}")


class BackwardCheck:
    """stack.probe_bwd: after the backward of linear l of block b, compare
    the E5M2 cast of its output gradient (codes, transpose, amax,
    scale-inverse) with the oracle bit for bit and the fused bias gradient
    with the oracle's exact column sums within the stated summation bound;
    for the blocks in `full`, also sampled dgrad and wgrad outputs against
    the oracle's products of the oracle's codes."""

    def __init__(self, stack, fwd: ForwardCheck, full=(0,), samples=400, seed=1):
        self.stack, self.fwd, self.full, self.samples = stack, fwd, set(full), samples
        self.rng = np.random.default_rng(seed)
        self.amax = {}
        self.checked = []

    def __call__(self, b, l, dy):
        torch.cuda.synchronize()
        s = self.stack
        st = s.state
        r = s.rec(b, l, R_DY)
        sdy = f32(st.scale)[r]
        dyb = bits16(dy)
        oq, oqt, ady, sidy = oracle.cast_transpose_amax(dyb, sdy, oracle.E5M2)
        np.testing.assert_array_equal(bits8(s.qdy[l].data), oq, err_msg=f"dY codes b{b} l{l}")
        np.testing.assert_array_equal(bits8(s.qdy[l].data_t), oqt, err_msg=f"dY^T b{b} l{l}")
        assert f32_bits(st.amax_cur)[r] == np.float32(ady).view(np.uint32), f"dY amax b{b} l{l}"
        assert f32_bits(s.qdy[l].scale_inv)[0] == np.float32(sidy).view(np.uint32)
        self.amax[r] = ady
        if s.grad_b[b][l] is not None:
            ref = oracle.dbias(dyb).astype(np.float64)
            got = f32(s.grad_b[b][l]).astype(np.float64)
            absum = np.abs(bf16_values(dyb)).sum(axis=0)
            bound = (np.ceil(M / 128) + 13) * 2.0 ** -24 * absum
            assert (np.abs(got - ref) <= bound).all(), f"dbias b{b} l{l}"
        if b in self.full:
            ox, oxt, six = self.fwd.x_codes[(b, l)]
            ow, owt, siw = self.fwd.w_codes[(b, l)]
            n = self.samples
            fin = s.dx[l].shape[1]
            fout = dy.shape[1]
            rr, cc = self.rng.integers(0, M, n), self.rng.integers(0, fin, n)
            ref = oracle.gemm_nt_sampled(oq, 1, owt, 0, sidy, siw, rr, cc)
            assert_gemm_close(bf16_values(bits16(s.dx[l]))[rr, cc], bf16_values(ref),
                              f"dgrad b{b} l{l}")
            rn, ck = self.rng.integers(0, fout, n), self.rng.integers(0, fin, n)
            ref = oracle.gemm_nt_sampled(oqt, 1, oxt, 0, sidy, six, rn, ck,
                                         out_kind=oracle.OUT_FP32)
            assert_gemm_close(f32(s.grad_w[b][l])[rn, ck].astype(np.float64),
                              ref.astype(np.float64), f"wgrad b{b} l{l}")
            self.checked.append((b, l))


def _x(seed):
    return workloads.uniform_bf16((M, H), seed).to(DEV)


def _moved_where_finite(pre, stack):
    """After an update from the initial scales: every record whose recorded
    amax was finite and positive has a new scale; a record whose amax was
    not finite keeps its scale.  Returns the number of non-finite records."""
    cur, scale = pre["amax_cur"], f32(stack.state.scale)
    fin = np.isfinite(cur) & (cur > 0)
    assert (scale[fin] != 1.0).all() and (scale[~fin] == 1.0).all()
    return int((~np.isfinite(cur)).sum())


def test_two_block_forward_every_linear_and_the_update_against_the_oracle():
    """The first forward runs at the initial scale 1: the E4M3 products then
    sum exactly on a coarse dyadic grid, so a modulation divisor (a linear
    output plus bias) can cancel to exactly zero and the unsanitised
    modulation gives infinities -- the oracle gives the same, bit for bit,
    and the update keeps those records' scales."""
    stack = ToyStack(dsl, workloads, 2, modulate="page")
    chk = ForwardCheck(stack)
    stack.probe = chk
    stack.forward(_x(workloads.SEED_X), fused=True, update=False)
    assert len(chk.w_codes) == 12
    pre = _update_and_check(stack, chk.amax)
    n = _moved_where_finite(pre, stack)
    print(f"records with a non-finite amax after the first forward: {n} of {stack.state.T}")


def test_cached_weights_second_micro_batch_against_the_oracle():
    """Micro-batch 1 casts the weights (flag 0); after the scale update,
    micro-batch 2 keeps them (flag 1).  On micro-batch 2 every product must
    equal the oracle's product of fresh input codes with the CACHED weight
    codes and the weights' scale-inverse snapshot of micro-batch 1 (not the
    updated weight scale), no weight amax is recorded, and the update after
    it matches the oracle for all 24 records (the weights' histories take a
    zero)."""
    stack = ToyStack(dsl, workloads, 2, modulate="page")
    chk = ForwardCheck(stack)
    stack.probe = chk
    stack.flag.fill_(0)
    stack.forward(_x(11), fused=True, update=False)
    _moved_where_finite(_update_and_check(stack, chk.amax), stack)
    w_scales_after_1 = f32(stack.state.scale)[[stack.rec(b, l, R_W) for b in range(2)
                                               for l in range(6)]]
    assert (w_scales_after_1 != 1.0).all()                # the recipe moved the weight scales ...
    chk.cached = True
    stack.flag.fill_(1)
    stack.forward(_x(12), fused=True, update=False)       # ... but the GEMMs use the snapshots
    for (b, l), (_, _, siw) in chk.w_codes.items():
        assert siw == np.float32(1.0)                     # micro-batch 1 cast with the initial scale
    pre = _update_and_check(stack, chk.amax)
    for b in range(2):
        for l in range(6):
            assert pre["amax_cur"][stack.rec(b, l, R_W)] == 0.0


def test_one_graph_serves_both_micro_batches():
    """The 2-block forward captured once and replayed with the flag flipped
    on the device gives the eager run's bits and state for both micro-batches."""
    x1, x2 = _x(11), _x(12)
    eager = ToyStack(dsl, workloads, 2, modulate="page")
    outs = []
    for xv, fl in ((x1, 0), (x2, 1)):
        eager.flag.fill_(fl)
        outs.append(eager.forward(xv, fused=True).clone())
    torch.cuda.synchronize()
    g = ToyStack(dsl, workloads, 2, modulate="page")
    warm = ToyStack(dsl, workloads, 1, modulate="page")
    xin = torch.empty_like(x1)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):                 # first launches on a side stream
        warm.forward(x1, fused=True)
        warm.forward(x1, fused=False)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        gout = g.forward(xin, fused=True)
    for rep, (xv, fl) in enumerate(((x1, 0), (x2, 1))):
        xin.copy_(xv)
        g.flag.fill_(fl)
        graph.replay()
        torch.cuda.synchronize()
        junk = torch.randn(256, 256, device=DEV) @ torch.randn(256, 256, device=DEV)
        torch.cuda.synchronize()
        del junk
        assert torch.equal(gout.view(torch.int16), outs[rep].view(torch.int16)), f"micro-batch {rep + 1}"
    for name in ("amax_history", "scale", "scale_inv"):
        assert torch.equal(getattr(g.state, name), getattr(eager.state, name)), name


@pytest.mark.parametrize("modulate", ["page", "finite"])
def test_fused_producers_match_torch_glue(modulate):
    """Modulation and residual adds fused into the casts give the bits of
    torch glue followed by plain casts, over two steps (the second with
    updated scales), outputs and state, infinities and NaNs included."""
    x = _x(21)
    a = ToyStack(dsl, workloads, 2, modulate=modulate)
    b = ToyStack(dsl, workloads, 2, modulate=modulate)
    for _ in range(2):
        ya = a.forward(x, fused=False)
        yb = b.forward(x, fused=True)
        torch.cuda.synchronize()
        assert torch.equal(ya.view(torch.int16), yb.view(torch.int16))
    for name in ("amax_history", "scale", "scale_inv"):
        assert torch.equal(getattr(a.state, name), getattr(b.state, name)), name


@pytest.mark.parametrize("tokens", [1024, 8192])
def test_grouped_weight_casts_match_per_linear_casts(tokens):
    """A block's six weight casts in one grouped launch give the bits of six
    casts each right before its product: outputs, codes of every weight and
    the whole scale state, over two steps (the second with updated scales)
    and a third with the cached-weights flag set."""
    x = _x(23) if tokens == 8192 else _x(23)[:tokens].contiguous()
    a = ToyStack(dsl, workloads, 2, tokens=tokens, group_weight_casts=False)
    b = ToyStack(dsl, workloads, 2, tokens=tokens, group_weight_casts=True)
    for step in range(3):
        if step == 2:
            a.flag.fill_(1)
            b.flag.fill_(1)
        ya = a.forward(x)
        yb = b.forward(x)
        torch.cuda.synchronize()
        assert torch.equal(ya.view(torch.int16), yb.view(torch.int16)), f"step {step}: output"
        for blk in range(2):
            for l in range(len(a.lin)):
                assert torch.equal(a.qw[blk][l].data, b.qw[blk][l].data), f"step {step}: codes"
        for name in ("amax_history", "scale", "scale_inv"):
            assert torch.equal(getattr(a.state, name), getattr(b.state, name)), name


def test_graph_capture_replays_match_eager():
    """One delayed-scaling iteration of one linear (two casts, the forward
    GEMM, the scale update) captured in a HIP graph and replayed three times,
    with eager work and synchronisations between replays, matches the same
    iteration run eagerly on a separate copy of the state: nothing in the
    library allocates, synchronises or reads device memory on the host."""
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
    assert float(g_st.scale[0]) == 1.0 and float(g_st.amax_history.abs().sum()) == 0.0
    for rep in range(3):
        graph.replay()
        iteration(e_st, e_qx, e_qw, e_y)
        torch.cuda.synchronize()
        junk = torch.randn(256, 256, device=DEV) @ torch.randn(256, 256, device=DEV)
        torch.cuda.synchronize()
        del junk
        for got, want in ((g_qx.data, e_qx.data), (g_qw.data, e_qw.data), (g_qw.data_t, e_qw.data_t)):
            assert torch.equal(got, want), f"replay {rep}: codes differ"
        assert torch.equal(g_y.view(torch.int16), e_y.view(torch.int16)), f"replay {rep}: Y differs"
        for name in ("amax_history", "amax_cur", "scale", "scale_inv"):
            assert torch.equal(getattr(g_st, name), getattr(e_st, name)), f"replay {rep}: {name}"
    assert float(g_st.scale[0]) != 1.0


def test_training_step_block0_against_the_oracle():
    """A training step of a 2-block stack at full shape (HYBRID: E4M3
    inputs and fp32-sourced weights, E5M2 output gradients).  The first step
    moves every scale off its initial 1; on the second, every linear's
    forward casts and products (both blocks), every gradient cast with its
    fused bias gradient (both blocks), and block 0's dgrad and wgrad
    products are checked against the oracle, and then the one update over
    all 36 records.  The stack uses the library's finite modulation, so a
    zero divisor cannot turn the gradients into NaNs."""
    stack = ToyStack(dsl, workloads, 2, train=True, modulate="finite")
    x = _x(workloads.SEED_X)
    target = workloads.uniform_bf16((M, H), workloads.SEED_X + 1).to(DEV)
    stack.train_step(x, target)                         # step 1 (scales start at 1)
    torch.cuda.synchronize()
    assert (f32(stack.state.scale)[[stack.rec(b, l, R_DY) for b in range(2)
                                    for l in range(6)]] != 1.0).all()
    fwd = ForwardCheck(stack)
    bwd = BackwardCheck(stack, fwd, full=(0,))
    stack.probe, stack.probe_bwd = fwd, bwd
    stack.refresh_bias_copies()
    out = stack.forward(x, fused=True, update=False)
    g = torch.sub(out, target).mul_(2.0 / out.numel())
    stack.backward(g)
    assert sorted(bwd.checked) == [(0, l) for l in range(6)]
    want = dict(fwd.amax)
    want.update(bwd.amax)
    assert len(want) == 36
    _update_and_check(stack, want)
    for l in range(6):
        assert float(stack.grad_w[0][l].abs().max()) > 0.0   # gradients reached block 0


@pytest.mark.parametrize("modulate", ["page", "finite"])
def test_full_32_block_forward_late_records_against_the_oracle(modulate):
    """The whole 32-block forward with fused producers: the last block's six
    linears are checked against the oracle (their inputs carry 31 blocks of
    residual growth), then the update over all 384 records against the
    oracle's update of the same state.  The output's non-finite count is
    reported for both modulations (the residual adds are not sanitised by
    either, so an overflow there would show)."""
    stack = ToyStack(dsl, workloads, 32, modulate=modulate)
    chk = ForwardCheck(stack, blocks={31})
    stack.probe = chk
    out = stack.forward(_x(workloads.SEED_X), fused=True, update=False)
    torch.cuda.synchronize()
    assert len(chk.w_codes) == 6
    _update_and_check(stack, chk.amax)
    nonfinite = int((~torch.isfinite(out.float())).sum())
    print(f"32-block forward ({modulate} modulation): {nonfinite} non-finite of "
          f"{out.numel()} outputs")



def test_training_step_graph_replays_match_eager_steps():
    """Two identical 2-block training stacks at full shape, each with a
    capturable AdamW: A takes eager steps; B takes its first two steps as the
    capture's warm-up and then replays its captured step.  After the third
    and fourth steps (eager work and a synchronisation between the replays)
    B's fp32 weights, weight and bias gradients and whole scale state equal
    A's bit for bit."""
    from bench import _adamw, capture_train_step

    def make():
        stack = ToyStack(dsl, workloads, 2, train=True, modulate="finite")
        params = []
        for b in range(2):
            for l in range(6):
                w = stack.w[b][l]
                w.requires_grad_(True)
                w.grad = stack.grad_w[b][l]
                params.append(w)
                if stack.b32[b][l] is not None:
                    bb = stack.b32[b][l]
                    bb.requires_grad_(True)
                    bb.grad = stack.grad_b[b][l]
                    params.append(bb)
        return stack, _adamw(params, capturable=True)

    x = _x(workloads.SEED_X)
    target = workloads.uniform_bf16((M, H), workloads.SEED_X + 1).to(DEV)
    a, opt_a = make()
    b, opt_b = make()

    def same(step):
        torch.cuda.synchronize()
        for blk in range(2):
            for l in range(6):
                assert torch.equal(a.w[blk][l].view(torch.int32), b.w[blk][l].view(torch.int32)), \
                    (step, blk, l)
                assert torch.equal(a.grad_w[blk][l].view(torch.int32),
                                   b.grad_w[blk][l].view(torch.int32)), (step, blk, l)
                if a.grad_b[blk][l] is not None:
                    assert torch.equal(a.grad_b[blk][l].view(torch.int32),
                                       b.grad_b[blk][l].view(torch.int32)), (step, blk, l)
        for name in ("amax_history", "amax_cur", "scale", "scale_inv"):
            assert torch.equal(getattr(a.state, name).view(torch.int32),
                               getattr(b.state, name).view(torch.int32)), (step, name)

    with torch.no_grad():
        for _ in range(2):
            a.train_step(x, target, opt_a)
        graph = capture_train_step(b, x, target, opt_b, warmup=2)
        same(2)
        a.train_step(x, target, opt_a)
        graph.replay()
        same(3)
        junk = torch.randn(4096, 4096, device=DEV) @ torch.randn(4096, 4096, device=DEV)
        torch.cuda.synchronize()
        del junk
        a.train_step(x, target, opt_a)
        graph.replay()
        same(4)
