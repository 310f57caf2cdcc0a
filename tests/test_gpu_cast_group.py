"""GPU parity: fp8_cast_transpose_amax_group, several casts in one launch,
through the C ABI.  Each item must come out exactly as the per-tensor cast
makes it (codes, transposed codes, amax, scale-inverse, bit for bit), for
bf16 and fp32 sources, both formats, every output layout, ragged and strided
sources and an empty item; one item is also checked against the oracle
directly.  The no-op flag skips every item, and a captured group replays to
the eager bits."""
import numpy as np
import pytest
import torch

import delayed_scaling_linear_amd as dsl
import oracle
import workloads
from tests.gpu_util import DEV, bits16, bits8, f32_bits

pytestmark = pytest.mark.gpu

# (rows, cols, extra columns of row stride): whole tiles, ragged tiles, a
# strided source, one row of tiles, an empty tensor
SHAPES = [(256, 384, 0), (144, 272, 0), (512, 128, 64), (128, 1040, 0), (0, 256, 0),
          (400, 48, 16)]


def _source(rows, cols, pad, dtype, seed):
    g = torch.Generator().manual_seed(seed)
    full = torch.randn(rows, cols + pad, generator=g) * float(2.0 ** (seed % 7 - 3))
    if rows:
        full[0, 0] = float(seed + 1) * 37.0          # a distinct amax per item
    return full.to(dtype)[:, :cols].to(DEV)


def _out(rows, cols, fmt, q, qt):
    out = dsl.Float8Tensor.empty(rows, cols, fmt, data=q, transpose=qt, device=DEV)
    if q:
        out.data.fill_(0xAA)
    if qt:
        out.data_t.fill_(0xAA)
    out.scale_inv.fill_(-1.0)
    return out


def _same(a, b, what):
    if a is None:
        assert b is None
        return
    assert torch.equal(a, b), what


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("fmt", [oracle.E4M3, oracle.E5M2])
@pytest.mark.parametrize("q,qt", [(True, True), (True, False), (False, True)])
def test_group_matches_one_cast_per_tensor(dtype, fmt, q, qt):
    xs = [_source(r, c, p, dtype, 40 + k) for k, (r, c, p) in enumerate(SHAPES)]
    scales = [torch.tensor([v], device=DEV) for v in (1.0, 448.0 / 300.0, 0.5, 3.0, 2.0, 0.125)]
    print(f"group {dtype} fmt={fmt} q={q} qt={qt}: {len(xs)} items", flush=True)
    grp = [(_out(x.shape[0], x.shape[1], fmt, q, qt), torch.zeros(1, device=DEV)) for x in xs]
    one = [(_out(x.shape[0], x.shape[1], fmt, q, qt), torch.zeros(1, device=DEV)) for x in xs]
    dsl.fp8_cast_transpose_amax_group([(x, s, o, a) for x, s, (o, a) in zip(xs, scales, grp)])
    for x, s, (o, a) in zip(xs, scales, one):
        dsl.fp8_cast_transpose_amax(x, s, o, a)
    torch.cuda.synchronize()
    for k, ((og, ag), (oo, ao)) in enumerate(zip(grp, one)):
        _same(og.data, oo.data, f"item {k}: codes")
        _same(og.data_t, oo.data_t, f"item {k}: transposed codes")
        assert torch.equal(ag.view(torch.int32), ao.view(torch.int32)), f"item {k}: amax"
        assert torch.equal(og.scale_inv.view(torch.int32), oo.scale_inv.view(torch.int32)), \
            f"item {k}: scale_inv"
    # one item straight against the oracle
    x, s, (o, a) = xs[1], scales[1], grp[1]
    src = bits16(x.cpu()) if dtype == torch.bfloat16 else x.cpu().numpy()
    oq, oqt, oamax, osinv = oracle.cast_transpose_amax(src, float(s[0]), fmt, want_q=q, want_qt=qt)
    if q:
        np.testing.assert_array_equal(bits8(o.data), oq)
    if qt:
        np.testing.assert_array_equal(bits8(o.data_t), oqt)
    assert f32_bits(a)[0] == np.float32(oamax).view(np.uint32)
    assert f32_bits(o.scale_inv)[0] == np.float32(osinv).view(np.uint32)


def test_noop_flag_skips_every_item():
    xs = [_source(r, c, p, torch.bfloat16, 60 + k) for k, (r, c, p) in enumerate(SHAPES[:4])]
    s = torch.ones(1, device=DEV)
    items = [(x, s, _out(x.shape[0], x.shape[1], oracle.E4M3, True, True),
              torch.full((1,), 5.0, device=DEV)) for x in xs]
    flag = torch.ones(1, dtype=torch.int32, device=DEV)
    dsl.fp8_cast_transpose_amax_group(items, noop_flag=flag)
    torch.cuda.synchronize()
    for _, _, o, a in items:
        assert int((o.data != 0xAA).sum()) == 0 and int((o.data_t != 0xAA).sum()) == 0
        assert float(a[0]) == 5.0 and float(o.scale_inv[0]) == -1.0
    flag.zero_()
    dsl.fp8_cast_transpose_amax_group(items, noop_flag=flag)
    torch.cuda.synchronize()
    assert all(float(o.scale_inv[0]) == 1.0 for _, _, o, _ in items)


def test_toy_block_weights_in_one_launch_and_a_graph_replay():
    """The six fp32 weights of the toy block (83.9M elements) as one group,
    against six casts; then the group captured in a HIP graph, replayed
    three times (eager work and a synchronisation between replays) on fresh
    outputs, matching the eager bits each time."""
    g = torch.Generator(device=DEV).manual_seed(3)
    ws = [torch.randn(fout, fin, generator=g, device=DEV) * 0.02
          for fin, fout, _ in workloads.toy_block_linears()]
    scales = [torch.tensor([448.0 / float(w.abs().max())], device=DEV) for w in ws]
    grp = [(_out(w.shape[0], w.shape[1], oracle.E4M3, True, True), torch.zeros(1, device=DEV))
           for w in ws]
    one = [(_out(w.shape[0], w.shape[1], oracle.E4M3, True, True), torch.zeros(1, device=DEV))
           for w in ws]
    items = [(w, s, o, a) for w, s, (o, a) in zip(ws, scales, grp)]
    dsl.fp8_cast_transpose_amax_group(items)
    for w, s, (o, a) in zip(ws, scales, one):
        dsl.fp8_cast_transpose_amax(w, s, o, a)
    torch.cuda.synchronize()
    for (og, ag), (oo, ao) in zip(grp, one):
        assert torch.equal(og.data, oo.data) and torch.equal(og.data_t, oo.data_t)
        assert torch.equal(ag, ao) and torch.equal(og.scale_inv, oo.scale_inv)
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        dsl.fp8_cast_transpose_amax_group(items)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        dsl.fp8_cast_transpose_amax_group(items)
    for rep in range(3):
        for o, a in grp:
            o.data.fill_(0xAA)
            o.data_t.fill_(0xAA)
            a.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        junk = torch.randn(256, 256, device=DEV) @ torch.randn(256, 256, device=DEV)
        torch.cuda.synchronize()
        del junk
        for (og, ag), (oo, ao) in zip(grp, one):
            assert torch.equal(og.data, oo.data), f"replay {rep}: codes"
            assert torch.equal(og.data_t, oo.data_t), f"replay {rep}: transposed codes"
            assert torch.equal(ag, ao), f"replay {rep}: amax"
