"""Benchmark of the delayed-scaling FP8 linear hot path on one MI355X.

A step is one pass of the whole path over one batch of the toy transformer's
MLP layer (X [8192, 2048], W [8192, 2048], dY [8192, 8192], HYBRID format,
history 16):

    cast X (E4M3, codes + transpose + amax)   cast W (E4M3, codes + transpose + amax)
    Y  = X W^T + b   (fp8_linear_fwd,   E4M3 x E4M3 -> bf16)
    cast dY (E5M2, codes + transpose + amax)
    dX = dY W        (fp8_linear_dgrad, E5M2 x E4M3 -> bf16)
    dW = dY^T X      (fp8_linear_wgrad, E5M2 x E4M3 -> fp32)
    one scale update over the three amax histories

`value` is the step's GEMM throughput (3 x 2*8192*8192*2048 FLOP per step over
the measured step time, casts and update included).  Per-kernel durations are
taken with HIP events around each launch on the launch stream inside a second
timed pass and reported as median, p10, p90 and mean over the steps (each
event pair adds a few microseconds of its own).  The roofline figures come from back-to-back launches between one
event pair (the forward GEMM at the step's shape; the cast-transpose-amax on
its own workload, bf16 [4096, 4096] with 0.1% outliers, rotating over 640 MiB
of buffers so that the 256 MiB last-level cache cannot serve it), next to a
measured device-to-device copy ceiling.

    python bench.py [--gpus 1] [--steps 50] [--warmup 10] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import torch

M, N, K = 8192, 8192, 2048
GEMM_FLOP = 2 * M * N * K
CAST_R = CAST_C = 4096
CAST_BYTES = 2 * CAST_R * CAST_C + 2 * CAST_R * CAST_C     # bf16 read + 2 FP8 writes
HBM_PEAK_GBS = 8000.0
FP8_PEAK_TFLOPS = 5000.0


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--cast-iters", type=int, default=50)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-toy-stack", action="store_true",
                   help="skip the 32-block toy-stack forward timing (eager vs HIP graph)")
    p.add_argument("--no-train-step", action="store_true",
                   help="skip the 32-block toy-stack training step (FP8 vs torch bf16 autocast)")
    p.add_argument("--probe-kernels", action="store_true",
                   help="launch the forward GEMM, the [4096,4096] cast and a 64 MiB device copy "
                        "once each (after a warm-up) and exit: the command profiled for HBM "
                        "traffic counters")
    p.add_argument("--probe-toy-stack", action="store_true",
                   help="replay the 32-block 1024-token forward graph (fused producers, cached "
                        "FP8 weights) 6 times, then run 4 training steps of the 8192-token "
                        "stack, and exit: the command profiled for the toy stack's kernel traces")
    return p.parse_args()


class Timer:
    """Event pairs around launches on the current stream; average in ms."""

    def __init__(self):
        self.pairs = {}

    def start(self, name):
        e = torch.cuda.Event(enable_timing=True)
        e.record()
        return (name, e)

    def stop(self, tok):
        name, s = tok
        e = torch.cuda.Event(enable_timing=True)
        e.record()
        self.pairs.setdefault(name, []).append((s, e))

    def stats_ms(self, name):
        """Median, p10, p90 and mean of the per-call durations (ms)."""
        v = sorted(s.elapsed_time(e) for s, e in self.pairs[name])
        q = lambda f: v[min(len(v) - 1, int(round(f * (len(v) - 1))))]
        return q(0.5), q(0.1), q(0.9), sum(v) / len(v)


def gpu_step(dsl, st, t: Timer | None):
    def run(name, fn, *a):
        tok = t.start(name) if t else None
        fn(*a)
        if t:
            t.stop(tok)

    g = st["state"]
    run("cast_x", dsl.fp8_cast_transpose_amax, st["x"], g.scale[0:1], st["qx"], g.amax_cur[0:1])
    run("cast_w", dsl.fp8_cast_transpose_amax, st["w"], g.scale[1:2], st["qw"], g.amax_cur[1:2])
    run("gemm_fwd", dsl.fp8_linear_fwd, st["qx"], st["qw"], st["b"], st["y"])
    run("cast_dy", dsl.fp8_cast_transpose_amax, st["dy"], g.scale[2:3], st["qdy"], g.amax_cur[2:3])
    run("gemm_dgrad", dsl.fp8_linear_dgrad, st["qdy"], st["qw"], st["dx"])
    run("gemm_wgrad", dsl.fp8_linear_wgrad, st["qdy"], st["qx"], st["dw"])
    run("scale_update", g.update)


def cast_bandwidth(dsl, workloads, iters: int):
    """bf16 [4096, 4096] -> E4M3 codes + transpose + amax, rotating over 10
    buffer sets (640 MiB, more than the 256 MiB last-level cache), with both
    source-load policies: the default entry point (non-temporal loads, what
    a training step wants; the roofline kernel) and
    fp8_cast_transpose_amax_cached (ordinary loads).  One event pair
    brackets `iters` back-to-back launches.  Returns {policy: (ms, GB/s)}."""
    dev = "cuda"
    src = workloads.cast_only().to(dev)
    nsets = 10
    xs = [src.clone() for _ in range(nsets)]
    outs = [dsl.Float8Tensor.empty(CAST_R, CAST_C, 0, device=dev) for _ in range(nsets)]
    scale = torch.tensor([448.0 / 3920.0], device=dev)
    amax = torch.zeros(1, device=dev)
    res = {}
    for _ in range(2):                        # interleaved rounds, best of each
        for name, fn in (("nontemporal", dsl.fp8_cast_transpose_amax),
                         ("cached", dsl.fp8_cast_transpose_amax_cached)):
            for i in range(nsets):            # warm-up
                fn(xs[i], scale, outs[i], amax)
            torch.cuda.synchronize()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            for i in range(iters):
                fn(xs[i % nsets], scale, outs[i % nsets], amax)
            e1.record()
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / iters
            if name not in res or ms < res[name][0]:
                res[name] = (ms, CAST_BYTES / (ms * 1e-3) / 1e9)
    del xs, outs
    torch.cuda.empty_cache()
    return res


def copy_ceiling(dsl, iters: int = 40):
    """Measured HBM ceiling at the cast's exact volume: the library's
    reference copy of 32 MiB into 32 MiB (the bytes one [4096, 4096] bf16
    cast reads and writes), rotating over 10 buffer pairs (640 MiB), best
    over workgroup counts and load policies.  Returns (GB/s, config)."""
    n = CAST_BYTES // 2
    nsets = 10
    src = [torch.empty(n, dtype=torch.uint8, device="cuda").fill_(i + 1) for i in range(nsets)]
    dst = [torch.empty(n, dtype=torch.uint8, device="cuda") for _ in range(nsets)]
    best = (0.0, None)
    for wg in (1024, 2048, 4096):
        for nt in (False, True):
            for i in range(nsets):
                dsl.fp8_reference_copy(src[i], dst[i], wg, nt)
            torch.cuda.synchronize()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            for i in range(iters):
                dsl.fp8_reference_copy(src[i % nsets], dst[i % nsets], wg, nt)
            e1.record()
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / iters
            gbs = 2 * n / (ms * 1e-3) / 1e9
            if gbs > best[0]:
                best = (gbs, {"workgroups": wg, "nontemporal": nt, "us": round(ms * 1e3, 2)})
    del src, dst
    torch.cuda.empty_cache()
    return best


def gemm_fwd_back_to_back(dsl, st, iters: int):
    """The forward GEMM alone, `iters` back-to-back launches between one event
    pair on the launch stream: its average duration per launch.  The launches
    rotate over three [8192, 8192] bf16 outputs (384 MiB, more than the
    256 MiB last-level cache), so every launch's output reaches memory as it
    does in a network, where each layer writes a buffer of its own."""
    ys = [st["y"]] + [torch.empty_like(st["y"]) for _ in range(2)]
    for i in range(3):
        dsl.fp8_linear_fwd(st["qx"], st["qw"], st["b"], ys[i])
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(iters):
        dsl.fp8_linear_fwd(st["qx"], st["qw"], st["b"], ys[i % 3])
    e1.record()
    torch.cuda.synchronize()
    del ys
    return e0.elapsed_time(e1) / iters


def dbias_cast_cost(dsl, st, iters: int = 20):
    """The dY [8192, 8192] E5M2 cast (codes + transpose + amax) back to back,
    plain and with the bias gradient fused in (fp8_cast_transpose_amax_dbias):
    what the fused column sums cost on top of the cast."""
    g = st["state"]
    dy, qdy = st["dy"], st["qdy"]
    dbias = torch.empty(N, dtype=torch.float32, device="cuda")
    ws = torch.empty(dsl.fp8_cast_dbias_workspace_bytes(M, N), dtype=torch.uint8, device="cuda")
    plain = lambda: dsl.fp8_cast_transpose_amax(dy, g.scale[2:3], qdy, g.amax_cur[2:3])
    fused = lambda: dsl.fp8_cast_transpose_amax_dbias(dy, g.scale[2:3], qdy, g.amax_cur[2:3],
                                                      dbias, ws)
    res = {}
    for _ in range(2):                        # interleaved rounds, best of each
        for name, fn in (("cast_us", plain), ("cast_dbias_us", fused)):
            for _ in range(3):
                fn()
            torch.cuda.synchronize()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(iters):
                fn()
            e1.record()
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) / iters * 1e3
            res[name] = min(res.get(name, us), us)
    return {k: round(v, 2) for k, v in res.items()}


def split_product_cost(dsl, workloads, iters: int = 20):
    """Products whose output leaves CUs idle over a long contraction, plain
    and through a workspace (split over K where the library's rule splits):
    weight gradients (fp32) of a 2048 -> 2048 linear over 16384 and 32768
    tokens and of a 2048 -> 1024 linear over 32768 tokens, and that of the
    toy block's 2048 -> 2048 linear over its 8192 tokens (which stays
    unsplit: parts 1).  Random E5M2 / E4M3 operand codes; interleaved rounds,
    best of each."""
    one = torch.ones(1, device="cuda")
    res = {}
    for name, (M_, N_, K_) in {
            "wgrad_2048x2048_k8192": (2048, 2048, 8192),
            "wgrad_2048x2048_k16384": (2048, 2048, 16384),
            "wgrad_2048x2048_k32768": (2048, 2048, 32768),
            "wgrad_1024x2048_k32768": (1024, 2048, 32768)}.items():
        a = workloads.random_fp8_codes((M_, K_), 31, 1).to("cuda")
        b = workloads.random_fp8_codes((N_, K_), 32, 0).to("cuda")
        need = dsl.fp8_gemm_workspace_bytes(M_, N_, K_)
        ws = torch.empty(max(need, 16), dtype=torch.uint8, device="cuda")
        # dW [M_, N_] = dY_t [M_, K_] . X_t [N_, K_]^T
        dyt = dsl.Float8Tensor(None, a, one, 1, K_, M_)
        xt = dsl.Float8Tensor(None, b, one, 0, K_, N_)
        dw = torch.empty(M_, N_, dtype=torch.float32, device="cuda")
        plain = lambda: dsl.fp8_linear_wgrad(dyt, xt, dw)
        split = lambda: dsl.fp8_linear_wgrad(dyt, xt, dw, workspace=ws)
        r = {"parts": need // (M_ * N_ * 4) if need else 1}
        for _ in range(2):
            for key, fn in (("plain_us", plain), ("split_us", split)):
                for _ in range(3):
                    fn()
                torch.cuda.synchronize()
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record()
                for _ in range(iters):
                    fn()
                e1.record()
                torch.cuda.synchronize()
                us = e0.elapsed_time(e1) / iters * 1e3
                r[key] = round(min(r.get(key, us), us), 2)
        r["split_tflops"] = round(2 * M_ * N_ * K_ / (r["split_us"] * 1e-6) / 1e12, 1)
        res[name] = r
        del a, b, ws, dw
    return res


def dynamic_vs_delayed(dsl, st, iters: int = 20):
    """Delayed scaling (one cast pass: codes + transpose + amax with the scale
    from earlier amaxes) against dynamic scaling (amax pass, scale, then the
    cast pass) on the step's X [8192, 2048] (E4M3) and dY [8192, 8192] (E5M2)
    casts, back to back."""
    g = st["state"]
    scale = torch.ones(1, device="cuda")
    amax = torch.zeros(1, device="cuda")
    cases = {
        "x": (lambda: dsl.fp8_cast_transpose_amax(st["x"], g.scale[0:1], st["qx"], g.amax_cur[0:1]),
              lambda: dsl.fp8_cast_transpose_dynamic(st["x"], scale, st["qx"], amax)),
        "dy": (lambda: dsl.fp8_cast_transpose_amax(st["dy"], g.scale[2:3], st["qdy"], g.amax_cur[2:3]),
               lambda: dsl.fp8_cast_transpose_dynamic(st["dy"], scale, st["qdy"], amax)),
    }
    res = {}
    for _ in range(2):
        for name, (delayed, dynamic) in cases.items():
            for kind, fn in (("delayed", delayed), ("dynamic", dynamic)):
                for _ in range(3):
                    fn()
                torch.cuda.synchronize()
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record()
                for _ in range(iters):
                    fn()
                e1.record()
                torch.cuda.synchronize()
                us = e0.elapsed_time(e1) / iters * 1e3
                key = f"{name}_{kind}_us"
                res[key] = min(res.get(key, us), us)
    return {k: round(v, 2) for k, v in res.items()}


def fp8_output_forward(dsl, st, iters: int = 20):
    """The forward product with an FP8 output and its amax (torch._scaled_mm
    with an FP8 out_dtype) at the step's shape [8192, 2048] x [8192, 2048]^T,
    against what it replaces: the bf16 output followed by a codes-only cast
    of it (which takes the amax), back to back."""
    M, N = st["y"].shape
    g = st["state"]
    qy = dsl.Float8Tensor.empty(M, N, 0, transpose=False, device="cuda")
    scale = torch.tensor([448.0 / 6.0], device="cuda")
    amax = torch.zeros(1, device="cuda")
    cases = {
        "bf16_out_then_cast": lambda: (dsl.fp8_linear_fwd(st["qx"], st["qw"], st["b"], st["y"]),
                                       dsl.fp8_cast_transpose_amax(st["y"], scale, qy, amax)),
        "fp8_out_fused": lambda: dsl.fp8_linear_fwd_fp8out(st["qx"], st["qw"], st["b"], scale,
                                                           qy, amax),
    }
    res = {}
    for _ in range(2):
        for name, fn in cases.items():
            for _ in range(3):
                fn()
            torch.cuda.synchronize()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(iters):
                fn()
            e1.record()
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) / iters * 1e3
            res[name + "_us"] = min(res.get(name + "_us", us), us)
    del g
    return {k: round(v, 2) for k, v in res.items()}


def producer_cast_cost(dsl, workloads, iters: int = 20):
    """The toy block's glue in front of a linear at its real shapes, as torch
    elementwise code followed by the cast, and fused into one pass
    (fp8_produce_cast_transpose_amax): the modulation, the input times one
    column slice of the [8192, 12288] modulation output divided by another,
    and the residual add of the first 2048 columns of the [8192, 6144]
    self-attention output; E4M3 codes + transpose + amax of the result each
    time."""
    dev = "cuda"
    H, Mt = workloads.HIDDEN, workloads.TOKENS
    g = torch.Generator(device=dev).manual_seed(30)
    mod = (torch.randn(Mt, 6 * H, generator=g, device=dev) * 0.5).to(torch.bfloat16)
    qkv = (torch.randn(Mt, 3 * H, generator=g, device=dev) * 0.02).to(torch.bfloat16)
    x = torch.rand(Mt, H, generator=g, device=dev).to(torch.bfloat16)
    shift, scale_m, r = mod[:, :H], mod[:, H:2 * H], qkv[:, :H]   # gain, divisor, residual
    y = torch.empty_like(x)
    out = dsl.Float8Tensor.empty(Mt, H, 0, device=dev)
    s = torch.tensor([3.5], device=dev)
    amax = torch.zeros(1, device=dev)

    def torch_mod():
        t = (shift.float() * x.float() / scale_m.float()).to(torch.bfloat16)
        dsl.fp8_cast_transpose_amax(t, s, out, amax)

    def torch_add():
        dsl.fp8_cast_transpose_amax(x + r, s, out, amax)

    fused_mod = lambda: dsl.fp8_produce_cast_transpose_amax(dsl.PRODUCE_MODULATE, x, shift,
                                                            scale_m, y, s, out, amax)
    fused_add = lambda: dsl.fp8_produce_cast_transpose_amax(dsl.PRODUCE_ADD, x, r, None, y, s,
                                                            out, amax)
    res = {}
    for _ in range(2):
        for name, fn in (("modulate_torch_then_cast_us", torch_mod), ("modulate_fused_us", fused_mod),
                         ("add_torch_then_cast_us", torch_add), ("add_fused_us", fused_add)):
            for _ in range(3):
                fn()
            torch.cuda.synchronize()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(iters):
                fn()
            e1.record()
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) / iters * 1e3
            res[name] = min(res.get(name, us), us)
    return {k: round(v, 2) for k, v in res.items()}


# ------------------------------------------------------------- toy stack ----

# The six linears of one toy block, by position in workloads.toy_block_linears().
L_MOD, L_SELF, L_CROSS_Q, L_CROSS_KV, L_UP, L_DOWN = range(6)
# Delayed-scaling records of one linear: its input, its weight and (when
# training) its output gradient.
R_X, R_W, R_DY = 0, 1, 2


class ToyStack:
    """The toy transformer stack of "CPU Overhead of te.Linear FP8 Layers"
    (hidden 2048, batch 8 x seq 1024 = 8192 tokens, mlp_ratio 4) run through
    the library: every linear casts its input and weight with delayed scaling
    and multiplies in FP8; when, its output gradient is cast to E5M2
    (with the bias gradient fused in for the biased linears) and dgrad and
    wgrad run from the cached transposes.  One scale update per step covers
    every record.

    A block acts on the residual stream h (width H) through its six linears
    (in -> out features, bias):

        0  2048 -> 12288 +b   modulation: h <- out[:, :H] * h / out[:, H:2H]
        1  2048 ->  6144      h <- h + out[:, :H]
        2  2048 ->  2048      \\  both read the same h;
        3  2048 ->  4096      /   h <- (h + out2) + out3[:, :H]
        4  2048 ->  8192 +b   u = out
        5  8192 ->  2048 +b   of u;  h <- h + out

    `fused` computes the modulation and residual adds inside the casts of the
    linear inputs they produce (fp8_produce_cast_transpose_amax); otherwise
    they run as torch elementwise ops followed by plain casts.

    `modulate="page"` is the page's modulation, unsanitised: a divisor that
    is exactly zero gives infinities (the casts saturate them, residual sums
    can turn them into NaNs).  At the initial scale 1 the E4M3 products sum
    exactly on a coarse grid, so linear output + bf16 bias cancels to zero a
    few times in 10^6; a record whose amax is then infinite keeps scale 1
    under delayed scaling, so the stack never leaves it.  `modulate="finite"`
    (this library's addition, on no page) replaces non-finite quotients by
    +0; the timed workloads use it.

    `group_weight_casts` casts a block's six weights in one launch at the
    block's start (fp8_cast_transpose_amax_group) instead of each right before
    its product; by default for 2048 tokens or fewer.  Measured on MI355X: at
    1024 tokens the launches are the cost (fused graph with cached weights
    6.59 -> 6.36 ms); at 8192 tokens a weight's codes cast right before its
    product are still in the last-level cache when the product reads them,
    and grouping loses that (fused graph 23.3 -> 26.2 ms).

    `train` keeps what the backward needs (every FP8 input with its
    transpose, the block inputs and modulation outputs) and holds fp32 master
    weights (the FP8 run of the page keeps fp32 parameters) whose FP8 casts
    read fp32 directly.
    """

    def __init__(self, dsl, workloads, blocks: int, *, train: bool = False, dev: str = "cuda",
                 seed: int = 20, weights=None, modulate: str = "finite", tokens: int = 0,
                 group_weight_casts=None):
        self.dsl, self.blocks, self.train, self.dev = dsl, blocks, train, dev
        if modulate not in ("page", "finite"):
            raise ValueError("modulate must be 'page' or 'finite'")
        self.finite = modulate == "finite"
        self.mod_op = dsl.PRODUCE_MODULATE_FINITE if self.finite else dsl.PRODUCE_MODULATE
        self.H, self.M = workloads.HIDDEN, tokens or workloads.TOKENS
        self.group_w = self.M <= 2048 if group_weight_casts is None else bool(group_weight_casts)
        self.lin = workloads.toy_block_linears()
        nl = len(self.lin)
        self.R = 3 if train else 2
        fmts = ([dsl.E4M3, dsl.E4M3, dsl.E5M2][:self.R]) * (nl * blocks)
        self.state = dsl.DelayedScalingState(fmts, device=dev)
        self.flag = torch.zeros(1, dtype=torch.int32, device=dev)   # 1: keep cached FP8 weights
        # Optional checks called after each linear's forward product,
        # probe(b, l, y), and after its backward, probe_bwd(b, l, dy); the
        # bf16 tensor each input cast read is kept in last_in[l].
        self.probe = self.probe_bwd = None
        self.last_in = [None] * len(workloads.toy_block_linears())
        M, H = self.M, self.H
        wdt = torch.float32 if train else torch.bfloat16
        if weights is None:
            gen = torch.Generator(device=dev).manual_seed(seed)
            weights = []
            for _ in range(blocks):
                ws = []
                for fin, fout, hb in self.lin:
                    w = torch.randn(fout, fin, generator=gen, device=dev) * 0.02
                    b = torch.randn(fout, generator=gen, device=dev) * 0.02 if hb else None
                    ws.append((w, b))
                weights.append(ws)
        self.w = [[w.to(wdt) for w, _ in ws] for ws in weights]
        self.b32 = [[None if b is None else b.float() for _, b in ws] for ws in weights]
        self.b16 = [[None if b is None else b.to(torch.bfloat16) for _, b in ws] for ws in weights]
        self.qw = [[dsl.Float8Tensor.empty(fout, fin, dsl.E4M3, transpose=train, device=dev)
                    for fin, fout, _ in self.lin] for _ in range(blocks)]
        per_block = lambda make: [make() for _ in range(blocks)] if train else [make()] * blocks
        self.qx = [per_block(lambda fin=fin: dsl.Float8Tensor.empty(M, fin, dsl.E4M3,
                                                                    transpose=train, device=dev))
                   for fin, _, _ in self.lin]                         # qx[l][b]
        bf = lambda n: torch.empty(M, n, dtype=torch.bfloat16, device=dev)
        self.out = [bf(fout) for _, fout, _ in self.lin]
        self.mod_out = per_block(lambda: bf(6 * H)) if train else [self.out[L_MOD]] * blocks
        self.h_in = per_block(lambda: bf(H)) if train else None       # block inputs
        self.hbuf = [bf(H) for _ in range(4)]
        # One workspace for the products that alone would leave CUs idle
        # (split over K); the stack's calls are ordered on one stream.
        shapes = [(M, fout, fin) for fin, fout, _ in self.lin]
        if train:
            shapes += [(M, fin, fout) for fin, fout, _ in self.lin]     # dgrad
            shapes += [(fout, fin, M) for fin, fout, _ in self.lin]     # wgrad
        gbytes = max(dsl.fp8_gemm_workspace_bytes(*s) for s in shapes)
        self.gemm_ws = torch.empty(gbytes, dtype=torch.uint8, device=dev) if gbytes else None
        if train:
            self.grad_w = [[torch.zeros_like(w) for w in ws] for ws in self.w]
            self.grad_b = [[None if b is None else torch.zeros_like(b) for b in bs]
                           for bs in self.b32]
            # output gradients, zero beyond the columns the block reads
            self.dy = [torch.zeros(M, fout, dtype=torch.bfloat16, device=dev)
                       for _, fout, _ in self.lin]
            self.qdy = [dsl.Float8Tensor.empty(M, fout, dsl.E5M2, device=dev)
                        for _, fout, _ in self.lin]
            self.dx = [bf(fin) for fin, _, _ in self.lin]
            self.g_h0 = bf(H)                    # gradient at a block's input, direct part
            ws_bytes = max(dsl.fp8_cast_dbias_workspace_bytes(M, fout) for _, fout, _ in self.lin)
            self.ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)

    def rec(self, b: int, l: int, kind: int) -> int:
        return (len(self.lin) * b + l) * self.R + kind

    def _sl(self, t, r):
        return t[r:r + 1]

    def refresh_bias_copies(self):
        """bf16 copies of the fp32 master biases for the forward GEMMs."""
        dst = [b for bs in self.b16 for b in bs if b is not None]
        src = [b for bs in self.b32 for b in bs if b is not None]
        torch._foreach_copy_(dst, src)

    # -- forward --
    def _cast_in(self, b, l, x):
        r, st = self.rec(b, l, R_X), self.state
        self.last_in[l] = x
        self.dsl.fp8_cast_transpose_amax(x, self._sl(st.scale, r), self.qx[l][b],
                                         self._sl(st.amax_cur, r))

    def _cast_weights(self, b):
        """The six weight casts of block b in one launch (skipped on the
        device when the cache flag is set), when they are grouped."""
        if not self.group_w:
            return
        st = self.state
        self.dsl.fp8_cast_transpose_amax_group(
            [(self.w[b][l], self._sl(st.scale, self.rec(b, l, R_W)), self.qw[b][l],
              self._sl(st.amax_cur, self.rec(b, l, R_W))) for l in range(len(self.lin))],
            noop_flag=self.flag)

    def _linear(self, b, l, out=None):
        """The FP8 product of linear l of block b, its input already cast; its
        weight cast first unless the block's weights were cast as a group
        (either way skipped on the device when the cache flag is set)."""
        qw = self.qw[b][l]
        if not self.group_w:
            r, st = self.rec(b, l, R_W), self.state
            self.dsl.fp8_cast_transpose_amax(self.w[b][l], self._sl(st.scale, r), qw,
                                             self._sl(st.amax_cur, r), noop_flag=self.flag)
        y = self.out[l] if out is None else out
        self.dsl.fp8_linear_fwd(self.qx[l][b], qw, self.b16[b][l], y, workspace=self.gemm_ws)
        if self.probe is not None:
            self.probe(b, l, y)
        return y

    def _produce(self, b, l, op, x, a, c, out, fused):
        """out = op(x, a, c) in bf16, cast as the input of linear l of block b."""
        dsl = self.dsl
        if fused:
            r, st = self.rec(b, l, R_X), self.state
            self.last_in[l] = out
            dsl.fp8_produce_cast_transpose_amax(op, x, a, c, out, self._sl(st.scale, r),
                                                self.qx[l][b], self._sl(st.amax_cur, r))
            return out
        if op in (dsl.PRODUCE_MODULATE, dsl.PRODUCE_MODULATE_FINITE):
            out.copy_(torch.div(a.float() * x.float(), c.float()))
            if op == dsl.PRODUCE_MODULATE_FINITE:
                torch.nan_to_num_(out, nan=0.0, posinf=0.0, neginf=0.0)
        elif op == dsl.PRODUCE_ADD:
            torch.add(x, a, out=out)
        else:
            torch.add(torch.add(x, a), c, out=out)
        self._cast_in(b, l, out)
        return out

    def forward(self, x, fused: bool = True, update: bool = True):
        dsl, H = self.dsl, self.H
        h1, h2, h3, hn = self.hbuf
        if self.train:
            self.h_in[0].copy_(x)
            x = self.h_in[0]
        self._cast_in(0, L_MOD, x)
        h = x
        for b in range(self.blocks):
            self._cast_weights(b)
            m = self._linear(b, L_MOD, out=self.mod_out[b])
            self._produce(b, L_SELF, self.mod_op, h, m[:, :H], m[:, H:2 * H], h1, fused)
            s = self._linear(b, L_SELF)
            self._produce(b, L_CROSS_Q, dsl.PRODUCE_ADD, h1, s[:, :H], None, h2, fused)
            self._cast_in(b, L_CROSS_KV, h2)
            q = self._linear(b, L_CROSS_Q)
            k = self._linear(b, L_CROSS_KV)
            self._produce(b, L_UP, dsl.PRODUCE_ADD2, h2, q, k[:, :H], h3, fused)
            u = self._linear(b, L_UP)
            self._cast_in(b, L_DOWN, u)
            o = self._linear(b, L_DOWN)
            if b + 1 < self.blocks:
                nxt = self.h_in[b + 1] if self.train else hn
                h = self._produce(b + 1, L_MOD, dsl.PRODUCE_ADD, h3, o, None, nxt, fused)
            else:
                h = h3 + o
        if update:
            self.state.update()
        return h

    # -- backward (train) --
    def _linear_bwd(self, b, l, dy):
        """Output gradient dy [M, out] of linear l of block b: its E5M2 cast
        (bias gradient fused for the biased linears), dgrad from the cached
        weight transpose into self.dx[l], wgrad (fp32) into grad_w."""
        dsl, st = self.dsl, self.state
        r = self.rec(b, l, R_DY)
        if self.grad_b[b][l] is not None:
            dsl.fp8_cast_transpose_amax_dbias(dy, self._sl(st.scale, r), self.qdy[l],
                                              self._sl(st.amax_cur, r), self.grad_b[b][l],
                                              self.ws)
        else:
            dsl.fp8_cast_transpose_amax(dy, self._sl(st.scale, r), self.qdy[l],
                                        self._sl(st.amax_cur, r))
        dsl.fp8_linear_dgrad(self.qdy[l], self.qw[b][l], self.dx[l], workspace=self.gemm_ws)
        dsl.fp8_linear_wgrad(self.qdy[l], self.qx[l][b], self.grad_w[b][l],
                             workspace=self.gemm_ws)
        if self.probe_bwd is not None:
            self.probe_bwd(b, l, dy)
        return self.dx[l]

    def backward(self, g):
        """g: bf16 [M, H], the loss gradient at the stack's output.  Returns
        the gradient at the stack's input."""
        H = self.H
        for b in reversed(range(self.blocks)):
            du = self._linear_bwd(b, L_DOWN, g)
            # The residual sums go straight into the first H columns of the
            # zero-padded output gradients of the two projections that read
            # only those columns (no copies); each bf16 add rounds as before.
            g2 = self.dy[L_CROSS_KV][:, :H]
            torch.add(g, self._linear_bwd(b, L_UP, du), out=g2)
            dk = self._linear_bwd(b, L_CROSS_KV, self.dy[L_CROSS_KV])
            g3 = self.dy[L_SELF][:, :H]
            torch.add(g2, self._linear_bwd(b, L_CROSS_Q, g2), out=g3)
            g3.add_(dk)
            g = g3 + self._linear_bwd(b, L_SELF, self.dy[L_SELF])
            # modulation h1 = gain * h0 / div: one library pass writes the
            # gradients of gain and div into the modulation linear's output
            # gradient and that of h0 into g_h0 (zero where the finite
            # modulation replaced a non-finite quotient)
            m = self.mod_out[b]
            dmod = self.dy[L_MOD]
            self.dsl.fp8_produce_modulate_backward(self.mod_op, g.contiguous(), self.h_in[b],
                                                   m[:, :H], m[:, H:2 * H], self.g_h0,
                                                   dmod[:, :H], dmod[:, H:2 * H])
            g = self.g_h0 + self._linear_bwd(b, L_MOD, dmod)
        return g

    def train_step(self, x, target, optimizer=None):
        """Forward, MSE loss gradient, backward, one scale update over every
        record (inputs, weights, output gradients), optimizer step."""
        self.refresh_bias_copies()
        out = self.forward(x, fused=True, update=False)
        g = torch.sub(out, target).mul_(2.0 / out.numel())
        self.backward(g)
        self.state.update()
        if optimizer is not None:
            optimizer.step()
        return out


def torch_block_forward(h, ws, H, finite: bool = True):
    """The same block in plain torch (bf16 activations; weights used as
    given, or under torch.autocast): the comparator of the FP8 stack, with
    the same choice of modulation."""
    f = torch.nn.functional.linear
    m = f(h, ws[L_MOD][0], ws[L_MOD][1])
    h = m[:, :H] * h / m[:, H:2 * H]
    if finite:
        h = torch.nan_to_num(h, nan=0.0, posinf=0.0, neginf=0.0)
    h = h + f(h, ws[L_SELF][0])[:, :H]
    h = (h + f(h, ws[L_CROSS_Q][0])) + f(h, ws[L_CROSS_KV][0])[:, :H]
    return h + f(f(h, ws[L_UP][0], ws[L_UP][1]), ws[L_DOWN][0], ws[L_DOWN][1])


def _time_loop(fn, reps: int, warmup: int = 1):
    """GPU ms per call (one event pair around `reps` calls after `warmup`) and
    host wall ms per call."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for _ in range(reps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps, (time.perf_counter() - t0) * 1e3 / reps


def toy_stack_forward(dsl, workloads, blocks: int = 32, reps: int = 3, tokens: int = 0):
    """The 32-block toy stack forward (at the default 8192 tokens 4.398e13
    GEMM FLOP, one scale update over all 384 records per forward), eagerly
    and as one captured HIP graph, each with the weights re-cast and with
    cached FP8 weights (the weight casts see a device no-op flag, so one
    graph serves both); as a graph with the modulation and residual adds
    fused into the following casts; and the same stack in plain torch bf16.
    Two interleaved rounds, best of each.  With few tokens the eager forward
    is bound by the host's launch rate, the case the graph is for."""
    dev = "cuda"
    H, Mt = workloads.HIDDEN, tokens or workloads.TOKENS
    stack = ToyStack(dsl, workloads, blocks, tokens=Mt)
    x0 = workloads.uniform_bf16((Mt, H), workloads.SEED_X).to(dev)
    xin = torch.empty_like(x0)
    xin.copy_(x0)
    stack.forward(xin, fused=False)            # first launches outside capture
    stack.forward(xin, fused=True)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        stack.forward(xin, fused=False)
    graph_fused = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph_fused):
        out_fused = stack.forward(xin, fused=True)
    ws16 = [list(zip(stack.w[b], stack.b16[b])) for b in range(blocks)]

    def forward_bf16():
        h = xin
        for b in range(blocks):
            h = torch_block_forward(h, ws16[b], H)
        return h

    modes = {"eager": (lambda: stack.forward(xin, fused=False), 0),
             "eager_cached_weights": (lambda: stack.forward(xin, fused=False), 1),
             "graph": (graph.replay, 0), "graph_cached_weights": (graph.replay, 1),
             "graph_fused_producers": (graph_fused.replay, 0),
             "graph_fused_producers_cached_weights": (graph_fused.replay, 1),
             "bf16_torch_eager": (forward_bf16, 0)}
    res = {}
    for _ in range(2):
        for name, (fn, fl) in modes.items():
            stack.flag.fill_(fl)
            ms, wall = _time_loop(fn, reps)
            if name + "_ms" not in res or ms < res[name + "_ms"]:
                res[name + "_ms"], res[name + "_wall_ms"] = ms, wall
    stack.flag.fill_(0)
    graph_fused.replay()
    torch.cuda.synchronize()
    nonfinite = int((~torch.isfinite(out_fused.float())).sum())
    flop = 2 * Mt * sum(fin * fout for fin, fout, _ in stack.lin) * blocks
    out = {k: round(v, 3) for k, v in res.items()}
    out.update({"blocks": blocks, "tokens": Mt, "gemm_flop": flop,
                "library_launches_per_forward": blocks * (13 if stack.group_w else 18) + 1,
                "grouped_weight_casts": stack.group_w,
                "graph_fused_producers_gemm_tflops":
                    round(flop / (res["graph_fused_producers_ms"] * 1e-3) / 1e12, 1),
                "nonfinite_outputs": nonfinite})
    del graph, graph_fused, stack
    torch.cuda.empty_cache()
    return out


def _stack_params(stack):
    """The training stack's fp32 master weights and biases as optimizer
    parameters, each with the library-written gradient buffer as its .grad."""
    params = []
    for b in range(stack.blocks):
        for l in range(len(stack.lin)):
            w = stack.w[b][l]
            w.requires_grad_(True)
            w.grad = stack.grad_w[b][l]
            params.append(w)
            if stack.b32[b][l] is not None:
                bb = stack.b32[b][l]
                bb.requires_grad_(True)
                bb.grad = stack.grad_b[b][l]
                params.append(bb)
    return params


def _adamw(params, capturable: bool = False):
    """torch's fused AdamW where the installed torch has it, else the foreach one;
    `capturable` keeps its step counts on the device so that a HIP graph can
    replay its step."""
    try:
        probe = torch.zeros(4, device="cuda", requires_grad=True)
        probe.grad = torch.ones(4, device="cuda")
        torch.optim.AdamW([probe], lr=1e-3, fused=True, capturable=capturable).step()
        return torch.optim.AdamW(params, lr=1e-3, fused=True, capturable=capturable)
    except (RuntimeError, ValueError):
        return torch.optim.AdamW(params, lr=1e-3, foreach=True, capturable=capturable)


def capture_train_step(stack, x, target, opt, warmup: int = 2):
    """The whole training step of `stack` (forward, loss gradient, backward,
    scale update, optimizer step) captured in one HIP graph.  `opt` must be
    capturable; `warmup` eager steps on a side stream first create its state
    (and run every launch once outside capture).  Returns the graph; each
    replay is one more training step on the same x and target."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(warmup):
            stack.train_step(x, target, opt)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        stack.train_step(x, target, opt)
    return graph


def toy_stack_train_step(dsl, workloads, blocks: int = 32, warmup: int = 10, iters: int = 50):
    """One training step of the 32-block toy stack, timed as the page times
    its model (10 warm-up iterations, then `iters` between one event pair):
    forward, MSE loss, backward, AdamW on fp32 master weights.

    FP8: the library stack (fused producers; per linear an E5M2 gradient cast
    with fused bias gradient, dgrad from the cached weight transpose, fp32
    wgrad written as the parameter's gradient; one scale update over 576
    records).  BF16: the same parameters through torch autograd under
    torch.autocast(bfloat16), the page's BF16 run.  The modulation's backward
    of the FP8 run is the library's fp8_produce_modulate_backward; its
    residual sums are torch ops."""
    dev = "cuda"
    H, Mt = workloads.HIDDEN, workloads.TOKENS
    stack = ToyStack(dsl, workloads, blocks, train=True)
    params = _stack_params(stack)
    opt = _adamw(params)
    x = workloads.uniform_bf16((Mt, H), workloads.SEED_X).to(dev)
    target = workloads.uniform_bf16((Mt, H), workloads.SEED_X + 1).to(dev)
    res = {}
    with torch.no_grad():
        fp8_ms, fp8_wall = _time_loop(lambda: stack.train_step(x, target, opt), iters, warmup)
        opt_ms, _ = _time_loop(opt.step, 10, 2)
    res["fp8_step_ms"], res["fp8_step_wall_ms"] = round(fp8_ms, 2), round(fp8_wall, 2)
    res["adamw_alone_ms"] = round(opt_ms, 2)
    # The same step as one HIP graph (capturable AdamW), as the page's
    # --cuda_graph run does.
    opt_g = _adamw(params, capturable=True)
    with torch.no_grad():
        graph = capture_train_step(stack, x, target, opt_g)
        g_ms, g_wall = _time_loop(graph.replay, iters, warmup)
    res["fp8_step_graph_ms"], res["fp8_step_graph_wall_ms"] = round(g_ms, 2), round(g_wall, 2)
    del graph, opt_g

    ws32 = [list(zip(stack.w[b], stack.b32[b])) for b in range(blocks)]
    crit = torch.nn.MSELoss()

    def bf16_step():
        opt.zero_grad(set_to_none=True)
        with torch.autocast(device_type="cuda", dtype=torch.bfloat16):
            h = x
            for b in range(blocks):
                h = torch_block_forward(h, ws32[b], H)
            loss = crit(h.float(), target.float())
        loss.backward()
        opt.step()

    bf_ms, bf_wall = _time_loop(bf16_step, iters, warmup)
    res["bf16_autocast_step_ms"], res["bf16_autocast_step_wall_ms"] = round(bf_ms, 2), round(bf_wall, 2)
    flop = 3 * 2 * Mt * sum(fin * fout for fin, fout, _ in stack.lin) * blocks
    res.update({"blocks": blocks, "gemm_flop_per_step": flop, "records": stack.state.T,
                "fp8_over_bf16_speedup": round(bf_ms / fp8_ms, 3),
                "protocol": f"{warmup} warm-up + {iters} timed iterations, one event pair"})
    del stack, opt, params
    torch.cuda.empty_cache()
    return res


def cpu_baseline(workloads, scales):
    """The oracle (plain C; OpenMP over independent outputs, on every thread
    it is given) running one whole step of the benchmark on the same inputs:
    the X, W and dY casts (codes, transpose, amax), the forward (with bias),
    dgrad and wgrad (fp32) products of the oracle's own codes, and the scale
    update.  No sampling and no extrapolation; `scales` are the GPU state's
    scales for x, w and dY."""
    import numpy as np
    import oracle
    oracle.build(force=False)

    def b16(t):
        return t.contiguous().view(torch.int16).numpy().view(np.uint16)

    x, w, b = workloads.mlp_forward(0)
    dy = workloads.mlp_grad()
    xb, wb, bb, dyb = b16(x), b16(w), b16(b), b16(dy)
    sx, sw, sdy = (float(v) for v in scales)
    t = {}

    def timed(name, fn):
        t0 = time.perf_counter()
        r = fn()
        t[name] = time.perf_counter() - t0
        return r

    qx, qxt, ax, six = timed("cast_x", lambda: oracle.cast_transpose_amax(xb, sx, oracle.E4M3))
    qw, qwt, aw, siw = timed("cast_w", lambda: oracle.cast_transpose_amax(wb, sw, oracle.E4M3))
    timed("gemm_fwd", lambda: oracle.gemm_nt(qx, 0, qw, 0, six, siw, bias=bb))
    qd, qdt, ad, sid = timed("cast_dy", lambda: oracle.cast_transpose_amax(dyb, sdy, oracle.E5M2))
    timed("gemm_dgrad", lambda: oracle.gemm_nt(qd, 1, qwt, 0, sid, siw))
    timed("gemm_wgrad", lambda: oracle.gemm_nt(qdt, 1, qxt, 0, sid, six,
                                               out_kind=oracle.OUT_FP32))
    hist = np.zeros((3, 16), np.float32)
    cur = np.array([ax, aw, ad], np.float32)
    sc = np.array([sx, sw, sdy], np.float32)
    timed("scale_update", lambda: oracle.scale_update(hist, cur, sc, np.zeros(3, np.float32),
                                                      np.array([0, 0, 1], np.uint8)))
    total = sum(t.values())
    return {"value": round(3 * GEMM_FLOP / total / 1e12, 6), "unit": "TFLOP/s",
            "cores": oracle.num_threads(), "kind": "oracle",
            "sample": (f"one whole step, no sampling: casts of X, W [8192,2048] and dY "
                       f"[8192,8192], fwd/dgrad/wgrad 8192x8192x2048 products, scale update; "
                       f"{total:.1f} s on {oracle.num_threads()} threads"),
            "seconds": {k: round(v, 3) for k, v in t.items()}}


def probe_kernels(dsl, workloads, st):
    """One launch each of the kernels whose HBM traffic and counters are
    reported, after a warm-up, with a synchronisation after each (so counter
    collection sees one dispatch per kernel), in this order: forward, dgrad
    and wgrad GEMMs at the step's shapes; the [4096, 4096] cast with both
    source policies; the dY [8192, 8192] E5M2 cast; a 64 MiB reference copy
    (32 MiB read + 32 MiB written, known traffic, calibrates the counters);
    the scale update over 384 and over 576 records."""
    src = workloads.cast_only().to("cuda")
    out = dsl.Float8Tensor.empty(CAST_R, CAST_C, 0, device="cuda")
    scale = torch.tensor([448.0 / 3920.0], device="cuda")
    amax = torch.zeros(1, device="cuda")
    a = torch.ones(32 << 20, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    g = st["state"]
    upd = {T: dsl.DelayedScalingState([0, 0, 1] * (T // 3), device="cuda") for T in (384, 576)}
    seq = [
        ("gemm_fwd", lambda: dsl.fp8_linear_fwd(st["qx"], st["qw"], st["b"], st["y"])),
        ("gemm_dgrad", lambda: dsl.fp8_linear_dgrad(st["qdy"], st["qw"], st["dx"])),
        ("gemm_wgrad", lambda: dsl.fp8_linear_wgrad(st["qdy"], st["qx"], st["dw"])),
        ("cast", lambda: dsl.fp8_cast_transpose_amax(src, scale, out, amax)),
        ("cast_cached", lambda: dsl.fp8_cast_transpose_amax_cached(src, scale, out, amax)),
        ("cast_dy", lambda: dsl.fp8_cast_transpose_amax(st["dy"], g.scale[2:3], st["qdy"],
                                                        g.amax_cur[2:3])),
        ("copy_64mib", lambda: dsl.fp8_reference_copy(a, b, 2048, False)),
        ("scale_update_384", lambda: upd[384].update()),
        ("scale_update_576", lambda: upd[576].update()),
    ]
    for _ in range(2):
        for _, fn in seq:
            fn()
    torch.cuda.synchronize()
    for _, fn in seq:
        fn()
        torch.cuda.synchronize()
    print("probe-kernels: " + ", ".join(n for n, _ in seq), flush=True)


def probe_toy_stack(dsl, workloads):
    """The toy stack's two measured workloads, synchronised between phases,
    for a kernel trace: 6 replays of the 32-block forward at 1024 tokens as
    one HIP graph with the producers fused and the FP8 weights cached (the
    no-op flag set), then 4 training steps of the 32-block stack at 8192
    tokens (fused AdamW on fp32 master weights)."""
    stack = ToyStack(dsl, workloads, 32, tokens=1024)
    xin = workloads.uniform_bf16((1024, workloads.HIDDEN), workloads.SEED_X).to("cuda")
    stack.forward(xin, fused=True)               # first launches outside capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        stack.forward(xin, fused=True)
    stack.flag.fill_(1)
    torch.cuda.synchronize()
    for _ in range(6):
        graph.replay()
    torch.cuda.synchronize()
    progress("probe-toy-stack: 1024-token forward graph done")
    del graph, stack
    torch.cuda.empty_cache()
    stack = ToyStack(dsl, workloads, 32, train=True)
    opt = _adamw(_stack_params(stack))
    x = workloads.uniform_bf16((workloads.TOKENS, workloads.HIDDEN), workloads.SEED_X).to("cuda")
    target = workloads.uniform_bf16((workloads.TOKENS, workloads.HIDDEN),
                                    workloads.SEED_X + 1).to("cuda")
    with torch.no_grad():
        for _ in range(4):
            stack.train_step(x, target, opt)
            torch.cuda.synchronize()
    progress("probe-toy-stack: 4 training steps done")


def scale_update_cost(dsl, iters: int = 50):
    """One fused update over 3 records (the step), the 384 of the 32-block
    forward and the 576 of its training step (history 16): us per launch,
    from `iters` launches captured in one HIP graph and replayed (the
    kernel's own time; the update issues no memset), and from an eager loop
    of the same launches (bound by the binding's host overhead per call)."""
    res = {}
    for T in (3, 384, 576):
        st = dsl.DelayedScalingState([0, 0, 1] * (T // 3), device="cuda")
        st.amax_cur.fill_(1.5)
        for _ in range(5):
            st.update()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(iters):
                st.update()
        g.replay()
        torch.cuda.synchronize()
        for name, run in (("graph", g.replay), ("eager", lambda: [st.update() for _ in range(iters)])):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            run()
            e1.record()
            torch.cuda.synchronize()
            res[f"T{T}_{name}_us"] = round(e0.elapsed_time(e1) / iters * 1e3, 2)
        del g
    return res


def traffic_record(root: str):
    """HBM bytes per launch measured with rocprofv3 counters for the current
    kernel sources, or None when the sources changed since the measurement."""
    import hashlib
    path = os.path.join(root, "profiles", "hbm_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    def sha(name):
        p = os.path.join(root, "delayed_scaling_linear_amd", "csrc", name)
        if not os.path.exists(p):
            return None
        with open(p, "rb") as f:
            return hashlib.sha256(f.read()).hexdigest()[:16]

    # A kernel's bytes count only while every source file it was built from
    # is unchanged.
    def unchanged(n):
        now = sha(n)
        return now is not None and rec["source_sha256"].get(n) == now

    return {k: v for k, v in rec["kernels"].items()
            if v.get("sources") and all(unchanged(n) for n in v["sources"])}


def progress(msg: str) -> None:
    """A line on stderr as each part of the benchmark finishes."""
    print(f"bench: {msg}", file=sys.stderr, flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); multi-GPU runs "
              "are not part of this library's measured path", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs an MI355X GPU", file=sys.stderr)
        sys.exit(2)
    root = os.path.dirname(os.path.abspath(__file__))
    sys.path.insert(0, root)
    import delayed_scaling_linear_amd as dsl
    import workloads

    if args.probe_toy_stack:
        probe_toy_stack(dsl, workloads)
        return
    dev = "cuda"
    x, w, b = workloads.mlp_forward(0)
    dy = workloads.mlp_grad()
    st = {
        "x": x.to(dev), "w": w.to(dev), "b": b.to(dev), "dy": dy.to(dev),
        "qx": dsl.Float8Tensor.empty(M, K, 0, device=dev),
        "qw": dsl.Float8Tensor.empty(N, K, 0, device=dev),
        "qdy": dsl.Float8Tensor.empty(M, N, 1, device=dev),
        "y": torch.empty(M, N, dtype=torch.bfloat16, device=dev),
        "dx": torch.empty(M, K, dtype=torch.bfloat16, device=dev),
        "dw": torch.empty(N, K, dtype=torch.float32, device=dev),
        "state": dsl.DelayedScalingState([0, 0, 1], device=dev),
    }
    for _ in range(args.warmup):
        gpu_step(dsl, st, None)
    torch.cuda.synchronize()
    if args.probe_kernels:
        probe_kernels(dsl, workloads, st)
        return

    # Whole-step timing (no per-kernel events inside).
    t0 = time.perf_counter()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        gpu_step(dsl, st, None)
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = e0.elapsed_time(e1) / args.steps

    # Same steps again with an event pair around every launch.
    timer = Timer()
    for _ in range(args.steps):
        gpu_step(dsl, st, timer)
    torch.cuda.synchronize()
    kernels = {}
    for name in ("cast_x", "cast_w", "gemm_fwd", "cast_dy", "gemm_dgrad", "gemm_wgrad",
                 "scale_update"):
        ms, p10, p90, mean = timer.stats_ms(name)
        k = {"us": round(ms * 1e3, 2), "us_p10": round(p10 * 1e3, 2),
             "us_p90": round(p90 * 1e3, 2), "us_mean": round(mean * 1e3, 2)}
        if name.startswith("gemm"):
            k["TFLOP/s"] = round(GEMM_FLOP / (ms * 1e-3) / 1e12, 1)
        elif name == "cast_dy":
            k["GB/s"] = round(4 * M * N / (ms * 1e-3) / 1e9, 1)
        elif name.startswith("cast"):
            k["GB/s"] = round(4 * M * K / (ms * 1e-3) / 1e9, 1)
        kernels[name] = k

    progress(f"step timing done ({ms_step * 1e3:.1f} us per step)")
    fwd_ms = gemm_fwd_back_to_back(dsl, st, max(args.steps, 10))
    fwd_tflops = GEMM_FLOP / (fwd_ms * 1e-3) / 1e12
    casts = cast_bandwidth(dsl, workloads, args.cast_iters)
    copy_gbs, copy_cfg = copy_ceiling(dsl)
    cast_ms, cast_gbs = casts["nontemporal"]  # the default entry point, as the step calls it

    progress("roofline loops done")
    update_cost = scale_update_cost(dsl)
    dbias_cost = dbias_cast_cost(dsl, st)
    split_cost = split_product_cost(dsl, workloads)
    producer_cost = producer_cast_cost(dsl, workloads)
    dyn_cost = dynamic_vs_delayed(dsl, st)
    fp8out_cost = fp8_output_forward(dsl, st)
    progress("variant comparisons done")
    toy = None if args.no_toy_stack else toy_stack_forward(dsl, workloads)
    toy_small = None if args.no_toy_stack else toy_stack_forward(dsl, workloads, reps=10,
                                                                 tokens=1024)
    progress("toy-stack forward done")
    train = None if args.no_train_step else toy_stack_train_step(dsl, workloads)
    progress("toy-stack training step done")
    traffic = traffic_record(root)
    result = {
        "metric": "FP8 GEMM TFLOP/s (M8192 K2048 N8192) + cast-transpose-amax HBM GB/s",
        "value": round(3 * GEMM_FLOP / (ms_step * 1e-3) / 1e12, 1),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8",
        "data": "synthetic (seeded: X ~U(0,1), W ~N(0,0.02), dY ~N(0,1e-3), bf16)",
        "config": {"workload": "FP8 linear fwd+bwd, HYBRID, X/W [8192,2048], dY [8192,8192], "
                               "history 16 (toy-block MLP shape: hidden 2048, batch 8, seq 1024)",
                   "M": M, "N": N, "K": K, "global_batch": 8, "seq_len": 1024,
                   "parallelism": "none (1 GPU)"},
        "gemm_fwd_tflops": round(fwd_tflops, 1),
        "gemm_fwd_us": round(fwd_ms * 1e3, 2),
        "hbm_copy_ceiling_gbs": round(copy_gbs, 1),
        "cast_transpose_amax_gbs": round(cast_gbs, 1),
        "cast_transpose_amax_us": round(cast_ms * 1e3, 2),
        "cast_transpose_amax_policies": {
            k: {"us": round(v[0] * 1e3, 2), "GB/s": round(v[1], 1),
                "frac_of_hbm_peak": round(v[1] / HBM_PEAK_GBS, 4),
                "frac_of_measured_copy": round(v[1] / copy_gbs, 4)} for k, v in casts.items()},
        "kernels": kernels,
        "roofline": {"bound": "mfma", "kernel": "gemm_fwd (fp8_linear_fwd)",
                     "achieved": round(fwd_tflops, 1), "peak": FP8_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(fwd_tflops / FP8_PEAK_TFLOPS, 4),
                     "traffic": (traffic or {}).get("gemm_fwd", {}).get("bytes")},
        "roofline_cast": {"bound": "hbm",
                          "kernel": "fp8_cast_transpose_amax bf16 [4096,4096] -> E4M3 "
                                    "codes + transpose + amax (cold buffers)",
                          "achieved": round(cast_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                          "frac": round(cast_gbs / HBM_PEAK_GBS, 4),
                          "traffic": (traffic or {}).get("cast", {}).get("bytes"),
                          "measured_copy_ceiling_gbs": round(copy_gbs, 1),
                          "measured_copy_ceiling": copy_cfg,
                          "frac_of_measured_copy": round(cast_gbs / copy_gbs, 4)},
        "wall_s_timed": round(wall, 3),
    }
    result["scale_update_one_launch"] = update_cost
    result["dy_cast_dbias"] = dbias_cost
    result["split_products"] = split_cost
    result["producer_fused_cast"] = producer_cost
    result["delayed_vs_dynamic_cast"] = dyn_cost
    result["fp8_output_forward"] = fp8out_cost
    if toy is not None:
        result["toy_stack_forward"] = toy
        result["toy_stack_forward_1024_tokens"] = toy_small
    if train is not None:
        result["toy_stack_train_step"] = train
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(workloads, st["state"].scale.cpu().tolist())
        progress("cpu baseline done")
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
