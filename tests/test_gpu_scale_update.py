"""GPU parity: fp8_scale_update against the oracle, bit-exact, through the C ABI."""
import numpy as np
import pytest
import torch

import delayed_scaling_linear_amd as dsl
import oracle
from tests.gpu_util import DEV

pytestmark = pytest.mark.gpu


def _run_both(hist, cur, scale, fmt, margin=0, steps=1, amax_seq=None):
    """Run `steps` updates on the GPU and in the oracle from the same state;
    amax_seq[s] (if given) is written into amax_cur before step s."""
    h_o, c_o, s_o = hist.copy(), cur.copy(), scale.copy()
    si_o = np.zeros_like(scale)
    g_h, g_c = torch.from_numpy(hist).to(DEV), torch.from_numpy(cur).to(DEV)
    g_s, g_si = torch.from_numpy(scale).to(DEV), torch.zeros(len(scale), dtype=torch.float32, device=DEV)
    g_f = torch.from_numpy(fmt).to(DEV)
    for st in range(steps):
        if amax_seq is not None:
            c_o[:] = amax_seq[st]
            g_c.copy_(torch.from_numpy(amax_seq[st]))
        oracle.scale_update(h_o, c_o, s_o, si_o, fmt, margin=margin)
        dsl.fp8_scale_update(g_h, g_c, g_s, g_si, g_f, margin=margin)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(g_h.cpu().numpy().view(np.uint32), h_o.view(np.uint32))
        np.testing.assert_array_equal(g_c.cpu().numpy().view(np.uint32), c_o.view(np.uint32))
        np.testing.assert_array_equal(g_s.cpu().numpy().view(np.uint32), s_o.view(np.uint32))
        np.testing.assert_array_equal(g_si.cpu().numpy().view(np.uint32), si_o.view(np.uint32))


@pytest.mark.parametrize("H", [16, 1, 7, 33])
@pytest.mark.parametrize("margin", [0, 2, -3])
def test_random_histories(H, margin):
    rng = np.random.default_rng(H * 100 + margin + 50)
    T = 384          # 192 linears x {x, w} of the 32-block toy stack
    steps = 20
    hist = np.zeros((T, H), np.float32)
    cur = np.zeros(T, np.float32)
    scale = np.ones(T, np.float32)
    fmt = rng.integers(0, 2, T).astype(np.uint8)
    seq = [(10.0 ** rng.uniform(-6, 5, T)).astype(np.float32) for _ in range(steps)]
    _run_both(hist, cur, scale, fmt, margin, steps, seq)


def test_special_amax_values():
    T, H = 300, 16
    rng = np.random.default_rng(9)
    hist = (rng.uniform(0, 10, (T, H))).astype(np.float32)
    hist[:50] = 0.0
    scale = rng.uniform(0.5, 100, T).astype(np.float32)
    fmt = rng.integers(0, 2, T).astype(np.uint8)
    specials = np.array([0.0, np.inf, np.nan, 1e-44, 3e38, 1e-30, 448.0, 57344.0, -5.0, -0.0],
                        np.float32)
    cur = specials[rng.integers(0, specials.size, T)]
    _run_both(hist, cur, scale, fmt, margin=0, steps=1)
    _run_both(hist, cur, scale, fmt, margin=5, steps=1)


def test_window_eviction_on_gpu():
    T, H = 2, 16
    seq = [np.array([100.0, 3.0], np.float32)] + [np.array([1.0, 3.0], np.float32)] * 17
    _run_both(np.zeros((T, H), np.float32), np.zeros(T, np.float32), np.ones(T, np.float32),
              np.array([0, 1], np.uint8), 0, len(seq), seq)


def test_unaligned_history_takes_generic_path():
    T, H = 64, 16
    base = torch.zeros(T * H + 1, dtype=torch.float32, device=DEV)
    g_h = base[1:].view(T, H)          # 4-byte offset: not 16-byte aligned
    rng = np.random.default_rng(3)
    amax = rng.uniform(0.1, 10, T).astype(np.float32)
    g_c = torch.from_numpy(amax).to(DEV)
    g_s = torch.ones(T, device=DEV)
    g_si = torch.zeros(T, device=DEV)
    g_f = torch.zeros(T, dtype=torch.uint8, device=DEV)
    dsl.fp8_scale_update(g_h, g_c, g_s, g_si, g_f)
    h_o = np.zeros((T, H), np.float32)
    c_o, s_o, si_o = amax.copy(), np.ones(T, np.float32), np.zeros(T, np.float32)
    oracle.scale_update(h_o, c_o, s_o, si_o, np.zeros(T, np.uint8))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(g_s.cpu().numpy(), s_o)
    np.testing.assert_array_equal(g_h.cpu().numpy(), h_o)
    np.testing.assert_array_equal(g_si.cpu().numpy(), si_o)
