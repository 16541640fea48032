"""Sliding-window attention ([ZtF] "Dropout, block-sparsity, and other real-kernel
details") through the C ABI against the float64 oracle's window path, on seeded inputs:
narrow and wide windows, one-sided and two-sided, ragged shapes, rows that see no key,
the special windows that are causal and full attention, and the full-size workload on
sampled rows."""
import math

import numpy as np
import pytest

import io_aware_exact_02_amd as fa
from io_aware_exact_02_amd import inputs as I
from oracle import naive
from tests.gpu_util import TOL_GRAD, TOL_LSE, TOL_O, draw, maxabs, to_f64, torch

pytestmark = pytest.mark.gpu

WINDOWS = [(0, 0), (5, 3), (63, 0), (64, 0), (127, 0), (128, 64), (300, -1), (-1, 200), (1000, 1000)]
SHAPES = [(1, 1), (100, 100), (300, 300), (257, 513), (513, 257), (1000, 1000)]


def _grad_tol(ref):
    """The 5e-2 bound holds for gradients of unit scale; narrow windows leave rows a few
    keys, so P, dS and the gradients grow, and with them the bf16 rounding of dS."""
    return TOL_GRAD["bf16"] * max(1.0, float(np.abs(ref).max()) if np.size(ref) else 1.0)


def _check_lse(got, ref):
    got = to_f64(got)
    inf_r, inf_g = np.isneginf(ref), np.isneginf(got)
    assert np.array_equal(inf_r, inf_g), int(np.sum(inf_r != inf_g))
    assert maxabs(got[~inf_r], ref[~inf_r]) <= TOL_LSE


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("Tq,Tk", SHAPES)
@pytest.mark.parametrize("win", WINDOWS)
def test_window_forward_parity(d, Tq, Tk, win):
    B, H = 1, 2
    dev, f = draw(B, H, Tq, Tk, d, "bf16", seed=5000 + Tq + 7 * Tk + d)
    O, lse = fa.forward_window(dev["q"], dev["k"], dev["v"], win)
    torch().cuda.synchronize()
    Or, Lr = naive.forward(f["q"], f["k"], f["v"], 1 / math.sqrt(d), False, window=win)
    assert maxabs(to_f64(O), Or) <= TOL_O["bf16"]
    _check_lse(lse, Lr)


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("Tq,Tk", SHAPES[1:])
@pytest.mark.parametrize("win", WINDOWS)
def test_window_backward_parity(d, Tq, Tk, win):
    t = torch()
    B, H = 1, 2
    dev, f = draw(B, H, Tq, Tk, d, "bf16", seed=6000 + Tq + 7 * Tk + d, with_do=True)
    O, lse = fa.forward_window(dev["q"], dev["k"], dev["v"], win)
    dQ, dK, dV = fa.backward_window(dev["q"], dev["k"], dev["v"], O, dev["do"], lse, win, grad_dtype=t.float32)
    t.cuda.synchronize()
    rQ, rK, rV, _, _ = naive.backward(f["q"], f["k"], f["v"], f["do"], 1 / math.sqrt(d), False, window=win)
    for got, ref, name in ((dQ, rQ, "dQ"), (dK, rK, "dK"), (dV, rV, "dV")):
        g = to_f64(got)
        assert np.isfinite(g).all(), name
        assert maxabs(g, ref) <= _grad_tol(ref), name


def test_special_windows_run_the_causal_and_dense_kernels():
    t = torch()
    B, H, T, d = 2, 2, 700, 128
    dev, _ = draw(B, H, T, T, d, "bf16", seed=6500, with_do=True)
    for win, causal in (((-1, 0), True), ((-1, -1), False)):
        O0, L0 = fa.forward(dev["q"], dev["k"], dev["v"], causal=causal)
        O1, L1 = fa.forward_window(dev["q"], dev["k"], dev["v"], win)
        g0 = fa.backward(dev["q"], dev["k"], dev["v"], O0, dev["do"], L0, causal=causal)
        g1 = fa.backward_window(dev["q"], dev["k"], dev["v"], O1, dev["do"], L1, win)
        t.cuda.synchronize()
        assert t.equal(O0, O1) and t.equal(L0, L1)
        for a, b in zip(g0, g1):
            assert t.equal(a, b)


@pytest.mark.parametrize("d", [64, 128, 256])
def test_rows_outside_every_window(d):
    """Tq > Tk + wl: rows past Tk + wl see no key (O = 0, lse = -inf, dQ = 0)."""
    t = torch()
    B, H, Tq, Tk = 1, 2, 900, 300
    win = (50, 10)
    dev, f = draw(B, H, Tq, Tk, d, "bf16", seed=6600, with_do=True)
    O, lse = fa.forward_window(dev["q"], dev["k"], dev["v"], win)
    dQ, dK, dV = fa.backward_window(dev["q"], dev["k"], dev["v"], O, dev["do"], lse, win)
    t.cuda.synchronize()
    last = Tk - 1 + win[0]
    assert t.all(O[:, :, last + 1:] == 0) and t.all(t.isneginf(lse[:, :, last + 1:]))
    assert t.all(dQ[:, :, last + 1:] == 0)
    Or, Lr = naive.forward(f["q"], f["k"], f["v"], 1 / math.sqrt(d), False, window=win)
    assert maxabs(to_f64(O), Or) <= TOL_O["bf16"]
    _check_lse(lse, Lr)
    for x in (O, dQ, dK, dV):
        assert t.isfinite(x.float()).all()


def test_window_results_repeat_bit_for_bit():
    t = torch()
    B, H, T, d = 2, 3, 1500, 128
    dev, _ = draw(B, H, T, T, d, "bf16", seed=6700, with_do=True)
    runs = []
    for _ in range(2):
        O, lse = fa.forward_window(dev["q"], dev["k"], dev["v"], (200, 0))
        g = fa.backward_window(dev["q"], dev["k"], dev["v"], O, dev["do"], lse, (200, 0))
        runs.append((O, lse) + tuple(g))
    t.cuda.synchronize()
    for a, b in zip(*runs):
        assert t.equal(a, b)


def test_swa_workload_sampled_rows():
    """The sliding-window workload at full size (32 heads x 32768, d = 128, window (4095, 0)):
    O, lse and dQ on sampled rows of sampled heads against the oracle (each is exact per
    row), and dV through sum_l dV_l = sum_r dO_r (every row keeps at least its own key),
    bounded by the bf16 rounding of P: 2^-9 sum_r |dO_r|."""
    t = torch()
    w = I.WORKLOADS["swa_bf16_b1h32_t32768_d128_w4096"]
    dev, f = draw(w.B, w.H, w.Tq, w.Tk, w.d, w.dtype, w.seed, w.qk_spread, True)
    O, lse = fa.forward_window(dev["q"], dev["k"], dev["v"], w.window)
    dQ, dK, dV = fa.backward_window(dev["q"], dev["k"], dev["v"], O, dev["do"], lse, w.window,
                                    grad_dtype=t.float32)
    t.cuda.synchronize()
    rng = np.random.default_rng(8)
    rows = np.unique(np.concatenate([[0, 1, 4095, 4096, 4097, 16384, w.Tq - 1], rng.integers(0, w.Tq, 25)]))
    scale = 1 / math.sqrt(w.d)
    for h in (0, 13, 31):
        args = (f["q"][0, h], f["k"][0, h], f["v"][0, h])
        Or, Lr = naive.forward_head(*args, scale, False, rows=rows, window=w.window)
        assert maxabs(to_f64(O[0, h][rows]), Or) <= TOL_O["bf16"], h
        assert maxabs(to_f64(lse[0, h][rows]), Lr) <= TOL_LSE, h
        ref = naive.dq_rows(*args, f["do"][0, h], scale, False, rows, window=w.window)
        assert maxabs(to_f64(dQ[0, h][rows]), ref) <= TOL_GRAD["bf16"], h
    dv_sum = dV.sum(dim=2, dtype=t.float64).cpu().numpy()
    bound = (2.0 ** -9 + 1e-5) * np.abs(f["do"]).sum(axis=2) + 1e-3
    assert np.all(np.abs(dv_sum - f["do"].sum(axis=2)) <= bound)
