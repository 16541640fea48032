"""Pins of the oracle's sliding-window path ([ZtF] "Dropout, block-sparsity, and other
real-kernel details": windows are masks that are functions of (r, l)).  Each pin checks
against something other than the window code: the causal and dense definitions, a closed
form, an explicit loop over (r, l) with math.exp, and central finite differences."""
import math

import numpy as np
import pytest

from oracle import naive


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def test_special_windows_are_causal_and_dense():
    rng = np.random.default_rng(11)
    q, k, v = _rand(rng, 70, 6), _rand(rng, 53, 6), _rand(rng, 53, 6)
    for win, causal in (((-1, 0), True), ((-1, -1), False)):
        O0, L0 = naive.forward_head(q, k, v, 0.4, causal)
        O1, L1 = naive.forward_head(q, k, v, 0.4, False, window=win)
        assert np.array_equal(O0, O1) and np.array_equal(L0, L1)


def test_zero_width_window_is_the_diagonal():
    """Window (0, 0): row r sees only key r, so O_r = v_r and lse_r = c q_r . k_r;
    rows past the last key see nothing (O = 0, lse = -inf)."""
    rng = np.random.default_rng(12)
    Tq, Tk, d, c = 30, 24, 5, 0.7
    q, k, v = _rand(rng, Tq, d), _rand(rng, Tk, d), _rand(rng, Tk, d)
    O, L = naive.forward_head(q, k, v, c, False, window=(0, 0))
    assert np.allclose(O[:Tk], v, atol=1e-15)
    assert np.allclose(L[:Tk], c * np.sum(q[:Tk] * k, axis=1), atol=1e-14)
    assert np.all(O[Tk:] == 0) and np.all(L[Tk:] == -np.inf)


@pytest.mark.parametrize("win", [(3, 2), (0, 5), (7, 0), (-1, 3), (4, -1)])
def test_window_against_an_explicit_loop(win):
    rng = np.random.default_rng(13)
    Tq, Tk, d, c = 17, 15, 4, 0.5
    q, k, v = _rand(rng, Tq, d), _rand(rng, Tk, d), _rand(rng, Tk, d)
    O, L = naive.forward_head(q, k, v, c, False, window=win)
    wl, wr = win
    for r in range(Tq):
        keys = [l for l in range(Tk) if (wl < 0 or l >= r - wl) and (wr < 0 or l <= r + wr)]
        if not keys:
            assert np.all(O[r] == 0) and L[r] == -np.inf
            continue
        s = [c * sum(q[r, j] * k[l, j] for j in range(d)) for l in keys]
        m = max(s)
        e = [math.exp(x - m) for x in s]
        tot = sum(e)
        o = [sum(e[i] * v[l, j] for i, l in enumerate(keys)) / tot for j in range(d)]
        assert np.allclose(O[r], o, atol=1e-13)
        assert abs(L[r] - (m + math.log(tot))) < 1e-13


@pytest.mark.parametrize("win", [(3, 2), (5, 0)])
def test_window_gradients_by_finite_differences(win):
    rng = np.random.default_rng(14)
    Tq, Tk, d, c = 12, 11, 3, 0.8
    q, k, v, do = _rand(rng, Tq, d), _rand(rng, Tk, d), _rand(rng, Tk, d), _rand(rng, Tq, d)
    dQ, dK, dV = naive.backward_head(q, k, v, do, c, False, window=win)[:3]

    def loss(q_, k_, v_):
        return float(np.sum(naive.forward_head(q_, k_, v_, c, False, window=win)[0] * do))

    h = 1e-6
    for name, arr, grad in (("q", q, dQ), ("k", k, dK), ("v", v, dV)):
        for idx in [(0, 0), (5, 2), (arr.shape[0] - 1, 1)]:
            p, m = arr.copy(), arr.copy()
            p[idx] += h
            m[idx] -= h
            ap = {"q": q, "k": k, "v": v}
            am = dict(ap)
            ap[name], am[name] = p, m
            fd = (loss(ap["q"], ap["k"], ap["v"]) - loss(am["q"], am["k"], am["v"])) / (2 * h)
            assert abs(fd - grad[idx]) <= 1e-6 * (1 + abs(fd)), (name, idx, fd, grad[idx])
    assert np.allclose(naive.dq_rows(q, k, v, do, c, False, np.array([0, 4, 11]), window=win),
                       dQ[[0, 4, 11]], atol=1e-13)
