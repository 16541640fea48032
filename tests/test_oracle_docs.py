"""Pins of the oracle's document masks ([ZtF] "Dropout, block-sparsity, and other
real-kernel details"): a packed sequence of documents is, document by document,
the unmasked (or causal) problem on that document alone; checked against the
oracle's own dense path on the slices, an explicit loop, and finite differences."""
import math

import numpy as np
import pytest

from oracle import naive


def _rand(rng, *shape):
    return rng.standard_normal(shape)


@pytest.mark.parametrize("causal", [False, True])
def test_documents_are_independent_problems(causal):
    rng = np.random.default_rng(21)
    cu = [0, 1, 40, 41, 130, 300]
    T, d = cu[-1], 6
    q, k, v, do = (_rand(rng, T, d) for _ in range(4))
    O, L = naive.forward_head(q, k, v, 0.45, causal, docs=cu)
    dQ, dK, dV = naive.backward_head(q, k, v, do, 0.45, causal, docs=cu)[:3]
    for a, b in zip(cu[:-1], cu[1:]):
        s = slice(a, b)
        Or, Lr = naive.forward_head(q[s], k[s], v[s], 0.45, causal)
        assert np.allclose(O[s], Or, atol=1e-13) and np.allclose(L[s], Lr, atol=1e-13)
        rQ, rK, rV = naive.backward_head(q[s], k[s], v[s], do[s], 0.45, causal)[:3]
        assert np.allclose(dQ[s], rQ, atol=1e-12) and np.allclose(dK[s], rK, atol=1e-12)
        assert np.allclose(dV[s], rV, atol=1e-12)


def test_documents_against_an_explicit_loop():
    rng = np.random.default_rng(22)
    cu = [0, 5, 6, 13, 20]
    T, d, c = cu[-1], 3, 0.6
    q, k, v = _rand(rng, T, d), _rand(rng, T, d), _rand(rng, T, d)
    O, L = naive.forward_head(q, k, v, c, False, docs=cu)
    for r in range(T):
        i = max(j for j in range(len(cu) - 1) if cu[j] <= r)
        keys = range(cu[i], cu[i + 1])
        s = [c * sum(q[r, j] * k[l, j] for j in range(d)) for l in keys]
        m = max(s)
        e = [math.exp(x - m) for x in s]
        o = [sum(e[t] * v[l, j] for t, l in enumerate(keys)) / sum(e) for j in range(d)]
        assert np.allclose(O[r], o, atol=1e-13) and abs(L[r] - m - math.log(sum(e))) < 1e-13


def test_single_document_is_the_plain_problem():
    rng = np.random.default_rng(23)
    q, k, v = _rand(rng, 50, 4), _rand(rng, 50, 4), _rand(rng, 50, 4)
    for causal in (False, True):
        a = naive.forward_head(q, k, v, 0.5, causal)
        b = naive.forward_head(q, k, v, 0.5, causal, docs=[0, 50])
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


@pytest.mark.parametrize("causal", [False, True])
def test_document_gradients_by_finite_differences(causal):
    rng = np.random.default_rng(24)
    cu = [0, 4, 9, 14]
    T, d, c = cu[-1], 3, 0.7
    q, k, v, do = (_rand(rng, T, d) for _ in range(4))
    dQ, dK, dV = naive.backward_head(q, k, v, do, c, causal, docs=cu)[:3]

    def loss(q_, k_, v_):
        return float(np.sum(naive.forward_head(q_, k_, v_, c, causal, docs=cu)[0] * do))

    h = 1e-6
    for name, arr, grad in (("q", q, dQ), ("k", k, dK), ("v", v, dV)):
        for idx in [(0, 0), (4, 1), (8, 2), (13, 0)]:
            p, m = arr.copy(), arr.copy()
            p[idx] += h
            m[idx] -= h
            ap = {"q": q, "k": k, "v": v}
            am = dict(ap)
            ap[name], am[name] = p, m
            fd = (loss(ap["q"], ap["k"], ap["v"]) - loss(am["q"], am["k"], am["v"])) / (2 * h)
            assert abs(fd - grad[idx]) <= 1e-6 * (1 + abs(fd)), (name, idx, fd, grad[idx])
