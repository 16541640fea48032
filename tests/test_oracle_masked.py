"""Pins of the oracle's block-mask path ([ZtF] "Dropout, block-sparsity, and other
real-kernel details"), each checked against something other than the masked code
itself: the unmasked oracle on the restricted problem, closed forms for rows with
no visible key, and central finite differences."""
import math

import numpy as np
import pytest

from oracle import naive

MB = naive.MASK_BLOCK


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def test_all_ones_mask_equals_unmasked():
    rng = np.random.default_rng(1)
    Tq, Tk, d = 300, 260, 8
    q, k, v, do = _rand(rng, Tq, d), _rand(rng, Tk, d), _rand(rng, Tk, d), _rand(rng, Tq, d)
    bm = np.ones((math.ceil(Tq / MB), math.ceil(Tk / MB)), np.uint8)
    for causal in (False, True):
        O0, L0 = naive.forward_head(q, k, v, 0.3, causal)
        O1, L1 = naive.forward_head(q, k, v, 0.3, causal, block_mask=bm)
        assert np.array_equal(O0, O1) and np.array_equal(L0, L1)
        g0 = naive.backward_head(q, k, v, do, 0.3, causal)
        g1 = naive.backward_head(q, k, v, do, 0.3, causal, block_mask=bm)
        for a, b in zip(g0, g1):
            assert np.array_equal(a, b)


def test_single_key_block_is_the_restricted_problem():
    """Query block 1 keeps only key block 2: its rows equal attention over those keys alone,
    and dK, dV vanish outside the kept keys."""
    rng = np.random.default_rng(2)
    Tq, Tk, d = 2 * MB, 3 * MB + 40, 6
    q, k, v, do = _rand(rng, Tq, d), _rand(rng, Tk, d), _rand(rng, Tk, d), _rand(rng, Tq, d)
    bm = np.zeros((2, 4), np.uint8)
    bm[0, :] = 1                     # query block 0: everything
    bm[1, 2] = 1                     # query block 1: keys 256..383 only
    O, L = naive.forward_head(q, k, v, 0.4, False, block_mask=bm)
    sub = slice(2 * MB, 3 * MB)
    Or, Lr = naive.forward_head(q[MB:], k[sub], v[sub], 0.4, False)
    assert np.allclose(O[MB:], Or, atol=1e-13) and np.allclose(L[MB:], Lr, atol=1e-13)
    Of, Lf = naive.forward_head(q[:MB], k, v, 0.4, False)
    assert np.allclose(O[:MB], Of, atol=1e-13) and np.allclose(L[:MB], Lf, atol=1e-13)
    # backward: rows of query block 1 only touch keys of block 2
    do1 = do.copy()
    do1[:MB] = 0.0
    dQ, dK, dV, _, _, _ = naive.backward_head(q, k, v, do1, 0.4, False, block_mask=bm)
    rQ, rK, rV, _, _, _ = naive.backward_head(q[MB:], k[sub], v[sub], do1[MB:], 0.4, False)
    assert np.allclose(dQ[MB:], rQ, atol=1e-12)
    assert np.allclose(dK[sub], rK, atol=1e-12) and np.allclose(dV[sub], rV, atol=1e-12)
    outside = np.ones(Tk, bool)
    outside[sub] = False
    assert np.abs(dK[outside]).max() == 0.0 and np.abs(dV[outside]).max() == 0.0


def test_rows_without_visible_keys():
    """A query block whose mask row is empty: O = 0, lse = -inf, no gradient in or out."""
    rng = np.random.default_rng(3)
    Tq, Tk, d = MB + 30, 2 * MB, 5
    q, k, v, do = _rand(rng, Tq, d), _rand(rng, Tk, d), _rand(rng, Tk, d), _rand(rng, Tq, d)
    bm = np.array([[1, 0], [0, 0]], np.uint8)
    O, L = naive.forward_head(q, k, v, 0.5, False, block_mask=bm)
    assert np.all(O[MB:] == 0.0) and np.all(L[MB:] == -np.inf)
    assert np.all(np.isfinite(O[:MB]))
    dQ, dK, dV, _, _, D = naive.backward_head(q, k, v, do, 0.5, False, block_mask=bm)
    assert np.all(dQ[MB:] == 0.0) and np.all(D[MB:] == 0.0)
    assert np.all(dK[MB:] == 0.0) and np.all(dV[MB:] == 0.0)      # key block 1 is never seen
    # the visible part equals the unmasked problem on query block 0 and key block 0
    rQ, rK, rV, _, _, _ = naive.backward_head(q[:MB], k[:MB], v[:MB], do[:MB], 0.5, False)
    assert np.allclose(dQ[:MB], rQ, atol=1e-12) and np.allclose(dK[:MB], rK, atol=1e-12)
    assert np.allclose(dV[:MB], rV, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_masked_gradients_by_finite_differences(causal):
    """Central differences of L = sum(O * dO) on sampled entries, with a block mask that
    leaves one query block partly blind (only its diagonal key block)."""
    rng = np.random.default_rng(4)
    Tq, Tk, d = MB + 7, MB + 9, 3
    q, k, v, do = _rand(rng, Tq, d), _rand(rng, Tk, d), _rand(rng, Tk, d), _rand(rng, Tq, d)
    bm = np.array([[1, 1], [0, 1]], np.uint8)
    c = 0.7
    dQ, dK, dV, _, _, _ = naive.backward_head(q, k, v, do, c, causal, block_mask=bm)

    def loss(q_, k_, v_):
        O, _ = naive.forward_head(q_, k_, v_, c, causal, block_mask=bm)
        return float(np.sum(O * do))

    h = 1e-6
    for name, arr, grad in (("q", q, dQ), ("k", k, dK), ("v", v, dV)):
        for idx in [(0, 0), (MB - 1, 2), (MB, 1), (arr.shape[0] - 1, 0), (arr.shape[0] // 2, 2)]:
            p, m = arr.copy(), arr.copy()
            p[idx] += h
            m[idx] -= h
            args_p = {"q": q, "k": k, "v": v}
            args_m = {"q": q, "k": k, "v": v}
            args_p[name], args_m[name] = p, m
            fd = (loss(**{f"{x}_": args_p[x] for x in "qkv"}) - loss(**{f"{x}_": args_m[x] for x in "qkv"})) / (2 * h)
            assert abs(fd - grad[idx]) <= 1e-6 * (1 + abs(fd)), (name, idx, fd, grad[idx])


def test_batched_wrapper_broadcasts_one_mask_or_takes_one_per_head():
    rng = np.random.default_rng(5)
    B, H, T, d = 1, 2, MB + 3, 4
    Q, K, V = (_rand(rng, B, H, T, d) for _ in range(3))
    shared = np.array([[[1, 0], [1, 1]]], np.uint8)
    per_head = np.array([[[1, 0], [1, 1]], [[1, 1], [1, 1]]], np.uint8)
    O1, _ = naive.forward(Q, K, V, 0.5, False, block_mask=shared, workers=1)
    O2, _ = naive.forward(Q, K, V, 0.5, False, block_mask=per_head, workers=1)
    O3, _ = naive.forward(Q, K, V, 0.5, False, workers=1)
    assert np.array_equal(O1[0, 0], O2[0, 0])
    assert np.array_equal(O2[0, 1], O3[0, 1])
    assert not np.allclose(O1[0, 1, :MB], O3[0, 1, :MB])
