"""Pins for the fp64 oracle against facts the pages and the mathematics fix.

Each `check_*` function takes a (forward_head, backward_head) pair so that the
same pin runs against the oracle (must pass) and against deliberately broken
copies of it (`test_pins_catch_planted_mistakes`, must fail): a dropped term,
a wrong sign or index, or a transposed operand anywhere in the oracle trips at
least one pin.  CPU only.
"""
import math
import os

import numpy as np
import pytest

from oracle import naive, tiled_model

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    vals = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            k, v = (s.strip() for s in line.split("=", 1))
            nums = [float(x) for x in v.split()]
            vals[k] = nums[0] if len(nums) == 1 else nums
    return vals


def _rand(shape, seed, scale=1.0):
    return scale * np.random.default_rng(seed).standard_normal(shape)


ORACLE = (naive.forward_head, naive.backward_head)


# --------------------------------------------------------------------------------------
# pin functions
# --------------------------------------------------------------------------------------
def check_worked_example(fwd, bwd):
    """[LDD] "Concept": scores [1,3] then [5] -> l = 1.154, weight on 3 = 0.117."""
    g = _golden("online_softmax_worked_example.txt")
    q = np.array([[1.0, 0.0, 0.0]])
    k = np.array([[1.0, 0, 0], [3.0, 0, 0], [5.0, 0, 0]])
    v = np.eye(3)
    O, lse = fwd(q, k, v, 1.0, False)
    tol = 5e-4 + 1e-12                       # the page prints three decimals
    assert abs(O[0, 1] - g["true_weight_of_3"]) <= tol
    assert abs(math.exp(lse[0] - 5.0) - g["l_final"]) <= tol
    assert abs(O[0, 2] * math.exp(lse[0] - 5.0) - g["direct_terms"][2]) <= tol
    assert abs(O[0, 0] * math.exp(lse[0] - 5.0) - g["direct_terms"][0]) <= tol
    # exact values derived from the same scores
    assert abs(lse[0] - math.log(math.exp(1) + math.exp(3) + math.exp(5))) < 1e-13
    assert abs(O[0, 1] - 0.11731042782619835) < 1e-13


def check_rows_sum_to_one(fwd, bwd):
    """Rows of P sum to 1 ([ZtF] "The forward pass", why the result is exact): with
    V = ones-column-augmented identity, O's extra column is the row sum of P."""
    for causal in (False, True):
        q, k = _rand((7, 5), 1), _rand((7, 5), 2)
        v = np.concatenate([np.eye(7), np.ones((7, 1))], axis=1)
        O, _ = fwd(q, k, v, 0.7, causal)
        assert np.allclose(O[:, -1], 1.0, atol=1e-14, rtol=0)
        assert np.allclose(O[:, :-1].sum(axis=1), 1.0, atol=1e-14, rtol=0)
        assert (O[:, :-1] >= 0).all()
        if causal:
            assert np.all(np.triu(O[:, :-1], 1) == 0.0)    # key l > query r weighs 0


def check_constant_v(fwd, bwd):
    """V with identical rows gives O = v for any Q, K, mask, and dQ = dK = 0."""
    for causal in (False, True):
        q, k = _rand((6, 4), 3), _rand((9, 4), 4)
        row = _rand((1, 4), 5)
        v = np.repeat(row, 9, axis=0)
        O, _ = fwd(q, k, v, 0.5, causal)
        assert np.allclose(O, np.repeat(row, 6, axis=0), atol=1e-14, rtol=0)
        do = _rand((6, 4), 6)
        dQ, dK, dV = bwd(q, k, v, do, 0.5, causal)[:3]
        assert np.abs(dQ).max() < 1e-13 and np.abs(dK).max() < 1e-13
        assert np.allclose(dV.sum(axis=0), do.sum(axis=0), atol=1e-13)


def check_zero_query(fwd, bwd):
    """Q = 0: uniform weights over visible keys.  O_r = mean of visible V rows,
    lse_r = ln(#visible): ln(Tk) non-causal, ln(r + 1) causal (top-left)."""
    for Tq, Tk in ((8, 8), (5, 9), (9, 5)):
        q = np.zeros((Tq, 3)); k = _rand((Tk, 3), 7); v = _rand((Tk, 2), 8)
        O, lse = fwd(q, k, v, 1.3, False)
        assert np.allclose(O, np.repeat(v.mean(axis=0, keepdims=True), Tq, 0), atol=1e-14)
        assert np.allclose(lse, math.log(Tk), atol=1e-14)
        O, lse = fwd(q, k, v, 1.3, True)
        for r in range(Tq):
            n = min(r + 1, Tk)
            assert np.allclose(O[r], v[:n].mean(axis=0), atol=1e-14)
            assert abs(lse[r] - math.log(n)) < 1e-14


def _loss(fwd, q, k, v, do, scale, causal):
    return float(np.sum(fwd(q, k, v, scale, causal)[0] * do))


def check_finite_differences(fwd, bwd):
    """Central differences of L = sum(O * dO) ([ZtF] "In PyTorch": gradcheck)."""
    h = 1e-6
    for causal in (False, True):
        q, k, v = _rand((3, 4), 10), _rand((5, 4), 11), _rand((5, 4), 12)
        do = _rand((3, 4), 13)
        scale = 0.8
        dQ, dK, dV = bwd(q, k, v, do, scale, causal)[:3]
        for X, G in ((q, dQ), (k, dK), (v, dV)):
            num = np.zeros_like(X)
            for idx in np.ndindex(X.shape):
                old = X[idx]
                X[idx] = old + h; lp = _loss(fwd, q, k, v, do, scale, causal)
                X[idx] = old - h; lm = _loss(fwd, q, k, v, do, scale, causal)
                X[idx] = old
                num[idx] = (lp - lm) / (2 * h)
            assert np.allclose(G, num, rtol=1e-6, atol=1e-8), (causal, np.abs(G - num).max())


def check_invariants(fwd, bwd):
    """sum_l dV_l = sum_r dO_r; sum_l dK_l = 0; <dQ,Q> = <dK,K>; D_r = dO_r . O_r."""
    for causal in (False, True):
        q, k, v, do = _rand((12, 6), 20), _rand((12, 6), 21), _rand((12, 6), 22), _rand((12, 6), 23)
        dQ, dK, dV, O, lse, D = bwd(q, k, v, do, 0.4, causal)
        assert np.allclose(dV.sum(axis=0), do.sum(axis=0), atol=1e-12)
        assert np.allclose(dK.sum(axis=0), 0.0, atol=1e-12)
        assert abs(np.sum(dQ * q) - np.sum(dK * k)) < 1e-12
        O2, lse2 = fwd(q, k, v, 0.4, causal)
        assert np.allclose(O, O2, atol=1e-14) and np.allclose(lse, lse2, atol=1e-14)
        assert np.allclose(D, np.sum(do * O2, axis=1), atol=1e-13)


def check_single_key(fwd, bwd):
    """Tk = 1: O = v_0, lse = s_00, dQ = dK = 0, dV_0 = sum_r dO_r."""
    q, k, v, do = _rand((4, 3), 30), _rand((1, 3), 31), _rand((1, 3), 32), _rand((4, 3), 33)
    for causal in (False, True):
        O, lse = fwd(q, k, v, 0.9, causal)
        assert np.allclose(O, np.repeat(v, 4, axis=0), atol=1e-15)
        assert np.allclose(lse, 0.9 * (q @ k[0]), atol=1e-14)
        dQ, dK, dV = bwd(q, k, v, do, 0.9, causal)[:3]
        assert np.abs(dQ).max() < 1e-14 and np.abs(dK).max() < 1e-14
        assert np.allclose(dV[0], do.sum(axis=0), atol=1e-14)


def check_torch_sdpa(fwd, bwd):
    """PyTorch's own CPU float64 scaled_dot_product_attention (an independent
    implementation) with autograd ([ZtF] "In PyTorch")."""
    torch = pytest.importorskip("torch")
    F = torch.nn.functional
    for causal in (False, True):
        # causal with Tq != Tk too: torch's is_causal keeps key l <= query r (top-left),
        # the alignment the library takes (both ways round)
        for (Tq, Tk) in ((11, 11), (6, 13), (13, 6)):
            d = 8
            q, k, v, do = _rand((Tq, d), 40), _rand((Tk, d), 41), _rand((Tk, d), 42), _rand((Tq, d), 43)
            scale = 1.0 / math.sqrt(d) * 1.7
            tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
            to = F.scaled_dot_product_attention(tq[None], tk[None], tv[None], is_causal=causal, scale=scale)[0]
            to.backward(torch.tensor(do))
            O, _ = fwd(q, k, v, scale, causal)
            dQ, dK, dV = bwd(q, k, v, do, scale, causal)[:3]
            assert np.abs(O - to.detach().numpy()).max() < 1e-12
            assert np.abs(dQ - tq.grad.numpy()).max() < 1e-12
            assert np.abs(dK - tk.grad.numpy()).max() < 1e-12
            assert np.abs(dV - tv.grad.numpy()).max() < 1e-12


def check_brute_force(fwd, bwd):
    """Pure-Python loops with math.exp on a tiny case, straight from the formula."""
    Tq, Tk, d = 4, 6, 3
    q, k, v = _rand((Tq, d), 50), _rand((Tk, d), 51), _rand((Tk, d), 52)
    scale = 0.6
    for causal in (False, True):
        O, lse = fwd(q, k, v, scale, causal)
        for r in range(Tq):
            vis = [l for l in range(Tk) if (not causal or l <= r)]
            s = {l: scale * sum(q[r, t] * k[l, t] for t in range(d)) for l in vis}
            z = sum(math.exp(s[l]) for l in vis)
            assert abs(lse[r] - math.log(z)) < 1e-13
            for c in range(d):
                ref = sum(math.exp(s[l]) / z * v[l, c] for l in vis)
                assert abs(O[r, c] - ref) < 1e-13


def check_overflow_safety(fwd, bwd):
    """Scores of order 1e4 stay finite; exponent S - lse never positive
    ([ZtF] "What the forward pass leaves behind")."""
    q, k, v = _rand((8, 4), 60, 100.0), _rand((8, 4), 61, 100.0), _rand((8, 4), 62)
    for causal in (False, True):
        O, lse = fwd(q, k, v, 0.5, causal)
        assert np.isfinite(O).all() and np.isfinite(lse).all()
        S = naive.scores_head(q, k, 0.5, causal)
        assert np.nanmax(S - lse[:, None]) <= 0.0
        dQ, dK, dV = bwd(q, k, v, _rand((8, 4), 63), 0.5, causal)[:3]
        assert np.isfinite(dQ).all() and np.isfinite(dK).all() and np.isfinite(dV).all()


def check_permutations(fwd, bwd):
    """Non-causal: permuting K,V rows together leaves O unchanged; permuting Q rows
    permutes O."""
    q, k, v = _rand((7, 4), 70), _rand((9, 4), 71), _rand((9, 4), 72)
    O, lse = fwd(q, k, v, 0.5, False)
    p = np.random.default_rng(73).permutation(9)
    O2, lse2 = fwd(q, k[p], v[p], 0.5, False)
    assert np.allclose(O, O2, atol=1e-14) and np.allclose(lse, lse2, atol=1e-14)
    r = np.random.default_rng(74).permutation(7)
    O3, _ = fwd(q[r], k, v, 0.5, False)
    assert np.allclose(O3, O[r], atol=1e-15)


PINS = [check_worked_example, check_rows_sum_to_one, check_constant_v, check_zero_query,
        check_finite_differences, check_invariants, check_single_key, check_torch_sdpa,
        check_brute_force, check_overflow_safety, check_permutations]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_oracle_pin(pin):
    pin(*ORACLE)


# --------------------------------------------------------------------------------------
# planted mistakes: each broken copy of the oracle must fail at least one pin
# --------------------------------------------------------------------------------------
def _mutant(kind):
    def scores(q, k, scale, causal, rows=None):
        q = np.asarray(q, float); k = np.asarray(k, float)
        rows = np.arange(q.shape[0]) if rows is None else np.asarray(rows)
        sc = 1.0 if kind == "no_scale" else scale
        S = sc * (q[rows] @ k.T)
        if causal:
            vis = np.arange(k.shape[0])[None, :] <= rows[:, None]
            if kind == "mask_flipped":
                vis = np.arange(k.shape[0])[None, :] >= rows[:, None]
            if kind == "mask_strict":
                vis = np.arange(k.shape[0])[None, :] < rows[:, None] + (rows[:, None] == 0)
            S = np.where(vis, S, -np.inf)
        return S

    def probs(q, k, scale, causal, rows=None):
        S = scores(q, k, scale, causal, rows)
        m = S.max(axis=1)
        E = np.exp(S - m[:, None])
        l = E.sum(axis=1)
        lse = np.log(l) if kind == "lse_no_max" else m + np.log(l)
        if kind == "lse_log2":
            lse = (m + np.log(l)) / math.log(2)
        return E / l[:, None], lse

    def fwd(q, k, v, scale, causal, rows=None):
        P, lse = probs(q, k, scale, causal, rows)
        v = np.asarray(v, float)
        if kind == "pv_transposed" and P.shape[1] == v.shape[0] and P.shape[0] == P.shape[1]:
            return P.T @ v, lse
        return P @ v, lse

    def bwd(q, k, v, do, scale, causal):
        q, k, v, do = (np.asarray(x, float) for x in (q, k, v, do))
        P, lse = probs(q, k, scale, causal)
        O = P @ v
        dV = P.T @ do
        dP = do @ v.T
        D = np.sum(do * O, axis=1)
        if kind == "D_dropped":
            D = 0 * D
        dS = P * (dP - D[:, None]) if kind != "dS_sign" else P * (D[:, None] - dP)
        dQ = (1.0 if kind == "dq_no_scale" else scale) * (dS @ k)
        dK = scale * (dS.T @ (k if kind == "dk_wrong_operand" else q))   # wrong operand
        if kind == "dv_transposed":
            dV = P @ do                                                  # P instead of P^T
        return dQ, dK, dV, O, lse, D

    return fwd, bwd


MUTANTS = ["no_scale", "mask_flipped", "mask_strict", "lse_no_max", "lse_log2", "pv_transposed",
           "D_dropped", "dS_sign", "dq_no_scale", "dk_wrong_operand", "dv_transposed"]


@pytest.mark.parametrize("kind", MUTANTS)
def test_pins_catch_planted_mistakes(kind):
    fwd, bwd = _mutant(kind)
    failed = []
    for pin in PINS:
        try:
            pin(fwd, bwd)
        except (AssertionError, ValueError, IndexError):
            failed.append(pin.__name__)
    assert failed, f"no pin caught the planted mistake {kind!r}"


def test_mutant_harness_is_faithful_when_unbroken():
    """The mutant factory with no mistake passes every pin (so failures above are
    due to the planted mistake, not the harness)."""
    fwd, bwd = _mutant("none")
    for pin in PINS:
        pin(fwd, bwd)


# --------------------------------------------------------------------------------------
# batched wrappers and sampled rows
# --------------------------------------------------------------------------------------
def test_batched_matches_per_head_and_rows_subset():
    Q, K, V, dO = (_rand((2, 3, 10, 4), s) for s in (80, 81, 82, 83))
    O, L = naive.forward(Q, K, V, 0.5, True, workers=2)
    dQ, dK, dV, O2, L2 = naive.backward(Q, K, V, dO, 0.5, True, workers=2)
    for b in range(2):
        for h in range(3):
            o, l = naive.forward_head(Q[b, h], K[b, h], V[b, h], 0.5, True)
            assert np.array_equal(O[b, h], o) and np.array_equal(L[b, h], l)
            assert np.allclose(O2[b, h], o, atol=1e-15)
    rows = np.array([0, 3, 9])
    Os, Ls = naive.forward(Q, K, V, 0.5, True, heads=[(1, 2)], rows=rows)
    assert np.allclose(Os[1, 2], O[1, 2][rows], atol=1e-15)
    assert np.isnan(Os[0, 0]).all()


@pytest.mark.parametrize("causal", [False, True])
def test_dq_rows_by_finite_differences(causal):
    """dq_rows pinned by central differences of L = sum(O * dO) in q[r, j]: a change of
    query r moves only row r of O, so the difference needs the forward of that row alone."""
    rng = np.random.default_rng(90)
    Tq, Tk, d, c = 40, 37, 5, 0.6
    q, k, v, do = (rng.standard_normal(sh) for sh in ((Tq, d), (Tk, d), (Tk, d), (Tq, d)))
    rows = np.array([0, 7, 23, 39])
    got = naive.dq_rows(q, k, v, do, c, causal, rows)
    h = 1e-6
    for i, r in enumerate(rows):
        for j in range(d):
            p, m = q.copy(), q.copy()
            p[r, j] += h
            m[r, j] -= h
            Op, _ = naive.forward_head(p, k, v, c, causal, rows=np.array([r]))
            Om, _ = naive.forward_head(m, k, v, c, causal, rows=np.array([r]))
            fd = float(np.sum((Op - Om)[0] * do[r])) / (2 * h)
            assert abs(fd - got[i, j]) <= 1e-7 * (1 + abs(fd)), (r, j, fd, got[i, j])
    # and it is the same rows of the whole-head backward (block mask included)
    bm = np.array([[1]], np.uint8)
    full = naive.backward_head(q, k, v, do, c, causal, block_mask=bm)[0]
    assert np.allclose(naive.dq_rows(q, k, v, do, c, causal, rows, block_mask=bm), full[rows], atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_dk_cols_by_finite_differences(causal):
    """dk_cols pinned by central differences of L = sum(O * dO) in k[l, j] (every row
    of O that sees key l moves), and equal to the same columns of the whole-head
    backward, with and without a block mask and in row blocks smaller than the head."""
    rng = np.random.default_rng(91)
    Tq, Tk, d, c = 23, 29, 5, 0.7
    q, k, v, do = (rng.standard_normal(sh) for sh in ((Tq, d), (Tk, d), (Tk, d), (Tq, d)))
    cols = np.array([0, 4, 17, 22, 28])
    got = naive.dk_cols(q, k, v, do, c, causal, cols, row_block=7)
    h = 1e-6
    for i, l in enumerate(cols):
        for j in range(d):
            p, m = k.copy(), k.copy()
            p[l, j] += h
            m[l, j] -= h
            fd = (_loss(naive.forward_head, q, p, v, do, c, causal) -
                  _loss(naive.forward_head, q, m, v, do, c, causal)) / (2 * h)
            assert abs(fd - got[i, j]) <= 1e-7 * (1 + abs(fd)), (l, j, fd, got[i, j])
    full = naive.backward_head(q, k, v, do, c, causal)[1]
    assert np.allclose(got, full[cols], atol=1e-13)
    bm = np.array([[1]], np.uint8)
    full_m = naive.backward_head(q, k, v, do, c, causal, block_mask=bm)[1]
    assert np.allclose(naive.dk_cols(q, k, v, do, c, causal, cols, block_mask=bm, row_block=5), full_m[cols],
                       atol=1e-13)
