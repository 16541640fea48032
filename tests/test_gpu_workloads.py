"""The five workloads at full size, in the launch configuration the benchmark times,
checked against the float64 oracle on sampled heads (whole heads: every output of
the head) or, where a head's score matrix is too large for the oracle, on sampled
query rows (each row is exact on its own: it depends only on its query and all
keys)."""
import math

import numpy as np
import pytest

import io_aware_exact_02_amd as fa
from io_aware_exact_02_amd.inputs import WORKLOADS
from oracle import naive
from tests.gpu_util import TOL_GRAD, TOL_LSE, TOL_O, draw, maxabs, to_f64, torch

pytestmark = pytest.mark.gpu


def _inputs(name, with_do):
    w = WORKLOADS[name]
    dev, f = draw(w.B, w.H, w.Tq, w.Tk, w.d, w.dtype, w.seed, w.qk_spread, with_do)
    return w, dev, f


def _heads(w, n, seed):
    allh = [(b, h) for b in range(w.B) for h in range(w.H)]
    pick = {allh[0], allh[-1]}
    rng = np.random.default_rng(seed)
    while len(pick) < min(n, len(allh)):
        pick.add(allh[int(rng.integers(len(allh)))])
    return sorted(pick)


def _check_fwd_heads(w, f, O, lse, heads):
    scale = 1 / math.sqrt(w.d)
    for b, h in heads:
        Or, Lr = naive.forward_head(f["q"][b, h], f["k"][b, h], f["v"][b, h], scale, w.causal)
        assert maxabs(to_f64(O[b, h]), Or) <= TOL_O[w.dtype], (b, h)
        assert maxabs(to_f64(lse[b, h]), Lr) <= TOL_LSE, (b, h)


def _check_bwd_heads(w, f, dQ, dK, dV, heads):
    scale = 1 / math.sqrt(w.d)
    for b, h in heads:
        rQ, rK, rV = naive.backward_head(f["q"][b, h], f["k"][b, h], f["v"][b, h], f["do"][b, h], scale,
                                         w.causal)[:3]
        for got, ref, name in ((dQ, rQ, "dQ"), (dK, rK, "dK"), (dV, rV, "dV")):
            err = maxabs(to_f64(got[b, h]), ref)
            assert err <= TOL_GRAD[w.dtype], (name, b, h, err)


def test_fwd_f32_b1h1_t256_d64():
    w, dev, f = _inputs("fwd_f32_b1h1_t256_d64", False)
    O, lse = fa.forward(dev["q"], dev["k"], dev["v"], causal=w.causal)
    torch().cuda.synchronize()
    _check_fwd_heads(w, f, O, lse, [(0, 0)])


def test_causal_bf16_b8h32_t4096_d128_forward_and_backward():
    w, dev, f = _inputs("causal_bf16_b8h32_t4096_d128", True)
    O, lse = fa.forward(dev["q"], dev["k"], dev["v"], causal=True)
    torch().cuda.synchronize()
    _check_fwd_heads(w, f, O, lse, _heads(w, 4, 1))
    dQ, dK, dV = fa.backward(dev["q"], dev["k"], dev["v"], O, dev["do"], lse, causal=True)
    torch().cuda.synchronize()
    _check_bwd_heads(w, f, dQ, dK, dV, _heads(w, 2, 2))


def test_causal_bf16_b4h16_t16384_d64_forward_and_backward():
    w, dev, f = _inputs("causal_bf16_b4h16_t16384_d64", True)
    O, lse = fa.forward(dev["q"], dev["k"], dev["v"], causal=True)
    dQ, dK, dV = fa.backward(dev["q"], dev["k"], dev["v"], O, dev["do"], lse, causal=True)
    torch().cuda.synchronize()
    heads = _heads(w, 1, 3)
    _check_fwd_heads(w, f, O, lse, heads)
    _check_bwd_heads(w, f, dQ, dK, dV, heads)


def test_causal_bf16_b1h24_t65536_d256_forward_sampled_rows():
    w, dev, f = _inputs("causal_bf16_b1h24_t65536_d256", False)
    O, lse = fa.forward(dev["q"], dev["k"], dev["v"], causal=True)
    torch().cuda.synchronize()
    rng = np.random.default_rng(4)
    rows = np.unique(np.concatenate([[0, 1, 127, 128, 4095, 32768, w.Tq - 2, w.Tq - 1],
                                     rng.integers(0, w.Tq, 40)]))
    scale = 1 / math.sqrt(w.d)
    for b, h in _heads(w, 2, 5):
        Or, Lr = naive.forward_head(f["q"][b, h], f["k"][b, h], f["v"][b, h], scale, True, rows=rows)
        assert maxabs(to_f64(O[b, h][rows]), Or) <= TOL_O[w.dtype]
        assert maxabs(to_f64(lse[b, h][rows]), Lr) <= TOL_LSE
    assert torch().isfinite(O).all() and torch().isfinite(lse).all()


def test_d256_backward_whole_heads_t4096():
    """The d = 256 backward (key-block sweep plus dQ sweep) on whole heads of T = 4096,
    causal and not, against the oracle element by element."""
    t = torch()
    B, H, T, d = 1, 2, 4096, 256
    dev, f = draw(B, H, T, T, d, "bf16", seed=9256, with_do=True)
    scale = 1 / math.sqrt(d)
    for causal in (True, False):
        O, lse = fa.forward(dev["q"], dev["k"], dev["v"], causal=causal)
        dQ, dK, dV = fa.backward(dev["q"], dev["k"], dev["v"], O, dev["do"], lse, causal=causal)
        t.cuda.synchronize()
        for h in range(H):
            rQ, rK, rV = naive.backward_head(f["q"][0, h], f["k"][0, h], f["v"][0, h], f["do"][0, h], scale,
                                             causal)[:3]
            for got, ref, name in ((dQ, rQ, "dQ"), (dK, rK, "dK"), (dV, rV, "dV")):
                err = maxabs(to_f64(got[0, h]), ref)
                assert err <= TOL_GRAD["bf16"], (causal, name, h, err)


def test_causal_bf16_b1h24_t65536_d256_backward_sampled_rows():
    """The d = 256 backward at full size (24 heads x 65536): dQ on sampled rows against
    the oracle (a dQ row needs only its own row of P, dP and D), dK on sampled keys of
    the sequence's tail, and dV through an exact identity: rows of P sum to 1, so sum_l dV_l = sum_r dO_r.  With P rounded to bf16
    before the dV product each row's weights sum to 1 within 2^-9, which bounds the
    difference by 2^-9 sum_r |dO_r| (plus float32 summation slack)."""
    t = torch()
    w, dev, f = _inputs("causal_bf16_b1h24_t65536_d256", True)
    O, lse = fa.forward(dev["q"], dev["k"], dev["v"], causal=True)
    dQ, dK, dV = fa.backward(dev["q"], dev["k"], dev["v"], O, dev["do"], lse, causal=True, grad_dtype=t.float32)
    t.cuda.synchronize()
    assert t.isfinite(dQ).all() and t.isfinite(dK).all() and t.isfinite(dV).all()
    rng = np.random.default_rng(6)
    rows = np.unique(np.concatenate([[0, 1, 127, 128, 32768, w.Tq - 1], rng.integers(0, w.Tq, 26)]))
    scale = 1 / math.sqrt(w.d)
    dv_sum = dV.sum(dim=2, dtype=t.float64).cpu().numpy()
    for b, h in _heads(w, 2, 7):
        ref = naive.dq_rows(f["q"][b, h], f["k"][b, h], f["v"][b, h], f["do"][b, h], scale, True, rows)
        assert maxabs(to_f64(dQ[b, h][rows]), ref) <= TOL_GRAD["bf16"], (b, h)
    do = f["do"]
    bound = (2.0 ** -9 + 1e-5) * np.abs(do).sum(axis=2) + 1e-3
    assert np.all(np.abs(dv_sum - do.sum(axis=2)) <= bound)
    # dK on sampled keys: a key's column of dK needs D_r (hence O) of every row that
    # sees it; keys in the last 2048 positions are seen by at most 2048 rows each
    keys = np.unique(np.concatenate([[w.Tk - 2048, w.Tk - 1], rng.integers(w.Tk - 2048, w.Tk, 14)]))
    for b, h in _heads(w, 2, 8):
        ref = naive.dk_cols(f["q"][b, h], f["k"][b, h], f["v"][b, h], f["do"][b, h], scale, True, keys)
        assert maxabs(to_f64(dK[b, h][keys]), ref) <= TOL_GRAD["bf16"], (b, h)


def test_cross_bf16_b16h16_tq1024_tk8192_d128_forward_and_backward():
    """Q, K ~ N(0, 9): peaked softmax with large logits.

    The bf16 forward output O is checked at the O tolerance.  For the backward,
    O is carried between the passes in float32 and the gradients are returned
    in float32: rounding O to bf16 alone moves D = dO . O enough to put dQ past
    the gradient tolerance (dQ errs by scale * dD * the weighted mean key, and
    the keys are three times larger here), and the gradients reach magnitudes
    where bf16's own rounding step is of the order of the tolerance."""
    t = torch()
    w, dev, f = _inputs("cross_bf16_b16h16_tq1024_tk8192_d128", True)
    heads = _heads(w, 3, 6)
    O, lse = fa.forward(dev["q"], dev["k"], dev["v"], causal=False)
    t.cuda.synchronize()
    _check_fwd_heads(w, f, O, lse, heads)
    O32, lse32 = fa.forward(dev["q"], dev["k"], dev["v"], causal=False, out_dtype=t.float32)
    dQ, dK, dV = fa.backward(dev["q"], dev["k"], dev["v"], O32, dev["do"], lse32, causal=False,
                             grad_dtype=t.float32)
    t.cuda.synchronize()
    _check_fwd_heads(w, f, O32, lse32, heads)
    _check_bwd_heads(w, f, dQ, dK, dV, heads)
    del dQ, dK, dV, O32, lse32
    _check_bwd_through_bf16_o(w, f, dev, O, lse, heads)


def _check_bwd_through_bf16_o(w, f, dev, O, lse, heads):
    """The same backward fed the bf16 O of the forward (and returning bf16 or float32
    gradients), against a bound derived from the rounding of O.  Rounding O to
    bf16 moves each element by at most 2^-8 of itself, so D_r = dO_r . O_r moves
    by at most e_r = 2^-8 sum_k |dO_rk O_rk|.  D enters every dS_rl = P_rl (dP_rl -
    D_r), so dQ_r moves by at most c e_r |(P K)_r| and dK_l by at most
    c sum_r P_rl e_r |Q_r|, elementwise; dV does not depend on D.  The check is the
    gradient tolerance plus that bound (plus, for bf16 gradients, their own
    rounding of at most 2^-8 of the value)."""
    t = torch()
    c = 1 / math.sqrt(w.d)
    u = 2.0 ** -8
    tol = TOL_GRAD[w.dtype]
    for gdt in (t.float32, t.bfloat16):
        dQ, dK, dV = fa.backward(dev["q"], dev["k"], dev["v"], O, dev["do"], lse, causal=w.causal, grad_dtype=gdt)
        t.cuda.synchronize()
        out_u = u if gdt == t.bfloat16 else 0.0
        worst = {"dQ": 0.0, "dK": 0.0, "dV": 0.0}
        for b, h in heads:
            q, k, v, do = (f[n][b, h] for n in ("q", "k", "v", "do"))
            rQ, rK, rV, rO = naive.backward_head(q, k, v, do, c, w.causal)[:4]
            P = naive.probs_head(q, k, c, w.causal)[0]
            e = u * np.sum(np.abs(do * rO), axis=1)                      # bound on |dD_r|
            bq = c * e[:, None] * np.abs(P @ k)
            bk = c * (P.T @ (e[:, None] * np.abs(q)))
            for got, ref, bnd, name in ((dQ, rQ, bq, "dQ"), (dK, rK, bk, "dK"), (dV, rV, 0.0, "dV")):
                err = np.abs(to_f64(got[b, h]) - ref)
                lim = tol + bnd
                lim = lim + out_u * (np.abs(ref) + lim)
                assert np.all(err <= lim), (name, str(gdt), b, h, float((err - lim).max()))
                worst[name] = max(worst[name], float(err.max()))
        print(f"cross-attention backward through bf16 O, {gdt} gradients: max abs errors {worst}", flush=True)
        del dQ, dK, dV
