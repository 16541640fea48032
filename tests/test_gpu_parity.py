"""HIP path against the float64 oracle, element by element, on seeded inputs:
small and ragged shapes (several tiles plus a tail), the three head widths, both
dtypes, causal and full attention, and the special cases with closed forms."""
import math

import numpy as np
import pytest

import io_aware_exact_02_amd as fa
from oracle import naive
from tests.gpu_util import TOL_GRAD, TOL_LSE, TOL_O, draw, maxabs, to_dev, to_f64, torch

pytestmark = pytest.mark.gpu

# causal workgroups take a short and a long block each: 200 gives two 128-row blocks (one
# workgroup runs both), 300 three (the middle one alone), 1000 eight
SHAPES = [(1, 1), (17, 17), (100, 100), (200, 200), (300, 300), (1000, 1000), (100, 257), (257, 100), (64, 513)]
DIMS = [64, 128, 256]


def _oracle_fwd(f, scale, causal):
    return naive.forward(f["q"], f["k"], f["v"], scale, causal)


@pytest.mark.parametrize("dtype", ["bf16", "f32", "bf16_outf32"])
@pytest.mark.parametrize("d", DIMS)
@pytest.mark.parametrize("Tq,Tk", SHAPES)
@pytest.mark.parametrize("causal", [False, True])
def test_forward_parity(dtype, d, Tq, Tk, causal):
    B, H = 2, 3
    out32 = dtype == "bf16_outf32"
    dtype = "bf16" if out32 else dtype
    dev, f = draw(B, H, Tq, Tk, d, dtype, seed=1000 + Tq + 7 * Tk + d)
    O, lse = fa.forward(dev["q"], dev["k"], dev["v"], causal=causal,
                        out_dtype=torch().float32 if out32 else None)
    if out32:
        assert O.dtype == torch().float32
    torch().cuda.synchronize()
    Or, Lr = _oracle_fwd(f, 1 / math.sqrt(d), causal)
    assert maxabs(to_f64(O), Or) <= TOL_O[dtype]
    assert maxabs(to_f64(lse), Lr) <= TOL_LSE


@pytest.mark.parametrize("dtype,grad", [("bf16", "bf16"), ("bf16", "f32"), ("bf16", "f32o"), ("f32", "f32")])
@pytest.mark.parametrize("d", DIMS)
# 700: an odd number of 256-query dQ blocks and an even number of 128-key blocks; 200: two
# 128-key blocks in one workgroup (causal workgroups take two blocks each; with an odd count
# the middle one runs alone)
@pytest.mark.parametrize("Tq,Tk", [(1, 1), (17, 17), (100, 100), (200, 200), (300, 300), (700, 700), (100, 257),
                                   (257, 100)])
@pytest.mark.parametrize("causal", [False, True])
def test_backward_parity(dtype, grad, d, Tq, Tk, causal):
    t = torch()
    B, H = 2, 2
    dev, f = draw(B, H, Tq, Tk, d, dtype, seed=2000 + Tq + 7 * Tk + d, with_do=True)
    scale = 1 / math.sqrt(d)
    odt = t.float32 if grad == "f32o" else None          # f32o: O kept in float32 between passes
    O, lse = fa.forward(dev["q"], dev["k"], dev["v"], causal=causal, out_dtype=odt)
    gd = t.float32 if grad in ("f32", "f32o") else t.bfloat16
    dQ, dK, dV = fa.backward(dev["q"], dev["k"], dev["v"], O, dev["do"], lse, causal=causal, grad_dtype=gd)
    t.cuda.synchronize()
    rQ, rK, rV, _, _ = naive.backward(f["q"], f["k"], f["v"], f["do"], scale, causal)
    tol = TOL_GRAD[dtype]
    assert maxabs(to_f64(dQ), rQ) <= tol
    assert maxabs(to_f64(dK), rK) <= tol
    assert maxabs(to_f64(dV), rV) <= tol


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_worked_example_in_d64(dtype):
    """[LDD] "Concept": scores [1, 3] in the first key tile, [5] in a later one, scale 1.

    The query is e_0 and key j is s_j e_0, so the score is s_j; keys 2..127 are
    filler at score -100 (weight ~e^-105) so that key 128 (score 5) lies in a
    later key tile for every head width's tile size.  V maps the three scored
    keys to e_0, e_1, e_2 and the filler to e_3, so O holds the weights."""
    d, Tk = 64, 129
    q = np.zeros((1, 1, 1, d), np.float32); q[0, 0, 0, 0] = 1.0
    k = np.zeros((1, 1, Tk, d), np.float32)
    k[0, 0, :, 0] = -100.0
    k[0, 0, 0, 0], k[0, 0, 1, 0], k[0, 0, 128, 0] = 1.0, 3.0, 5.0
    v = np.zeros((1, 1, Tk, d), np.float32); v[0, 0, :, 3] = 1.0
    v[0, 0, 0, :] = 0; v[0, 0, 0, 0] = 1.0
    v[0, 0, 1, :] = 0; v[0, 0, 1, 1] = 1.0
    v[0, 0, 128, :] = 0; v[0, 0, 128, 2] = 1.0
    from io_aware_exact_02_amd.inputs import f32_to_bf16_bits
    conv = (lambda a: f32_to_bf16_bits(a)) if dtype == "bf16" else (lambda a: a)
    O, lse = fa.forward(to_dev(conv(q), dtype), to_dev(conv(k), dtype), to_dev(conv(v), dtype), scale=1.0)
    O, lse = to_f64(O)[0, 0, 0], to_f64(lse)[0, 0, 0]
    assert abs(O[1] - 0.117) <= 5e-4 + TOL_O[dtype]            # the page's true weight on score 3
    assert abs(math.exp(lse - 5.0) - 1.154) <= 5e-4 + TOL_LSE   # the page's final running sum
    Or, Lr = naive.forward_head(q[0, 0].astype(np.float64), k[0, 0].astype(np.float64),
                                v[0, 0].astype(np.float64), 1.0, False)
    assert maxabs(O, Or[0]) <= TOL_O[dtype] and abs(lse - Lr[0]) <= TOL_LSE


@pytest.mark.parametrize("d", DIMS)
def test_constant_v_and_zero_query(d):
    """Constant V gives O = v; Q = 0 gives the prefix mean and lse = ln(#visible)."""
    t = torch()
    B, H, T = 1, 2, 300
    dev, f = draw(B, H, T, T, d, "bf16", seed=3000 + d)
    v_const = dev["v"][:, :, :1, :].expand(B, H, T, d).contiguous()
    O, _ = fa.forward(dev["q"], dev["k"], v_const, causal=True)
    assert maxabs(to_f64(O), to_f64(v_const)) <= TOL_O["bf16"]
    zq = t.zeros_like(dev["q"])
    O, lse = fa.forward(zq, dev["k"], dev["v"], causal=True)
    vf = f["v"]
    prefix = np.cumsum(vf, axis=2) / np.arange(1, T + 1)[None, None, :, None]
    assert maxabs(to_f64(O), prefix) <= TOL_O["bf16"]
    assert maxabs(to_f64(lse), np.log(np.arange(1, T + 1))[None, None, :]) <= TOL_LSE
    O, lse = fa.forward(zq, dev["k"], dev["v"], causal=False)
    assert maxabs(to_f64(lse), math.log(T)) <= TOL_LSE


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("d", DIMS)
@pytest.mark.parametrize("causal", [False, True])
def test_guard_bands_untouched(dtype, d, causal):
    """Outputs written into the middle of NaN-filled buffers leave the margins alone."""
    t = torch()
    B, H, Tq, Tk = 2, 2, 77, 130
    dev, _ = draw(B, H, Tq, Tk, d, dtype, seed=4000, with_do=True)
    tdt = t.bfloat16 if dtype == "bf16" else t.float32
    M = 64

    def framed(n, dt):
        buf = t.full((n + 2 * M,), float("nan"), dtype=dt, device="cuda")
        return buf, buf[M:M + n]

    ob, o = framed(B * H * Tq * d, tdt)
    lb, lse = framed(B * H * Tq, t.float32)
    fa.fa_fwd(dev["q"], dev["k"], dev["v"], o.view(B, H, Tq, d), lse.view(B, H, Tq), causal=causal)
    qb, dq = framed(B * H * Tq * d, tdt)
    kb, dk = framed(B * H * Tk * d, tdt)
    vb, dv = framed(B * H * Tk * d, tdt)
    nb = fa.fa_bwd_workspace_bytes(B, H, Tq, Tk, d, fa._dtype_code(dev["q"]), fa._dtype_code(dq))
    ws = t.empty(nb, dtype=t.uint8, device="cuda")
    fa.fa_bwd(dev["q"], dev["k"], dev["v"], o.view(B, H, Tq, d), dev["do"], lse.view(B, H, Tq),
              dq.view(B, H, Tq, d), dk.view(B, H, Tk, d), dv.view(B, H, Tk, d), ws, causal=causal)
    t.cuda.synchronize()
    for buf, inner in ((ob, o), (lb, lse), (qb, dq), (kb, dk), (vb, dv)):
        assert t.isnan(buf[:M]).all() and t.isnan(buf[-M:]).all()
        assert t.isfinite(inner).all()


@pytest.mark.parametrize("d", DIMS)
def test_forward_bitwise_repeatable(d):
    B, H, T = 2, 4, 1000
    dev, _ = draw(B, H, T, T, d, "bf16", seed=5000)
    O1, L1 = fa.forward(dev["q"], dev["k"], dev["v"], causal=True)
    O2, L2 = fa.forward(dev["q"], dev["k"], dev["v"], causal=True)
    torch().cuda.synchronize()
    assert torch().equal(O1, O2) and torch().equal(L1, L2)


@pytest.mark.parametrize("d", DIMS)
def test_backward_invariants(d):
    """sum_l dV_l = sum_r dO_r and sum_l dK_l = 0 hold for the GPU gradients too."""
    t = torch()
    B, H, T = 1, 2, 257
    dev, f = draw(B, H, T, T, d, "bf16", seed=6000 + d, with_do=True)
    O, lse = fa.forward(dev["q"], dev["k"], dev["v"], causal=True)
    dQ, dK, dV = fa.backward(dev["q"], dev["k"], dev["v"], O, dev["do"], lse, causal=True, grad_dtype=t.float32)
    t.cuda.synchronize()
    assert maxabs(to_f64(dV).sum(axis=2), f["do"].sum(axis=2)) < 5e-2
    assert np.abs(to_f64(dK).sum(axis=2)).max() < 5e-2


@pytest.mark.parametrize("d", [64, 128, 256])
def test_backward_bitwise_repeatable(d):
    """Every gradient is summed in a fixed order (no atomics), for every head width."""
    t = torch()
    B, H, T = 2, 3, 777
    dev, _ = draw(B, H, T, T, d, "bf16", seed=7000 + d, with_do=True)
    O, lse = fa.forward(dev["q"], dev["k"], dev["v"], causal=True)
    g1 = fa.backward(dev["q"], dev["k"], dev["v"], O, dev["do"], lse, causal=True)
    g2 = fa.backward(dev["q"], dev["k"], dev["v"], O, dev["do"], lse, causal=True)
    t.cuda.synchronize()
    for a, b in zip(g1, g2):
        assert t.equal(a, b)
