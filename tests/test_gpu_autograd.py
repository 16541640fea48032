"""The autograd wrapper ([ZtF] "In PyTorch") against the float64 oracle and against
torch's own scaled-dot-product attention run in float64 on the CPU with autograd, on
the same bf16/fp32 input values: output and the three gradients of a seeded random
cotangent; and torch.autograd.gradcheck of the float32 path."""
import math

import numpy as np
import pytest

from oracle import naive
from tests.gpu_util import TOL_GRAD, TOL_O, draw, maxabs, to_f64, torch

pytestmark = pytest.mark.gpu


def _reference(f, causal, scale):
    t = torch()
    q, k, v = (t.tensor(f[n], dtype=t.float64, requires_grad=True) for n in ("q", "k", "v"))
    out = t.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=causal, scale=scale)
    out.backward(t.tensor(f["do"], dtype=t.float64))
    return out.detach().numpy(), q.grad.numpy(), k.grad.numpy(), v.grad.numpy()


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("Tq,Tk", [(200, 200), (77, 300), (300, 77)])
def test_attention_autograd_matches_oracle_and_cpu_sdpa(dtype, d, causal, Tq, Tk):
    """Causal with Tq != Tk included: the oracle pins tie torch's is_causal to the
    library's top-left alignment (key l visible from query r iff l <= r)."""
    import io_aware_exact_02_amd.autograd as faa
    t = torch()
    B, H = 2, 2
    dev, f = draw(B, H, Tq, Tk, d, dtype, seed=8000 + d + Tq + 3 * Tk, with_do=True)
    q, k, v = (dev[n].clone().requires_grad_(True) for n in ("q", "k", "v"))
    out = faa.attention(q, k, v, causal=causal)
    out.backward(dev["do"])
    t.cuda.synchronize()
    scale = 1 / math.sqrt(d)
    oQ, oK, oV, oO, _ = naive.backward(f["q"], f["k"], f["v"], f["do"], scale, causal)
    rO, rQ, rK, rV = _reference(f, causal, scale)
    assert maxabs(to_f64(out.detach()), oO) <= TOL_O[dtype]
    assert maxabs(to_f64(out.detach()), rO) <= TOL_O[dtype]
    tol = TOL_GRAD[dtype]
    for got, oref, tref in ((q.grad, oQ, rQ), (k.grad, oK, rK), (v.grad, oV, rV)):
        assert got.dtype == q.dtype
        assert maxabs(to_f64(got), oref) <= tol
        assert maxabs(to_f64(got), tref) <= tol


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("Tq,Tk", [(13, 13), (7, 19), (19, 7)])
def test_attention_gradcheck_f32(causal, Tq, Tk):
    """torch.autograd.gradcheck of the float32 path ([ZtF] "In PyTorch" pairs the
    wrapper with gradcheck): the wrapper's Jacobian-vector products against central
    differences with step eps = 1e-3 in float32.  The kernels are exact to about
    1e-6 here, and a central difference in float32 carries about 1e-7 |O| / eps of
    rounding plus eps^2 of truncation, so atol = rtol = 2e-3 leaves a margin of
    more than ten."""
    import io_aware_exact_02_amd.autograd as faa
    t = torch()
    g = t.Generator(device="cuda").manual_seed(8300 + Tq + Tk + causal)
    q, k, v = (t.randn(1, 2, T, 64, device="cuda", generator=g, dtype=t.float32).requires_grad_(True)
               for T in (Tq, Tk, Tk))
    fn = lambda a, b, c: faa.attention(a, b, c, causal=causal)
    assert t.autograd.gradcheck(fn, (q, k, v), eps=1e-3, atol=2e-3, rtol=2e-3, fast_mode=True)


def test_attention_autograd_respects_scale_and_second_use():
    """A non-default scale reaches both passes; the graph can be reused after a fresh forward."""
    import io_aware_exact_02_amd.autograd as faa
    t = torch()
    B, H, T, d = 1, 3, 150, 64
    dev, f = draw(B, H, T, T, d, "bf16", seed=8100, with_do=True)
    scale = 0.3
    for _ in range(2):
        q, k, v = (dev[n].clone().requires_grad_(True) for n in ("q", "k", "v"))
        out = faa.attention(q, k, v, causal=True, scale=scale)
        out.backward(dev["do"])
        t.cuda.synchronize()
        rO, rQ, rK, rV = _reference(f, True, scale)
        oQ, oK, oV, oO, _ = naive.backward(f["q"], f["k"], f["v"], f["do"], scale, True)
        assert maxabs(to_f64(out.detach()), rO) <= TOL_O["bf16"]
        assert maxabs(to_f64(out.detach()), oO) <= TOL_O["bf16"]
        assert np.isfinite(to_f64(q.grad)).all()
        for got, ref, oref in ((q.grad, rQ, oQ), (k.grad, rK, oK), (v.grad, rV, oV)):
            assert maxabs(to_f64(got), ref) <= TOL_GRAD["bf16"]
            assert maxabs(to_f64(got), oref) <= TOL_GRAD["bf16"]


def test_attention_autograd_with_block_mask_matches_direct_calls():
    """With a block mask the wrapper runs the block-sparse kernels: same bits as calling
    fa_fwd_masked / fa_bwd_masked directly."""
    import io_aware_exact_02_amd as fa
    import io_aware_exact_02_amd.autograd as faa
    from io_aware_exact_02_amd import inputs as I
    t = torch()
    B, H, T, d = 2, 2, 700, 128
    dev, f = draw(B, H, T, T, d, "bf16", seed=8200, with_do=True)
    bm = I.block_mask(H, T, T, 0.5, 8201, keep_diagonal=True)
    mt = t.from_numpy(bm).cuda()
    q, k, v = (dev[n].clone().requires_grad_(True) for n in ("q", "k", "v"))
    out = faa.attention(q, k, v, causal=True, block_mask=mt)
    out.backward(dev["do"])
    O, lse = fa.forward_masked(dev["q"], dev["k"], dev["v"], mt, causal=True)
    dQ, dK, dV = fa.backward_masked(dev["q"], dev["k"], dev["v"], O, dev["do"], lse, mt, causal=True)
    t.cuda.synchronize()
    assert t.equal(out.detach(), O)
    for got, ref in ((q.grad, dQ), (k.grad, dK), (v.grad, dV)):
        assert t.equal(got, ref)
    # and against the oracle on the restricted problem (block mask R18 tolerance: the
    # gradients of rows that keep few keys grow, and so does their bf16 rounding)
    oQ, oK, oV, oO, _ = naive.backward(f["q"], f["k"], f["v"], f["do"], 1 / math.sqrt(d), True, block_mask=bm)
    assert maxabs(to_f64(out.detach()), oO) <= TOL_O["bf16"]
    for got, oref in ((q.grad, oQ), (k.grad, oK), (v.grad, oV)):
        assert maxabs(to_f64(got), oref) <= TOL_GRAD["bf16"] * max(1.0, float(np.abs(oref).max()))
