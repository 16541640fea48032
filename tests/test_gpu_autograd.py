"""The autograd wrapper ([ZtF] "In PyTorch") against torch's own scaled-dot-product
attention run in float64 on the CPU with autograd, on the same bf16/fp32 input values:
output and the three gradients of a seeded random cotangent."""
import math

import numpy as np
import pytest

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
@pytest.mark.parametrize("Tq,Tk", [(200, 200), (77, 300)])
def test_attention_autograd_matches_cpu_sdpa(dtype, d, causal, Tq, Tk):
    import io_aware_exact_02_amd.autograd as faa
    t = torch()
    if causal and Tq != Tk:
        pytest.skip("torch's is_causal with Tq != Tk is checked in the oracle pins")
    B, H = 2, 2
    dev, f = draw(B, H, Tq, Tk, d, dtype, seed=8000 + d + Tq, with_do=True)
    q, k, v = (dev[n].clone().requires_grad_(True) for n in ("q", "k", "v"))
    out = faa.attention(q, k, v, causal=causal)
    out.backward(dev["do"])
    t.cuda.synchronize()
    rO, rQ, rK, rV = _reference(f, causal, 1 / math.sqrt(d))
    assert maxabs(to_f64(out.detach()), rO) <= TOL_O[dtype]
    tol = TOL_GRAD[dtype]
    for got, ref in ((q.grad, rQ), (k.grad, rK), (v.grad, rV)):
        assert got.dtype == q.dtype
        assert maxabs(to_f64(got), ref) <= tol


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
        assert maxabs(to_f64(out.detach()), rO) <= TOL_O["bf16"]
        assert np.isfinite(to_f64(q.grad)).all()
        for got, ref in ((q.grad, rQ), (k.grad, rK), (v.grad, rV)):
            assert maxabs(to_f64(got), ref) <= TOL_GRAD["bf16"]


def test_attention_autograd_with_block_mask_matches_direct_calls():
    """With a block mask the wrapper runs the block-sparse kernels: same bits as calling
    fa_fwd_masked / fa_bwd_masked directly."""
    import io_aware_exact_02_amd as fa
    import io_aware_exact_02_amd.autograd as faa
    from io_aware_exact_02_amd import inputs as I
    t = torch()
    B, H, T, d = 2, 2, 700, 128
    dev, _ = draw(B, H, T, T, d, "bf16", seed=8200, with_do=True)
    mt = t.from_numpy(I.block_mask(H, T, T, 0.5, 8201, keep_diagonal=True)).cuda()
    q, k, v = (dev[n].clone().requires_grad_(True) for n in ("q", "k", "v"))
    out = faa.attention(q, k, v, causal=True, block_mask=mt)
    out.backward(dev["do"])
    O, lse = fa.forward_masked(dev["q"], dev["k"], dev["v"], mt, causal=True)
    dQ, dK, dV = fa.backward_masked(dev["q"], dev["k"], dev["v"], O, dev["do"], lse, mt, causal=True)
    t.cuda.synchronize()
    assert t.equal(out.detach(), O)
    for got, ref in ((q.grad, dQ), (k.grad, dK), (v.grad, dV)):
        assert t.equal(got, ref)
