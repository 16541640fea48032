"""Split-key forward (few query rows per head) against the float64 oracle: the
output and lse of the merged partials, for several chunk counts, ragged key
counts, both head widths it supports and both masks; plus bitwise repeatability
and the full-size decoding workload on sampled heads."""
import math

import numpy as np
import pytest

import io_aware_exact_02_amd as fa
from oracle import naive
from tests.gpu_util import TOL_LSE, TOL_O, draw, maxabs, to_f64, torch

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("Tq,Tk", [(1, 1), (1, 31), (1, 100), (4, 4097), (33, 700), (1, 5000)])
@pytest.mark.parametrize("nsplit", [0, 1, 3, 7])
@pytest.mark.parametrize("causal", [False, True])
def test_splitkv_parity(d, Tq, Tk, nsplit, causal):
    B, H = 2, 3
    dev, f = draw(B, H, Tq, Tk, d, "bf16", seed=9000 + Tq + 3 * Tk + d + nsplit)
    O, lse = fa.forward_splitkv(dev["q"], dev["k"], dev["v"], causal=causal, nsplit=nsplit)
    torch().cuda.synchronize()
    Or, Lr = naive.forward(f["q"], f["k"], f["v"], 1 / math.sqrt(d), causal)
    assert maxabs(to_f64(O), Or) <= TOL_O["bf16"]
    assert maxabs(to_f64(lse), Lr) <= TOL_LSE


def test_splitkv_large_logits_and_f32_output():
    """Q, K ~ N(0, 9): peaked rows whose maximum moves between chunks."""
    t = torch()
    B, H, Tq, Tk, d = 2, 2, 3, 3000, 128
    dev, f = draw(B, H, Tq, Tk, d, "bf16", seed=9500, qk_spread=3.0)
    O, lse = fa.forward_splitkv(dev["q"], dev["k"], dev["v"], out_dtype=t.float32, nsplit=5)
    t.cuda.synchronize()
    assert O.dtype == t.float32
    Or, Lr = naive.forward(f["q"], f["k"], f["v"], 1 / math.sqrt(d), False)
    assert maxabs(to_f64(O), Or) <= TOL_O["bf16"]
    assert maxabs(to_f64(lse), Lr) <= TOL_LSE


def test_splitkv_bitwise_repeatable_and_matches_forward():
    t = torch()
    B, H, Tq, Tk, d = 2, 4, 2, 4000, 128
    dev, _ = draw(B, H, Tq, Tk, d, "bf16", seed=9600)
    O1, L1 = fa.forward_splitkv(dev["q"], dev["k"], dev["v"])
    O2, L2 = fa.forward_splitkv(dev["q"], dev["k"], dev["v"])
    O3, L3 = fa.forward(dev["q"], dev["k"], dev["v"])
    t.cuda.synchronize()
    assert t.equal(O1, O2) and t.equal(L1, L2)
    assert maxabs(to_f64(O1), to_f64(O3)) <= TOL_O["bf16"]
    assert maxabs(to_f64(L1), to_f64(L3)) <= TOL_LSE


def test_decode_workload_sampled_heads():
    """B=8 H=16, one query row against 32768 keys, d=128 (the benchmark's decoding case);
    float64 values are formed for the sampled heads only."""
    from io_aware_exact_02_amd import inputs as I
    from tests.gpu_util import to_dev
    w = I.WORKLOADS["decode_bf16_b8h16_tq1_tk32768_d128"]
    raw = I.draw(w.B, w.H, w.Tq, w.Tk, w.d, w.dtype, w.seed)
    dev = {k: to_dev(v, w.dtype) for k, v in raw.items()}
    O, lse = fa.forward_splitkv(dev["q"], dev["k"], dev["v"], causal=w.causal)
    torch().cuda.synchronize()
    rng = np.random.default_rng(7)
    heads = {(0, 0), (w.B - 1, w.H - 1)} | {(int(rng.integers(w.B)), int(rng.integers(w.H))) for _ in range(4)}
    scale = 1 / math.sqrt(w.d)
    for b, h in sorted(heads):
        q, k, v = (I.as_f64(raw[n][b, h], w.dtype) for n in ("q", "k", "v"))
        Or, Lr = naive.forward_head(q, k, v, scale, w.causal)
        assert maxabs(to_f64(O[b, h]), Or) <= TOL_O[w.dtype], (b, h)
        assert maxabs(to_f64(lse[b, h]), Lr) <= TOL_LSE, (b, h)
