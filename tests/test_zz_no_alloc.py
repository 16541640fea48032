"""fa_bwd_noalloc (the backward pass with the library's fixed scratch as its
workspace) against fa_bwd with a caller workspace, called through the C ABI:
two calls in a row on one GPU, the second on a smaller problem, each bit for bit
equal to fa_bwd (both run the same kernels in the same order), and fa_bwd_noalloc
leaves no allocation behind it."""
import math

import pytest

import io_aware_exact_02_amd as fa
from tests.gpu_util import draw, torch

pytestmark = pytest.mark.gpu


def _case(B, H, T, d, causal, grad_f32, seed):
    t = torch()
    dev, _ = draw(B, H, T, T, d, "bf16", seed=seed, with_do=True)
    q, k, v, do = dev["q"], dev["k"], dev["v"], dev["do"]
    O, lse = fa.forward(q, k, v, causal=causal)
    gdt = t.float32 if grad_f32 else t.bfloat16
    ref = fa.backward(q, k, v, O, do, lse, causal=causal, grad_dtype=gdt)
    t.cuda.synchronize()
    out = [t.full_like(r, float("nan")) for r in ref]
    lib = fa.library()
    stream = t.cuda.current_stream()
    before = t.cuda.memory_allocated()
    st = lib.fa_bwd_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), O.data_ptr(), do.data_ptr(), lse.data_ptr(),
                            out[0].data_ptr(), out[1].data_ptr(), out[2].data_ptr(), B, H, T, T, d,
                            1.0 / math.sqrt(d), int(causal), fa.FA_BF16, fa.FA_BF16,
                            fa.FA_F32 if grad_f32 else fa.FA_BF16, stream.cuda_stream)
    assert st == 0, fa.fa_strerror(st)
    t.cuda.synchronize()
    assert t.cuda.memory_allocated() == before
    for name, got, want in zip(("dQ", "dK", "dV"), out, ref):
        assert t.equal(got, want), name


def test_noalloc_matches_fa_bwd_twice_second_smaller():
    print("[noalloc] B=2 H=4 T=1000 d=128 causal, then B=1 H=2 T=300 d=64 non-causal", flush=True)
    _case(2, 4, 1000, 128, True, False, seed=9901)
    _case(1, 2, 300, 64, False, True, seed=9902)
