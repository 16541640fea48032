"""Seeded synthetic inputs shared by the tests, the benchmark and the smoke check.

This module holds no part of the attention arithmetic: it only draws numbers and
rounds them to the storage type, so both the HIP path and the oracle can be fed
the very same values.

Recipe: NumPy PCG64 `default_rng(seed)`; float32 standard normals drawn in the
order Q, K, V, dO, each over its whole [B, H, T, d] shape; Q and K optionally
multiplied by a spread (3 for the large-logit cross-attention workload); bf16
tensors are the float32 draws rounded to nearest-even, and the oracle widens
exactly those bf16 values to float64.

Block masks (block-sparse attention): uint8 [heads][ceil(Tq/128)][ceil(Tk/128)]
drawn as Bernoulli(density) per block from `default_rng(seed)` in row-major
order (uniform draws < density), after which the listed forced blocks are set:
the diagonal (i, i) when `keep_diagonal`, so that every query block sees at
least one key block, and the rows in `empty_rows` cleared.

Documents (packed sequences): offsets int32 [ndocs + 1] from `default_rng(seed)`,
each document's length exp(U(ln lo, ln hi)) rounded to the nearest integer, laid
end to end from 0 until they reach T, the last one cut at T.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

BASE_SEED = 20261201


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); returns uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounded = u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    out = (rounded >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = 0x7FC0
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns to float32 (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    Tq: int
    Tk: int
    d: int
    dtype: str          # "f32" or "bf16"
    causal: bool
    backward: bool      # the workload includes the backward pass
    qk_spread: float = 1.0
    seed: int = BASE_SEED
    mask_density: float | None = None   # block-sparse: fraction of kept 128 x 128 blocks (one mask per head)
    window: tuple | None = None         # sliding window (wl, wr): keys r - wl .. r + wr of query r
    doc_len: tuple | None = None        # packed documents: lengths log-uniform in [lo, hi]

    def flops_fwd(self) -> float:
        """4 B H Tq Tk d, halved when causal (square causal: visible pairs ~ T^2 / 2)."""
        f = 4.0 * self.B * self.H * self.Tq * self.Tk * self.d
        return f / 2 if self.causal else f

    def flops_bwd(self) -> float:
        """Five tile products against the forward's two: 2.5 x forward."""
        return 2.5 * self.flops_fwd()


WORKLOADS = {
    "fwd_f32_b1h1_t256_d64": Workload("fwd_f32_b1h1_t256_d64", 1, 1, 256, 256, 64, "f32", False, False,
                                      seed=BASE_SEED + 1),
    "causal_bf16_b8h32_t4096_d128": Workload("causal_bf16_b8h32_t4096_d128", 8, 32, 4096, 4096, 128, "bf16",
                                             True, False, seed=BASE_SEED + 2),
    "causal_bf16_b4h16_t16384_d64": Workload("causal_bf16_b4h16_t16384_d64", 4, 16, 16384, 16384, 64, "bf16",
                                             True, True, seed=BASE_SEED + 3),
    "causal_bf16_b1h24_t65536_d256": Workload("causal_bf16_b1h24_t65536_d256", 1, 24, 65536, 65536, 256, "bf16",
                                              True, False, seed=BASE_SEED + 4),
    "cross_bf16_b16h16_tq1024_tk8192_d128": Workload("cross_bf16_b16h16_tq1024_tk8192_d128", 16, 16, 1024, 8192,
                                                     128, "bf16", False, True, qk_spread=3.0,
                                                     seed=BASE_SEED + 5),
    # block-sparse: a quarter of the 128 x 128 blocks of each head kept, diagonal always kept
    "blocksparse_bf16_b8h32_t4096_d128_s25": Workload("blocksparse_bf16_b8h32_t4096_d128_s25", 8, 32, 4096, 4096,
                                                      128, "bf16", False, True, seed=BASE_SEED + 7,
                                                      mask_density=0.25),
    # sliding window: 4096 keys up to and including the query's own (window (4095, 0))
    "swa_bf16_b1h32_t32768_d128_w4096": Workload("swa_bf16_b1h32_t32768_d128_w4096", 1, 32, 32768, 32768, 128,
                                                 "bf16", False, True, seed=BASE_SEED + 8, window=(4095, 0)),
    # packed documents: 32768 tokens of documents 64 .. 8192 long, causal within each
    "docs_bf16_b1h32_t32768_d128": Workload("docs_bf16_b1h32_t32768_d128", 1, 32, 32768, 32768, 128, "bf16",
                                            True, True, seed=BASE_SEED + 9, doc_len=(64, 8192)),
    # decoding: one query row per head against a long key cache (split-key forward)
    "decode_bf16_b8h16_tq1_tk32768_d128": Workload("decode_bf16_b8h16_tq1_tk32768_d128", 8, 16, 1, 32768, 128,
                                                   "bf16", False, False, seed=BASE_SEED + 6),
}


def draw(B, H, Tq, Tk, d, dtype, seed, qk_spread=1.0, with_do=False):
    """Draw Q, K, V (and dO) as NumPy arrays.

    bf16: uint16 bit patterns; f32: float32.  Returns a dict with keys
    'q', 'k', 'v' (and 'do').
    """
    rng = np.random.default_rng(seed)
    shapes = [("q", (B, H, Tq, d)), ("k", (B, H, Tk, d)), ("v", (B, H, Tk, d))]
    if with_do:
        shapes.append(("do", (B, H, Tq, d)))
    out = {}
    for name, shp in shapes:
        x = rng.standard_normal(shp, dtype=np.float32)
        if name in ("q", "k") and qk_spread != 1.0:
            x *= np.float32(qk_spread)
        out[name] = f32_to_bf16_bits(x) if dtype == "bf16" else x
    return out


def draw_workload(w: Workload, with_do=None):
    return draw(w.B, w.H, w.Tq, w.Tk, w.d, w.dtype, w.seed, w.qk_spread,
                w.backward if with_do is None else with_do)


def as_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """The exact float64 values of a drawn array (bf16 bits or float32)."""
    return bf16_bits_to_f32(a).astype(np.float64) if dtype == "bf16" else np.asarray(a, np.float64)


def block_mask(heads, Tq, Tk, density, seed, keep_diagonal=True, empty_rows=()):
    """A seeded block mask uint8 [heads][ceil(Tq/128)][ceil(Tk/128)] (recipe above)."""
    nq, nk = -(-Tq // 128), -(-Tk // 128)
    rng = np.random.default_rng(seed)
    m = (rng.random((heads, nq, nk)) < density).astype(np.uint8)
    if keep_diagonal:
        i = np.arange(min(nq, nk))
        m[:, i, i] = 1
    for r in empty_rows:
        m[:, r, :] = 0
    return m


def workload_mask(w: Workload, density=None):
    """The block mask of a block-sparse workload: one per head, seeded from the workload
    (`density` overrides the workload's own, for sweeps)."""
    return block_mask(w.H, w.Tq, w.Tk, w.mask_density if density is None else density, w.seed + 1000)


def doc_offsets(T, lo, hi, seed):
    """Seeded document offsets int32 [ndocs + 1] covering 0 .. T (recipe above)."""
    rng = np.random.default_rng(seed)
    cu = [0]
    while cu[-1] < T:
        n = int(np.rint(np.exp(rng.uniform(np.log(lo), np.log(hi)))))
        cu.append(min(T, cu[-1] + max(1, n)))
    return np.asarray(cu, dtype=np.int32)


def workload_docs(w: Workload):
    """The document offsets of a packed-document workload, seeded from the workload."""
    return doc_offsets(w.Tq, w.doc_len[0], w.doc_len[1], w.seed + 2000)
