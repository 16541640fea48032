"""Exact attention by its definition, in float64 on the CPU (the oracle).

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg; never by the HIP library or its binding.

Pages cited (title, then section):
  [Atlas] "FlashAttention -- IO-Aware Exact Attention" (atlas.blal.pro wiki)
  [ZtF]   "FlashAttention", zerotofrontier.app efficient-attention, textbook section 12.3
  [LDD]   "FlashAttention & IO-awareness", llmdeepdive.com lesson 7.7
  [Blog]  hemanths.vercel.app, "attention_training"

FlashAttention reaches the result of standard attention exactly, only the
floating-point order differs ([Atlas] "Online softmax: the trick that makes
tiling exact"; [ZtF] "The forward pass", the paragraph on why the result is
exactly attention).  So the oracle is the plain definition, not the tiled
algorithm:

  forward   S = c Q K^T with c the scale (1/sqrt(d) by default)
            ([ZtF] "The forward pass" step 2.2; [Blog] "Standard Attention:
            What Actually Happens");
            causal: query r sees key l iff l <= r, otherwise S = -inf
            ([ZtF] "The causal mask, and the tiles you never visit"; top-left
            alignment when Tq != Tk); optional block masks and sliding windows
            set further scores to -inf ([ZtF] "Dropout, block-sparsity, and
            other real-kernel details"); a row left without any key has no
            softmax and is given O = 0, lse = -inf;
            P = softmax(S) row-wise with the row maximum subtracted,
            O = P V ([Atlas] "Standard attention, and why it's wasteful");
            lse_r = m_r + ln sum_l exp(S_rl - m_r), natural log of the scaled
            and masked scores ([ZtF] "The forward pass" step 3 and "What the
            forward pass leaves behind"; [Atlas] "Recomputation in the
            backward pass").
  backward  for the loss sum(O * dO) ([ZtF] "The backward pass, derived"):
            dV = P^T dO, dP = dO V^T, D_r = dO_r . O_r (Observation 2),
            dS = P * (dP - D 1^T) (Observation 3), dQ = c dS K, dK = c dS^T Q
            (the scale sits in S = c Q K^T, so it multiplies dQ and dK and not
            dV).  The page's displayed backward equations did not survive
            extraction; this is the textbook chain rule that its prose states
            entry by entry, pinned by finite differences in the tests.

Every function works on one (batch, head) slice with NumPy float64 and library
matmuls; there is no tiling, fusion or reordering beyond the definition.  The
batched wrappers loop over heads (a thread pool only runs independent heads at
the same time).  Inputs that were bf16 on the GPU are widened to float64, which
is exact.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

__all__ = [
    "scores_head", "probs_head", "forward_head", "backward_head",
    "forward", "backward", "block_allowed", "MASK_BLOCK", "dq_rows", "dk_cols", "window_allowed", "doc_allowed",
]

MASK_BLOCK = 128   # side of a block-mask block, in query rows and in keys


def _visible(Tk: int, rows: np.ndarray, causal: bool) -> np.ndarray | None:
    """Boolean [len(rows), Tk]: key l visible to query r.  Causal keeps l <= r
    ([ZtF] "The causal mask, and the tiles you never visit"); None = all."""
    if not causal:
        return None
    return np.arange(Tk)[None, :] <= rows[:, None]


def window_allowed(Tk: int, rows, window) -> np.ndarray:
    """Boolean [len(rows), Tk]: key l inside the sliding window (wl, wr) of query r,
    r - wl <= l <= r + wr, a side of -1 being unbounded.  [ZtF] "Dropout,
    block-sparsity, and other real-kernel details" lists sliding windows among the
    masks that are functions of (r, l); (-1, 0) is the causal mask, (-1, -1) none."""
    wl, wr = window
    rows = np.asarray(rows)
    keys = np.arange(Tk)[None, :]
    ok = np.ones((len(rows), Tk), bool)
    if wl >= 0:
        ok &= keys >= rows[:, None] - wl
    if wr >= 0:
        ok &= keys <= rows[:, None] + wr
    return ok


def doc_allowed(Tk: int, rows, cu_seqlens) -> np.ndarray:
    """Boolean [len(rows), Tk]: query r and key l lie in the same document of a packed
    sequence whose documents start at cu_seqlens[i] and end before cu_seqlens[i + 1]
    (cu_seqlens[0] = 0, last = sequence length).  [ZtF] "Dropout, block-sparsity, and
    other real-kernel details" names document masks among the masks that are
    functions of (r, l); combined with causal, each document is attended causally."""
    cu = np.asarray(cu_seqlens)
    rows = np.asarray(rows)
    doc_r = np.searchsorted(cu, rows, side="right") - 1
    doc_l = np.searchsorted(cu, np.arange(Tk), side="right") - 1
    return doc_r[:, None] == doc_l[None, :]


def block_allowed(Tq: int, Tk: int, block_mask_h, rows=None) -> np.ndarray:
    """Boolean [len(rows), Tk] from a block mask [ceil(Tq/128)][ceil(Tk/128)] of one head.

    [ZtF] "Dropout, block-sparsity, and other real-kernel details": a block mask
    says which (query block, key block) tiles exist; attention restricted to it is
    the dense definition with every score outside the kept blocks set to -inf."""
    bm = np.asarray(block_mask_h) != 0
    rows = np.arange(Tq) if rows is None else np.asarray(rows)
    return bm[rows // MASK_BLOCK][:, np.arange(Tk) // MASK_BLOCK]


def scores_head(q, k, scale, causal, rows=None, block_mask=None, window=None, docs=None):
    """Scaled, masked scores S[rows, :] = c q k^T with -inf where masked (causal, a
    block mask of this head, a sliding window (wl, wr) and/or documents cu_seqlens)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    rows = np.arange(q.shape[0]) if rows is None else np.asarray(rows)
    S = scale * (q[rows] @ k.T)
    vis = _visible(k.shape[0], rows, causal)
    if vis is not None:
        S = np.where(vis, S, -np.inf)
    if block_mask is not None:
        S = np.where(block_allowed(q.shape[0], k.shape[0], block_mask, rows), S, -np.inf)
    if window is not None:
        S = np.where(window_allowed(k.shape[0], rows, window), S, -np.inf)
    if docs is not None:
        S = np.where(doc_allowed(k.shape[0], rows, docs), S, -np.inf)
    return S


def _softmax_rows(S):
    """Row softmax with the row maximum subtracted; also returns lse = m + ln l.

    A row with no visible key (possible only under a block mask) has no softmax;
    it is given zero weights and lse = -inf, so its output and gradients are 0."""
    m = S.max(axis=1)
    empty = ~np.isfinite(m)
    m0 = np.where(empty, 0.0, m)
    E = np.exp(S - m0[:, None])         # exp(-inf) = 0 for masked entries
    l = E.sum(axis=1)
    with np.errstate(divide="ignore", invalid="ignore"):
        P = np.where(empty[:, None], 0.0, E / np.where(empty, 1.0, l)[:, None])
        lse = np.where(empty, -np.inf, m0 + np.log(np.where(empty, 1.0, l)))
    return P, lse


def probs_head(q, k, scale, causal, rows=None, block_mask=None, window=None, docs=None):
    """P[rows, :] = softmax(S) and lse[rows] for one head."""
    return _softmax_rows(scores_head(q, k, scale, causal, rows, block_mask, window, docs))


def forward_head(q, k, v, scale, causal, rows=None, block_mask=None, window=None, docs=None):
    """O[rows] = softmax(c q k^T) v and lse[rows] for one head.

    q [Tq, d], k [Tk, d], v [Tk, dv].  Each output row depends only on its own
    query and all keys, so a subset `rows` is computed exactly by the same
    definition (used where the full T x T matrix would not fit in memory).
    """
    P, lse = probs_head(q, k, scale, causal, rows, block_mask, window, docs)
    return P @ np.asarray(v, dtype=np.float64), lse


def backward_head(q, k, v, do, scale, causal, block_mask=None, window=None, docs=None):
    """Gradients of sum(O * dO) for one head: returns dQ, dK, dV, O, lse, D."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    P, lse = probs_head(q, k, scale, causal, block_mask=block_mask, window=window, docs=docs)
    O = P @ v
    dV = P.T @ do
    dP = do @ v.T
    D = np.sum(do * O, axis=1)
    dS = P * (dP - D[:, None])
    dQ = scale * (dS @ k)
    dK = scale * (dS.T @ q)
    return dQ, dK, dV, O, lse, D


def dq_rows(q, k, v, do, scale, causal, rows, block_mask=None, window=None, docs=None):
    """dQ[rows] of one head by the same chain rule ([ZtF] "The backward pass,
    derived"): row r of dQ = c dS_r K needs only row r of P, of dP = dO V^T and
    D_r = dO_r . O_r, so sampled rows are exact without the T x T matrices."""
    rows = np.asarray(rows)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do_r = np.asarray(do, dtype=np.float64)[rows]
    P, _ = probs_head(q, k, scale, causal, rows, block_mask, window, docs)
    O = P @ v
    D = np.sum(do_r * O, axis=1)
    dS = P * (do_r @ v.T - D[:, None])
    return scale * (dS @ k)


def dk_cols(q, k, v, do, scale, causal, cols, block_mask=None, window=None, docs=None, row_block=1024):
    """dK[cols] of one head by the same chain rule ([ZtF] "The backward pass,
    derived"): column l of dK = c dS[:, l]^T Q needs column l of P and of
    dP = dO V^T for every query row, and D_r = dO_r . O_r, so it needs O and lse
    of every row that sees key l.  They come from the definition row block by
    row block (no T x T matrix is held), then only the sampled columns of P and
    dP are formed.  Under the causal rule a row r sees key l only when l <= r,
    so rows before the first sampled key add nothing and are not visited."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    cols = np.asarray(cols)
    out = np.zeros((len(cols), q.shape[1]))
    first = int(cols.min()) if causal and len(cols) else 0
    for r0 in range(first, q.shape[0], row_block):
        rows = np.arange(r0, min(r0 + row_block, q.shape[0]))
        P, _ = probs_head(q, k, scale, causal, rows, block_mask, window, docs)    # P[rows, :]
        O = P @ v
        D = np.sum(do[rows] * O, axis=1)
        Pc = P[:, cols]
        dS = Pc * (do[rows] @ v[cols].T - D[:, None])
        out += scale * (dS.T @ q[rows])
    return out


def _heads(B, H, heads):
    return [(b, h) for b in range(B) for h in range(H)] if heads is None else list(heads)


def _pool(workers):
    n = workers or os.cpu_count() or 1
    return ThreadPoolExecutor(max_workers=max(1, n)), n


def _one_blas_thread():
    """Context limiting BLAS to one thread per worker when threadpoolctl exists."""
    try:
        from threadpoolctl import threadpool_limits
        return threadpool_limits(limits=1)
    except Exception:  # pragma: no cover - threadpoolctl is optional
        import contextlib
        return contextlib.nullcontext()


def _head_mask(block_mask, h):
    """The block mask of head h from [Hm][nqb][nkb] (Hm = 1 is shared by all heads)."""
    if block_mask is None:
        return None
    bm = np.asarray(block_mask)
    return bm[0] if bm.shape[0] == 1 else bm[h]


def forward(Q, K, V, scale, causal, heads=None, rows=None, workers=None, block_mask=None, window=None,
            docs=None):
    """Batched forward over [B, H, T, d] arrays.

    heads: optional list of (b, h) pairs to compute (others are left NaN);
    rows: optional query-row subset applied to every selected head;
    block_mask: optional uint8 [Hm][ceil(Tq/128)][ceil(Tk/128)], Hm in {1, H};
    window: optional sliding window (wl, wr), see window_allowed;
    docs: optional document offsets cu_seqlens, see doc_allowed.
    Returns O [B, H, n_rows, d] and lse [B, H, n_rows] in float64.
    """
    B, H, Tq, _ = Q.shape
    n = Tq if rows is None else len(rows)
    O = np.full((B, H, n, V.shape[3]), np.nan)
    L = np.full((B, H, n), np.nan)
    todo = _heads(B, H, heads)

    def run(bh):
        b, h = bh
        O[b, h], L[b, h] = forward_head(Q[b, h], K[b, h], V[b, h], scale, causal, rows,
                                        _head_mask(block_mask, h), window, docs)

    ex, nw = _pool(workers)
    with _one_blas_thread() if nw > 1 else _nullctx(), ex:
        list(ex.map(run, todo))
    return O, L


def backward(Q, K, V, dO, scale, causal, heads=None, workers=None, block_mask=None, window=None, docs=None):
    """Batched backward over [B, H, T, d] arrays; returns dQ, dK, dV, O, lse."""
    B, H, Tq, d = Q.shape
    Tk = K.shape[2]
    dQ = np.full((B, H, Tq, d), np.nan)
    dK = np.full((B, H, Tk, d), np.nan)
    dV = np.full((B, H, Tk, V.shape[3]), np.nan)
    O = np.full((B, H, Tq, V.shape[3]), np.nan)
    L = np.full((B, H, Tq), np.nan)
    todo = _heads(B, H, heads)

    def run(bh):
        b, h = bh
        dQ[b, h], dK[b, h], dV[b, h], O[b, h], L[b, h], _ = backward_head(
            Q[b, h], K[b, h], V[b, h], dO[b, h], scale, causal, _head_mask(block_mask, h), window, docs)

    ex, nw = _pool(workers)
    with _one_blas_thread() if nw > 1 else _nullctx(), ex:
        list(ex.map(run, todo))
    return dQ, dK, dV, O, L


def _nullctx():
    import contextlib
    return contextlib.nullcontext()
