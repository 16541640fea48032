"""CPU model of tiled FlashAttention with an HBM-traffic counter (a test aid).

TEST INFRASTRUCTURE ONLY: imported by the tests; shares no code with the HIP
library.  It is not the oracle -- it is checked against `oracle.naive`.

Pages cited: [ZtF] "FlashAttention" (zerotofrontier.app, textbook section 12.3),
[LDD] "FlashAttention & IO-awareness" (llmdeepdive.com lesson 7.7), [Blog]
hemanths.vercel.app "attention_training".

What it models, in the pages' order and notation, one head at a time in float64:

* `fa2_forward`: [ZtF] "The forward pass": query block Q_i outside, key blocks
  inside; running m (init -inf), l (init 0), O~ (init 0); per tile
  S_ij = c Q_i K_j^T, m_new = max(m, rowmax S_ij), P~ = exp(S_ij - m_new),
  l <- e^{m - m_new} l + rowsum P~, O~ <- diag(e^{m - m_new}) O~ + P~ V_j;
  finally O_i = diag(l)^-1 O~ and lse_i = m + log l.  Causal tiles are
  classified as in [ZtF] "The causal mask, and the tiles you never visit":
  skipped when the first key of the block is after the last query of the
  block, masked on the diagonal, unmasked below it.
* `fa1_forward`: the original loop order used in the proof of [ZtF] "The IO
  complexity theorem": key/value blocks outside; every sweep re-reads Q_i,
  O_i, l_i, m_i and writes O_i, l_i, m_i back.
* `fa2_backward`: [ZtF] "The backward pass, derived" and "Which loop goes
  outside?": D = rowsum(dO * O) in one pre-pass, key blocks outside with dK_j
  and dV_j accumulated on chip and written once, dQ_i updated in HBM by a
  read-add-write per tile.
* `standard_forward`: the materialising algorithm whose traffic [Blog]
  "Standard Attention" / "The Real Bottleneck" counts: S and P written to and
  read back from HBM.

The counter counts values (not bytes) crossing HBM<->SRAM, as the pages do.
Where masked entries meet a fully masked running row, exp(-inf - (-inf)) is
taken as 0 by using 0 as the reference maximum (the pages are silent; with
top-left causal alignment and j visited in increasing order this never fires
for square blocks, but Br != Bc can create such rows inside a diagonal tile).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

__all__ = [
    "Counter", "fa2_forward", "fa1_forward", "fa2_backward", "standard_forward",
    "standard_traffic", "fa2_forward_traffic", "fa1_forward_traffic", "block_sizes",
    "skip_tile", "visited_tiles",
]


@dataclass
class Counter:
    """Values read from / written to HBM and tiles visited."""
    reads: int = 0
    writes: int = 0
    tiles: int = 0
    log: list = field(default_factory=list)

    @property
    def total(self) -> int:
        return self.reads + self.writes


def skip_tile(i: int, j: int, Br: int, Bc: int, Tq: int) -> bool:
    """Causal skip test: skip iff the block's first key comes after its last
    query ([ZtF] "The causal mask, and the tiles you never visit")."""
    first_key = j * Bc
    last_query = min((i + 1) * Br, Tq) - 1
    return first_key > last_query


def visited_tiles(Tq: int, Tk: int, Br: int, Bc: int, causal: bool) -> int:
    n_r, n_c = math.ceil(Tq / Br), math.ceil(Tk / Bc)
    if not causal:
        return n_r * n_c
    return sum(1 for i in range(n_r) for j in range(n_c) if not skip_tile(i, j, Br, Bc, Tq))


def _mask_tile(S, r0, l0, causal):
    if not causal:
        return S
    rows = np.arange(r0, r0 + S.shape[0])[:, None]
    cols = np.arange(l0, l0 + S.shape[1])[None, :]
    return np.where(cols <= rows, S, -np.inf)


def fa2_forward(Q, K, V, Br, Bc, causal=False, scale=None, counter=None, trace=None):
    """Tiled forward in FlashAttention-2 order.  Returns O, lse.

    trace, if given, is called as trace(i, j, m, l) after every visited tile.
    """
    Q = np.asarray(Q, np.float64); K = np.asarray(K, np.float64); V = np.asarray(V, np.float64)
    Tq, d = Q.shape
    Tk, dv = V.shape
    c = 1.0 / math.sqrt(d) if scale is None else scale
    cnt = counter if counter is not None else Counter()
    n_r, n_c = math.ceil(Tq / Br), math.ceil(Tk / Bc)
    O = np.zeros((Tq, dv)); lse = np.zeros(Tq)
    for i in range(n_r):
        r0, r1 = i * Br, min((i + 1) * Br, Tq)
        Qi = Q[r0:r1]; cnt.reads += Qi.size                       # step 1: load Q_i
        m = np.full(r1 - r0, -np.inf); l = np.zeros(r1 - r0); Ot = np.zeros((r1 - r0, dv))
        for j in range(n_c):
            if causal and skip_tile(i, j, Br, Bc, Tq):
                continue                                         # above the diagonal
            l0, l1 = j * Bc, min((j + 1) * Bc, Tk)
            Kj, Vj = K[l0:l1], V[l0:l1]; cnt.reads += Kj.size + Vj.size   # step 2.1
            cnt.tiles += 1
            S = _mask_tile(c * (Qi @ Kj.T), r0, l0, causal)        # step 2.2
            m_new = np.maximum(m, S.max(axis=1))                   # step 2.3
            ref = np.where(np.isneginf(m_new), 0.0, m_new)
            Pt = np.exp(S - ref[:, None])                          # step 2.4
            alpha = np.exp(m - ref)                                # e^{m - m_new}
            l = alpha * l + Pt.sum(axis=1)                         # step 2.5
            Ot = alpha[:, None] * Ot + Pt @ Vj
            m = m_new
            if trace is not None:
                trace(i, j, m.copy(), l.copy())
        O[r0:r1] = Ot / l[:, None]                                 # step 3
        lse[r0:r1] = m + np.log(l)
        cnt.writes += (r1 - r0) * dv + (r1 - r0)
    return O, lse


def fa1_forward(Q, K, V, Br, Bc, causal=False, scale=None, counter=None):
    """Tiled forward in the original (key/value blocks outside) order.

    Running O_i, l_i, m_i live in HBM between sweeps, so each inner step reads
    Q_i, O_i, l_i, m_i and writes O_i, l_i, m_i ([ZtF] "The IO complexity
    theorem", the counting paragraph).  O is kept normalised between sweeps.
    """
    Q = np.asarray(Q, np.float64); K = np.asarray(K, np.float64); V = np.asarray(V, np.float64)
    Tq, d = Q.shape
    Tk, dv = V.shape
    c = 1.0 / math.sqrt(d) if scale is None else scale
    cnt = counter if counter is not None else Counter()
    n_r, n_c = math.ceil(Tq / Br), math.ceil(Tk / Bc)
    O = np.zeros((Tq, dv)); l_hbm = np.zeros(Tq); m_hbm = np.full(Tq, -np.inf)
    for j in range(n_c):
        l0, l1 = j * Bc, min((j + 1) * Bc, Tk)
        Kj, Vj = K[l0:l1], V[l0:l1]; cnt.reads += Kj.size + Vj.size
        for i in range(n_r):
            if causal and skip_tile(i, j, Br, Bc, Tq):
                continue
            r0, r1 = i * Br, min((i + 1) * Br, Tq)
            Qi, Oi, li, mi = Q[r0:r1], O[r0:r1], l_hbm[r0:r1], m_hbm[r0:r1]
            cnt.reads += Qi.size + Oi.size + li.size + mi.size
            cnt.tiles += 1
            S = _mask_tile(c * (Qi @ Kj.T), r0, l0, causal)
            m_new = np.maximum(mi, S.max(axis=1))
            ref = np.where(np.isneginf(m_new), 0.0, m_new)
            Pt = np.exp(S - ref[:, None])
            alpha = np.exp(mi - ref)
            l_new = alpha * li + Pt.sum(axis=1)
            safe = np.where(l_new > 0, l_new, 1.0)
            O[r0:r1] = ((alpha * li)[:, None] * Oi + Pt @ Vj) / safe[:, None]
            l_hbm[r0:r1] = l_new; m_hbm[r0:r1] = m_new
            cnt.writes += Oi.size + li.size + mi.size
    return O, m_hbm + np.log(l_hbm)


def fa2_backward(Q, K, V, O, dO, lse, Br, Bc, causal=False, scale=None, counter=None):
    """Tiled backward, key blocks outside, recomputing P from lse.

    Returns dQ, dK, dV.  dQ is updated in HBM by read-add-write per tile.
    """
    Q = np.asarray(Q, np.float64); K = np.asarray(K, np.float64); V = np.asarray(V, np.float64)
    O = np.asarray(O, np.float64); dO = np.asarray(dO, np.float64); lse = np.asarray(lse, np.float64)
    Tq, d = Q.shape
    Tk, dv = V.shape
    c = 1.0 / math.sqrt(d) if scale is None else scale
    cnt = counter if counter is not None else Counter()
    n_r, n_c = math.ceil(Tq / Br), math.ceil(Tk / Bc)
    # pre-pass: D_r = dO_r . O_r (Observation 2)
    D = np.sum(dO * O, axis=1); cnt.reads += dO.size + O.size; cnt.writes += D.size
    dQ = np.zeros((Tq, d)); cnt.writes += dQ.size
    dK = np.zeros((Tk, d)); dV = np.zeros((Tk, dv))
    for j in range(n_c):
        l0, l1 = j * Bc, min((j + 1) * Bc, Tk)
        Kj, Vj = K[l0:l1], V[l0:l1]; cnt.reads += Kj.size + Vj.size
        dKj = np.zeros_like(Kj); dVj = np.zeros_like(Vj)
        for i in range(n_r):
            if causal and skip_tile(i, j, Br, Bc, Tq):
                continue
            r0, r1 = i * Br, min((i + 1) * Br, Tq)
            Qi, dOi, Li, Di = Q[r0:r1], dO[r0:r1], lse[r0:r1], D[r0:r1]
            cnt.reads += Qi.size + dOi.size + Li.size + Di.size
            cnt.tiles += 1
            S = _mask_tile(c * (Qi @ Kj.T), r0, l0, causal)       # Observation 1
            P = np.exp(S - Li[:, None])
            dVj += P.T @ dOi
            dP = dOi @ Vj.T
            dS = P * (dP - Di[:, None])                            # Observation 3
            dKj += c * (dS.T @ Qi)
            cnt.reads += (r1 - r0) * d                             # dQ_i read
            dQ[r0:r1] += c * (dS @ Kj)
            cnt.writes += (r1 - r0) * d                            # dQ_i write
        dK[l0:l1] = dKj; dV[l0:l1] = dVj; cnt.writes += dKj.size + dVj.size
    return dQ, dK, dV


def standard_forward(Q, K, V, causal=False, scale=None, counter=None):
    """Materialising attention with the traffic [Blog] "The Real Bottleneck" lists."""
    Q = np.asarray(Q, np.float64); K = np.asarray(K, np.float64); V = np.asarray(V, np.float64)
    Tq, d = Q.shape
    Tk = K.shape[0]
    c = 1.0 / math.sqrt(d) if scale is None else scale
    cnt = counter if counter is not None else Counter()
    cnt.reads += Q.size + K.size
    S = _mask_tile(c * (Q @ K.T), 0, 0, causal); cnt.writes += S.size
    cnt.reads += S.size
    P = np.exp(S - S.max(axis=1, keepdims=True)); P /= P.sum(axis=1, keepdims=True)
    cnt.writes += P.size
    cnt.reads += P.size + V.size
    O = P @ V; cnt.writes += O.size
    return O


def standard_traffic(Tq, Tk, d):
    """Values moved by materialising attention: 4 Tq Tk + 2 Tq d + 2 Tk d."""
    return 4 * Tq * Tk + 2 * Tq * d + 2 * Tk * d


def fa2_forward_traffic(T, d, Br):
    """FlashAttention-2 order count T d + 2 T d ceil(T/Br) + T d + T
    ([ZtF] "The IO complexity theorem", the paragraph on the FA-2 order)."""
    return T * d + 2 * T * d * math.ceil(T / Br) + T * d + T


def fa1_forward_traffic(T, d, Bc):
    """Original order: 2 T d + n_c (3 T d + 4 T) ([ZtF] proof of the theorem)."""
    return 2 * T * d + math.ceil(T / Bc) * (3 * T * d + 4 * T)


def block_sizes(M, d):
    """The proof's block sizes: Bc = ceil(M / 4d), Br = min(ceil(M / 4d), d)."""
    bc = math.ceil(M / (4 * d))
    return min(bc, d), bc
