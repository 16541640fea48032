"""The CPU tiled model against the oracle and against the pages' printed counts."""
import math
import os

import numpy as np
import pytest

from oracle import naive, tiled_model as tm
from tests.test_oracle import _golden, _rand

SHAPES = [(1, 1, 7, 3, 1), (37, 37, 5, 8, 16), (64, 64, 16, 16, 16), (50, 23, 6, 8, 4),
          (23, 50, 6, 4, 8), (100, 100, 8, 32, 16), (100, 100, 8, 16, 32)]


@pytest.mark.parametrize("Tq,Tk,d,Br,Bc", SHAPES)
@pytest.mark.parametrize("causal", [False, True])
def test_fa2_forward_matches_oracle(Tq, Tk, d, Br, Bc, causal):
    q, k, v = _rand((Tq, d), 1), _rand((Tk, d), 2), _rand((Tk, d), 3)
    O, lse = tm.fa2_forward(q, k, v, Br, Bc, causal)
    Or, Lr = naive.forward_head(q, k, v, 1 / math.sqrt(d), causal)
    assert np.abs(O - Or).max() < 1e-12 and np.abs(lse - Lr).max() < 1e-12


@pytest.mark.parametrize("Tq,Tk,d,Br,Bc", SHAPES)
@pytest.mark.parametrize("causal", [False, True])
def test_fa1_forward_matches_oracle(Tq, Tk, d, Br, Bc, causal):
    q, k, v = _rand((Tq, d), 4), _rand((Tk, d), 5), _rand((Tk, d), 6)
    O, lse = tm.fa1_forward(q, k, v, Br, Bc, causal)
    Or, Lr = naive.forward_head(q, k, v, 1 / math.sqrt(d), causal)
    assert np.abs(O - Or).max() < 1e-12 and np.abs(lse - Lr).max() < 1e-12


@pytest.mark.parametrize("Tq,Tk,d,Br,Bc", SHAPES)
@pytest.mark.parametrize("causal", [False, True])
def test_fa2_backward_matches_oracle(Tq, Tk, d, Br, Bc, causal):
    q, k, v, do = _rand((Tq, d), 7), _rand((Tk, d), 8), _rand((Tk, d), 9), _rand((Tq, d), 10)
    c = 1 / math.sqrt(d)
    O, lse = tm.fa2_forward(q, k, v, Br, Bc, causal)
    dQ, dK, dV = tm.fa2_backward(q, k, v, O, do, lse, Br, Bc, causal)
    rQ, rK, rV = naive.backward_head(q, k, v, do, c, causal)[:3]
    for a, b in ((dQ, rQ), (dK, rK), (dV, rV)):
        assert np.abs(a - b).max() < 1e-12


def test_worked_example_running_statistics():
    """[LDD] "Concept": with key blocks of two, l after [1,3] is 1.135 and after [5]
    is 1.154 relative to the running maximum 3, then 5."""
    g = _golden("online_softmax_worked_example.txt")
    q = np.array([[1.0, 0.0, 0.0]])
    k = np.array([[1.0, 0, 0], [3.0, 0, 0], [5.0, 0, 0]])
    seen = []
    O, lse = tm.fa2_forward(q, k, np.eye(3), 1, 2, scale=1.0,
                            trace=lambda i, j, m, l: seen.append((j, m[0], l[0])))
    assert [s[0] for s in seen] == [0, 1]
    assert seen[0][1] == g["m1"] and abs(seen[0][2] - g["l1"]) <= 5e-4
    assert seen[1][1] == 5.0 and abs(seen[1][2] - g["l_final"]) <= 5e-4
    assert abs(seen[0][2] * math.exp(3 - 5) - g["l1_rescaled"]) <= 5e-4
    assert abs(math.exp(3 - 5) - g["rescale"]) <= 5e-4
    # the wrong local softmax of the first block alone
    assert abs(math.exp(3) / (math.exp(1) + math.exp(3)) - g["local_weight_of_3"]) <= 5e-4
    assert abs(O[0, 1] - g["true_weight_of_3"]) <= 5e-4


def test_printed_traffic_and_tile_counts():
    """[ZtF] "The forward pass" and "The causal mask": 1.18 M vs 4.46 M values and
    72 of 128 tiles at the reconstructed T=1024, d=64, Br=128, Bc=64."""
    g = _golden("traffic_counts.txt")
    T, d, Br, Bc = (int(g[x]) for x in ("T", "d", "Br", "Bc"))
    q, k, v = _rand((T, d), 11), _rand((T, d), 12), _rand((T, d), 13)
    c2 = tm.Counter(); tm.fa2_forward(q, k, v, Br, Bc, False, counter=c2)
    cs = tm.Counter(); tm.standard_forward(q, k, v, False, counter=cs)
    assert c2.total == int(g["tiled_values_exact"]) == tm.fa2_forward_traffic(T, d, Br)
    assert cs.total == int(g["standard_values_exact"]) == tm.standard_traffic(T, T, d)
    assert round(c2.total / 1e6, 2) == g["tiled_values_printed_millions"]
    assert round(cs.total / 1e6, 2) == g["standard_values_printed_millions"]
    assert math.ceil(T / Br) == 8
    cc = tm.Counter(); tm.fa2_forward(q, k, v, Br, Bc, True, counter=cc)
    assert cc.tiles == int(g["causal_tiles_visited"])
    assert tm.visited_tiles(T, T, Br, Bc, False) == int(g["causal_tiles_total"])


def test_fa1_order_traffic_matches_the_proof_count():
    """[ZtF] "The IO complexity theorem": 2Td + n_c(3Td + 4T) for the original order."""
    T, d, Br, Bc = 96, 8, 16, 32
    q, k, v = _rand((T, d), 14), _rand((T, d), 15), _rand((T, d), 16)
    c1 = tm.Counter(); tm.fa1_forward(q, k, v, Br, Bc, False, counter=c1)
    assert c1.total == tm.fa1_forward_traffic(T, d, Bc)


def test_block_size_rule_and_theorem_scaling():
    """Bc = ceil(M/4d), Br = min(ceil(M/4d), d); the FA-1 count is about 12 T^2 d^2 / M."""
    T, d, M = 4096, 64, 100_000
    Br, Bc = tm.block_sizes(M, d)
    assert (Br, Bc) == (64, 391)
    count = tm.fa1_forward_traffic(T, d, Bc)
    assert 0.9 < count / (12 * T * T * d * d / M) < 1.2


def test_skip_rule_first_key_vs_last_query():
    """Skip iff first key > last query ([ZtF] "The causal mask").  Comparing first
    with first when Br != Bc drops keys some rows should see."""
    for Br, Bc in ((32, 16), (16, 32)):
        T, d = 96, 4
        n_r, n_c = T // Br, T // Bc
        for i in range(n_r):
            for j in range(n_c):
                needed = any(l <= r for r in range(i * Br, (i + 1) * Br) for l in range(j * Bc, (j + 1) * Bc))
                assert tm.skip_tile(i, j, Br, Bc, T) == (not needed)
    # Br = 2 Bc: first-vs-first would skip tile (0, 1) although row 31 sees key 16
    assert not tm.skip_tile(0, 1, 32, 16, 96) and 1 * 16 > 0 * 32


def test_causal_cost_approaches_half():
    """n(n+1)/2 of n^2 tiles for square blocks."""
    for n in (1, 4, 16):
        assert tm.visited_tiles(n * 8, n * 8, 8, 8, True) == n * (n + 1) // 2
