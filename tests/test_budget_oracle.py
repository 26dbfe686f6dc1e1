"""Pins of the per-query-block budget oracle (CPU only): the effective block
count on closed-form distributions, the largest-remainder sharing on a
worked example and its invariants, and the reduction to the fixed-k routing."""

import math

import numpy as np

from oracle import budget, pisa


def _binary_entropy_w(p):
    return math.exp(-(p * math.log(p) + (1 - p) * math.log(1 - p)))


def test_weights_closed_forms():
    d, scale = 8, 1 / math.sqrt(8)
    e1 = np.eye(d)[0]
    # equal centroids, equal block sizes: the masses are uniform, w = T
    q = np.tile(e1, (64 * 5, 1))
    w = budget.block_weights(q, np.tile(0.3 * e1, (5, 1)), scale, 64)
    assert np.allclose(w, 5.0, rtol=1e-12)
    # two blocks with logits 0 and scale * c: p_1 = 1 / (1 + e^-(scale c)), w = exp(H(p))
    c = 2.5
    q = np.tile(e1, (128, 1))
    w = budget.block_weights(q, np.stack([0 * e1, c * e1]), scale, 64)
    p1 = 1 / (1 + math.exp(-scale * c))
    assert np.allclose(w, _binary_entropy_w(p1), rtol=1e-12)
    # a partial block weighs by its size: equal logits, n = (64, 16) -> p = (0.8, 0.2)
    q = np.tile(e1, (80, 1))
    w = budget.block_weights(q, np.zeros((2, d)), scale, 64)
    assert np.allclose(w, _binary_entropy_w(0.2), rtol=1e-12)
    # one dominant block: w -> 1
    w = budget.block_weights(np.tile(e1, (192, 1)), np.stack([400 * e1, 0 * e1, 0 * e1]), scale, 64)
    assert np.allclose(w, 1.0, atol=1e-9)


def test_allocate_worked_example():
    # R = 6, sum wq = 4: quotas 1.5, 1.5, 3 -> floors 1, 1, 3 (5 blocks); the one left goes
    # to the largest remainder, 6 mod 4 = 2 in rows 0 and 1 (12 mod 4 = 0 in row 2), lower row
    assert budget.allocate(np.array([1, 1, 2]), 6, 0).tolist() == [2, 1, 3]
    # with a floor of one block per row: R = 7 - 3 = 4 shared exactly as 1, 1, 2
    assert budget.allocate(np.array([1, 1, 2]), 7, 1).tolist() == [2, 2, 3]
    # ties of remainders go to the lower row
    assert budget.allocate(np.array([1, 1, 1]), 4, 1).tolist() == [2, 1, 1]


def test_allocate_invariants():
    g = np.random.default_rng(0)
    for trial in range(50):
        T = int(g.integers(2, 300))
        k_min = int(g.integers(0, 4))
        K = int(g.integers(T * k_min, T * k_min + 8 * T))
        wq = budget.quantise_weights(g.uniform(1, T, T))
        k = budget.allocate(wq, K, k_min)
        assert k.sum() == min(K, T * T)   # the total is fixed (all rows full past T^2)
        assert (k >= min(k_min, T)).all()
        # a larger weight never gets fewer blocks, and equal weights differ by at most one
        for i in range(T - 1):
            j = i + 1
            if wq[i] > wq[j]:
                assert k[i] >= k[j]
            if wq[i] == wq[j]:
                assert abs(int(k[i]) - int(k[j])) <= 1
    # equal weights and K = T k: every row gets k
    assert budget.allocate(np.full(7, 99), 7 * 5, 1).tolist() == [5] * 7
    # a row that would exceed T is capped and its excess shared again: R = 5,
    # row 0's share 4.99 reaches the cap T - k_min = 2, so it gets 3; the 3
    # blocks left go to rows 1 and 2 (weights 1, 1: 1.5 each, the odd one to
    # the lower row)
    assert budget.allocate(np.array([10 ** 6, 1, 1]), 8, 1).tolist() == [3, 3, 2]
    # a cascade: T = 4, K = 12, weights 8, 4, 1, 1 (sum 14). Shares 6.9, 3.4,
    # 0.9, 0.9: row 0 is full (4), 8 left over rows 1-3 (sum 6): 5.3, 1.3,
    # 1.3, so row 1 is full too; 4 left over rows 2 and 3: 2 each
    assert budget.allocate(np.array([8, 4, 1, 1]), 12, 0).tolist() == [4, 4, 2, 2]
    # K = T^2: every row full
    assert budget.allocate(np.array([5, 1, 1, 1]), 16, 0).tolist() == [4, 4, 4, 4]


def test_ragged_routing_with_constant_k_is_the_fixed_k_routing():
    g = np.random.default_rng(1)
    L, d = 64 * 9 + 13, 16
    q, k = g.standard_normal((L, d)), g.standard_normal((L, d))
    st = pisa.block_stats(k, g.standard_normal((L, d)), 64)
    ref, sc = pisa.route(q, st["kbar"], st["M"], 4, 0.1, 0.25, 64)
    got, sc2 = budget.route_ragged(q, st["kbar"], st["M"], np.full(10, 4), 0.1, 0.25, 64)
    assert np.array_equal(np.stack(got), ref) and np.array_equal(sc, sc2)
    # ragged: each row's list is the top-k_i of its own score row
    ks = g.integers(0, 11, 10)
    got, _ = budget.route_ragged(q, st["kbar"], st["M"], ks, 0.1, 0.25, 64)
    for i in range(10):
        assert len(got[i]) == ks[i]
        if 0 < ks[i] < 10:
            rest = np.setdiff1d(np.arange(10), got[i])
            assert sc[i, got[i]].min() >= sc[i, rest].max()


def test_quantise_weights_worked_values():
    """wq = w 2^16 rounded to nearest, halves up (both sides of the sharing
    read the weights as these integers): 1.5 -> 98304 exactly; quotients that
    fall on a half go up (3 / 2^17 -> 1.5 -> 2, 1 / 2^17 -> 0.5 -> 1), just
    below a half go down; a truncating or half-even rounding fails here."""
    one = budget.WEIGHT_ONE
    assert one == 65536
    w = np.array([1.5, 3 / 2 ** 17, 1 / 2 ** 17, 5 / 2 ** 17, (2.5 - 2 ** -20) / one, 1.0, 72.0, (7 + 0.5) / one])
    assert budget.quantise_weights(w).tolist() == [98304, 2, 1, 3, 2, 65536, 72 * 65536, 8]
    assert budget.quantise_weights(np.array([0.25])).dtype == np.int64
