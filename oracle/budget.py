"""Plain CPU oracle of per-query-block budgets (ragged k_i under a fixed total).

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module. The
product path never imports it and shares no code with it.

Source: "Sparsity Should Be ALLOTted by Output: Training-Free Allocation of
Block-Sparse Attention for Video Diffusion Transformers" (review, sections 1
to 3): instead of one density for every output, a fixed total budget of
block-sparse attention is shared out unevenly, by an estimate of what each
output needs, without training.

The page gives no estimator; the reading taken here is the plainest one the
PISA quantities support:
  * need of query block i = the effective number of key blocks its attention
    spreads over, w_i = exp(H_i), H_i the entropy of the zeroth-order block
    masses p_ij proportional to n_j exp(scale qbar_i . kbar_j) (the tail
    estimate PISA itself uses);
  * the budget K (blocks per head) minus a floor of k_min per row is shared
    in proportion to w, with w fixed to integers first (wq_i = w_i 2^16
    rounded to nearest) so the sharing is exact integer arithmetic: row i
    gets floor(R wq_i / sum wq) and the R - sum of those leftover blocks go
    to the rows with the largest remainders (R wq_i mod sum wq), ties to the
    lower i (the largest-remainder method);
  * a row holds at most T blocks. The total is fixed, so what a full row
    cannot take is shared again: every row whose floor share reaches
    T - k_min is set to T and leaves, and the rest of R is shared among the
    remaining rows by the same rule, until no share reaches the cap
    (water-filling). The total is then exactly K whenever K <= T^2;
  * each row then keeps its k_i best blocks by the covariance-aware PISA
    score, exactly as the fixed-k routing does.
"""

from __future__ import annotations

import math

import numpy as np

from .pisa import block_ranges

__all__ = ["WEIGHT_ONE", "block_weights", "quantise_weights", "allocate", "route_ragged"]

WEIGHT_ONE = 1 << 16   # fixed-point unit of the integer weights


def block_weights(q: np.ndarray, kbar: np.ndarray, scale: float, block: int) -> np.ndarray:
    """w_i = exp(entropy of p_i.), p_ij = n_j exp(a_ij) / sum_j n_j exp(a_ij), a = scale qbar kbar^T."""
    q = np.asarray(q, dtype=np.float64)
    L = q.shape[0]
    rng_ = block_ranges(L, block)
    n = np.array([e - s for s, e in rng_], dtype=np.float64)
    qbar = np.stack([q[s:e].sum(axis=0) / (e - s) for s, e in rng_])
    a = scale * (qbar @ np.asarray(kbar, dtype=np.float64).T)   # [T, T]
    w = np.empty(len(rng_))
    for i in range(len(rng_)):
        x = a[i] + np.log(n)
        x = x - x.max()
        p = np.exp(x) / np.exp(x).sum()
        nz = p > 0
        w[i] = math.exp(-(p[nz] * np.log(p[nz])).sum())
    return w


def quantise_weights(w: np.ndarray) -> np.ndarray:
    """Integer weights: w * 2^16 rounded to nearest (halves up)."""
    return np.floor(np.asarray(w, dtype=np.float64) * WEIGHT_ONE + 0.5).astype(np.int64)


def allocate(wq: np.ndarray, k_total: int, k_min: int) -> np.ndarray:
    """k_i for one head from the integer weights (largest-remainder method,
    rows capped at T with the excess shared again among the others)."""
    wq = [int(x) for x in wq]
    T = len(wq)
    R = k_total - T * k_min
    assert R >= 0
    cap = T - k_min
    full = [False] * T
    while True:
        act = [i for i in range(T) if not full[i]]
        S = sum(wq[i] for i in act)
        if S == 0:
            break
        newly = [i for i in act if R * wq[i] // S >= cap]
        if not newly:
            break
        for i in newly:
            full[i] = True
        R -= cap * len(newly)
    k = [T if full[i] else k_min for i in range(T)]
    act = [i for i in range(T) if not full[i]]
    if act:
        S = sum(wq[i] for i in act)
        base = {i: R * wq[i] // S for i in act}
        rem = {i: R * wq[i] % S for i in act}
        left = R - sum(base.values())
        order = sorted(act, key=lambda i: (-rem[i], i))   # largest remainder first, ties to lower i
        for i in act:
            k[i] += base[i]
        for i in order[:left]:
            k[i] += 1
    return np.minimum(np.array(k, dtype=np.int64), T)


def route_ragged(q, kbar, M, k, lam: float, scale: float, block: int):
    """S_i = the k_i highest covariance-aware scores of row i (ties to the lower
    j), ascending. Returns (list of index arrays, score [T, T])."""
    q = np.asarray(q, dtype=np.float64)
    rng_ = block_ranges(q.shape[0], block)
    T = len(rng_)
    qbar = np.stack([q[s:e].sum(axis=0) / (e - s) for s, e in rng_])
    score = scale * (qbar @ np.asarray(kbar, dtype=np.float64).T) + lam * np.asarray(M)[None, :]
    cols = np.arange(T)
    out = []
    for i in range(T):
        order = np.lexsort((cols, -score[i]))
        out.append(np.sort(order[:int(k[i])]))
    return out, score
