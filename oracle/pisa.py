"""Plain fp64 CPU oracle of PISA block-sparse attention.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module. The
product path (the HIP kernels behind ``include/paro.h`` and their Python
binding) never imports it and shares no code with it.

Source of every formula: "PISA: Piecewise Sparse Attention Is Wiser for
Efficient Diffusion Transformers" (technical summary), section 2:
  * "core algorithm": o_t = N_t / D_t; the numerator N_t is the exact sum over
    the critical blocks S_i, plus the block-wise zeroth-order term
    alpha_{t,j} * sum_n v_{j,n} over the uncritical blocks U_i with
    alpha_{t,j} = exp(q_t kbar_j^T), plus the global first-order correction
    q_t Hbar sum_{j in U_i} alpha_{t,j}; Hbar is the mean of the block-wise
    first-order matrices over all blocks;
  * "covariance-aware routing": the block score combines the attention score
    with M_j = ||H_j - Hbar||_2;
  * "hardware implementation": precompute, then stage 1 exact, stage 2
    zeroth-order scan, stage 3 correction.

Readings taken where the page is silent (each one is listed with its reason
in the design notes of this repository):
  * scale: q' = scale * q (scale = 1/sqrt(d)) everywhere inside the softmax,
    including the correction q' Hbar; the routing score uses
    scale * qbar_i . kbar_j + lam * M_j, a raw sum with no softmax.
  * H_j = sum_n (k_{j,n} - kbar_j)^T v_{j,n} (a sum, d_k x d_v), which makes
    alpha_j q' H_j the exact first-order Taylor term of sum_n exp(q' k_n) v_n
    around kbar_j.
  * D_t (never printed) = exact terms + sum_{j in U_i} alpha_{t,j} n_j: the
    first-order term of the denominator is alpha_j q' sum_n (k_n - kbar_j) = 0.
  * ||.||_2 of a matrix is the spectral norm (largest singular value).
  * Hbar is the unweighted mean over all T blocks of the same (batch, head).
  * top-k: highest score first, exact ties to the lower block index, and S_i
    listed in ascending block order; no forced blocks.
  * a partial last block uses only its valid tokens (n_j < block) for the
    statistics, the exact keys and the denominator weight n_j; padded query
    rows produce no output.
  * one softmax maximum shared by the exact and approximate terms (it
    changes rounding only).

All arithmetic is float64. Library routines used as single steps: numpy
matmul and ``numpy.linalg.svd``.
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "block_ranges", "block_stats", "spectral_norm", "route", "attention",
    "dense_attention", "pisa_reference", "captured_mass",
]


def block_ranges(L: int, block: int):
    """Token ranges [start, stop) of the T = ceil(L / block) blocks."""
    T = -(-L // block)
    return [(j * block, min(j * block + block, L)) for j in range(T)]


def spectral_norm(A: np.ndarray) -> np.ndarray:
    """Largest singular value of each matrix in A[..., m, n] (LAPACK SVD)."""
    return np.linalg.svd(A, compute_uv=False)[..., 0]


def block_stats(k: np.ndarray, v: np.ndarray, block: int, keep_H: bool = False, spectral: bool = True):
    """Precompute stage for one (batch, head): k, v are [L, d] float64.

    Section 2, "hardware implementation", pre-computation step (block
    centroids, value sums, global statistic Hbar) and "covariance-aware
    routing" (M_j = ||H_j - Hbar||_2).

    Returns a dict with kbar [T, d], vsum [T, d], n [T] (valid tokens per
    block), Hbar [d, d] and M [T]; H [T, d, d] as well when ``keep_H``.
    ``spectral=False`` leaves M out (None): attention needs only the other
    statistics, and the SVDs dominate the cost.
    """
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    L, d = k.shape
    rng_ = block_ranges(L, block)
    T = len(rng_)
    n = np.array([e - s for s, e in rng_], dtype=np.int64)
    kbar = np.empty((T, d))
    vsum = np.empty((T, d))
    H = np.empty((T, d, v.shape[1]))
    for j, (s, e) in enumerate(rng_):
        kj, vj = k[s:e], v[s:e]
        kbar[j] = kj.sum(axis=0) / (e - s)           # block centroid
        vsum[j] = vj.sum(axis=0)                     # block value sum
        H[j] = (kj - kbar[j]).T @ vj                 # block first-order matrix
    Hbar = H.sum(axis=0) / T                         # mean over all blocks
    M = spectral_norm(H - Hbar[None]) if spectral else None   # covariance norm per block
    out = {"kbar": kbar, "vsum": vsum, "n": n, "Hbar": Hbar, "M": M}
    if keep_H:
        out["H"] = H
    return out


def route(q: np.ndarray, kbar: np.ndarray, M: np.ndarray, keep_k: int, lam: float,
          scale: float, block: int):
    """Covariance-aware top-k for one (batch, head).

    Section 2, "covariance-aware routing": score_ij = scale * qbar_i . kbar_j
    + lam * M_j; S_i = the keep_k highest scores (ties to the lower j), in
    ascending order of j.

    Returns (idx [T, keep_k] int64, score [T, T] float64).
    """
    q = np.asarray(q, dtype=np.float64)
    L, d = q.shape
    rng_ = block_ranges(L, block)
    T = len(rng_)
    qbar = np.stack([q[s:e].sum(axis=0) / (e - s) for s, e in rng_])
    score = scale * (qbar @ kbar.T) + lam * M[None, :]
    idx = np.empty((T, keep_k), dtype=np.int64)
    cols = np.arange(T)
    for i in range(T):
        order = np.lexsort((cols, -score[i]))        # score desc, then j asc
        idx[i] = np.sort(order[:keep_k])
    return idx, score


def attention(q, k, v, stats, idx, scale: float, block: int, first_order: str = "global",
              tail: bool = True, qblocks=None, return_parts: bool = False):
    """Piecewise attention output for one (batch, head).

    Section 2, "core algorithm" and "hardware implementation": for each query
    block i, stage 1 sums exp(q' k^T) v exactly over the blocks in S_i; stage
    2 adds alpha_{t,j} vsum_j (numerator) and alpha_{t,j} n_j (denominator)
    for every j in U_i, alpha_{t,j} = exp(q' kbar_j^T); stage 3 adds the
    global first-order correction (q' Hbar) sum_{j in U_i} alpha_{t,j};
    finally o_t = N_t / D_t.

    Test-only modes: ``first_order`` "global" (the method), "block" (the
    per-block term alpha_j q' H_j that the page rejects for its memory cost;
    needs stats["H"]) or "none"; ``tail=False`` drops U_i entirely (the
    keep-or-drop baseline of section 1).

    ``qblocks`` restricts the work to some query blocks. Returns a dict
    {i: o [n_i, d]} when qblocks is given, else the full [L, d] array; with
    ``return_parts`` also the per-block (N, D, c) pieces.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    L, d = q.shape
    rng_ = block_ranges(L, block)
    T = len(rng_)
    kbar, vsum, n, Hbar = stats["kbar"], stats["vsum"], stats["n"], stats["Hbar"]
    todo = range(T) if qblocks is None else qblocks
    outs, parts = {}, {}
    for i in todo:
        s, e = rng_[i]
        qp = scale * q[s:e]                                   # q'
        S = [int(j) for j in idx[i]]
        U = sorted(set(range(T)) - set(S)) if tail else []
        kS = np.concatenate([k[a:b] for a, b in (rng_[j] for j in S)], axis=0) if S else np.zeros((0, d))
        vS = np.concatenate([v[a:b] for a, b in (rng_[j] for j in S)], axis=0) if S else np.zeros((0, v.shape[1]))
        logit_exact = qp @ kS.T                               # [n_i, sum n_j]
        logit_tail = qp @ kbar[U].T                           # [n_i, |U|]
        m = np.full(e - s, -np.inf)
        if logit_exact.shape[1]:
            m = np.maximum(m, logit_exact.max(axis=1))
        if logit_tail.shape[1]:
            m = np.maximum(m, logit_tail.max(axis=1))
        # stage 1: exact sparse terms
        p = np.exp(logit_exact - m[:, None])
        N = p @ vS
        D = p.sum(axis=1)
        # stage 2: block-wise zeroth-order terms, alpha scaled by exp(-m)
        alpha = np.exp(logit_tail - m[:, None])
        N = N + alpha @ vsum[U]
        D = D + alpha @ n[U].astype(np.float64)
        c = alpha.sum(axis=1)
        # stage 3: first-order correction
        if first_order == "global":
            N = N + (qp @ Hbar) * c[:, None]
        elif first_order == "block":
            H = stats["H"]
            for a, j in enumerate(U):
                N = N + alpha[:, a:a + 1] * (qp @ H[j])
        elif first_order != "none":
            raise ValueError(first_order)
        outs[i] = N / D[:, None]
        if return_parts:
            parts[i] = {"N": N, "D": D, "c": c, "m": m}
    if qblocks is None:
        o = np.concatenate([outs[i] for i in range(T)], axis=0)
        return (o, parts) if return_parts else o
    return (outs, parts) if return_parts else outs


def dense_attention(q, k, v, scale: float, rows=None):
    """Textbook softmax(scale q k^T) v for one (batch, head), float64."""
    q = np.asarray(q, dtype=np.float64)
    if rows is not None:
        q = q[rows]
    s = scale * (q @ np.asarray(k, dtype=np.float64).T)
    s = s - s.max(axis=1, keepdims=True)
    p = np.exp(s)
    return (p @ np.asarray(v, dtype=np.float64)) / p.sum(axis=1, keepdims=True)


def captured_mass(q, k, idx, scale: float, block: int, qblocks):
    """Share of the dense softmax mass that falls on the exact blocks S_i.

    Diagnostic in the spirit of the attention-mass coverage reported for
    adaptive vector-quantised attention (Table 6 of that summary).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    rng_ = block_ranges(q.shape[0], block)
    out = {}
    for i in qblocks:
        s, e = rng_[i]
        lg = scale * (q[s:e] @ k.T)
        lg = lg - lg.max(axis=1, keepdims=True)
        p = np.exp(lg)
        mask = np.zeros(k.shape[0], dtype=bool)
        for j in idx[i]:
            a, b = rng_[int(j)]
            mask[a:b] = True
        out[i] = p[:, mask].sum(axis=1) / p.sum(axis=1)
    return out


def pisa_reference(Q, K, V, block: int, keep_k: int, lam: float, scale: float,
                   qblocks=None, heads=None, first_order: str = "global"):
    """Whole pipeline over [B, H, L, d] arrays (any float dtype, read as float64).

    Returns dict with per-(b, h) lists: stats, idx, score, and O ([L, d] array,
    or {i: rows} when ``qblocks`` is given). ``heads`` restricts to some
    (b, h) pairs.
    """
    Q = np.asarray(Q)
    B, H = Q.shape[:2]
    pairs = [(b, h) for b in range(B) for h in range(H)] if heads is None else list(heads)
    res = {}
    for b, h in pairs:
        st = block_stats(K[b, h], V[b, h], block, keep_H=(first_order == "block"))
        idx, score = route(Q[b, h], st["kbar"], st["M"], keep_k, lam, scale, block)
        o = attention(Q[b, h], K[b, h], V[b, h], st, idx, scale, block,
                      first_order=first_order, qblocks=qblocks)
        res[(b, h)] = {"stats": st, "idx": idx, "score": score, "O": o}
    return res
