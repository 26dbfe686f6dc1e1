"""Pins of the fp64 oracle to facts outside itself (CPU only).

Each test fixes the oracle against mathematics the PISA summary ("PISA:
Piecewise Sparse Attention Is Wiser for Efficient Diffusion Transformers",
section 2) implies, never against a retyped copy of the oracle's own formula:
  1. dense equality when every block is exact (a library softmax),
  2. the zeroth-order term is exact for blocks with constant keys,
  3. the first-order term drops out of the denominator (sum_n (k_n - kbar) = 0),
  4. agreement with a scalar brute-force Taylor evaluation,
plus Taylor-order slopes, closed-form spectral norms, brute-force routing,
and exact invariances (key shift, value shift, linearity, permutations).
"""

import math

import numpy as np
import pytest
import scipy.special

from oracle import pisa


def _rand(L, d, seed, scale=1.0):
    g = np.random.default_rng(seed)
    return (g.standard_normal((L, d)) * scale,
            g.standard_normal((L, d)) * scale,
            g.standard_normal((L, d)))


def _random_idx(T, k, seed):
    g = np.random.default_rng(seed)
    return np.stack([np.sort(g.choice(T, size=k, replace=False)) for _ in range(T)]) if k else np.zeros((T, 0), np.int64)


# ---------------------------------------------------------------- fact 1
@pytest.mark.parametrize("L,block,d,lam", [(200, 64, 16, 0.1), (64, 64, 8, 0.0), (37, 16, 8, 5.0), (256, 32, 12, 0.1)])
def test_dense_equality_when_all_blocks_exact(L, block, d, lam):
    q, k, v = _rand(L, d, seed=L + d)
    scale = 1 / math.sqrt(d)
    T = -(-L // block)
    st = pisa.block_stats(k, v, block)
    idx, _ = pisa.route(q, st["kbar"], st["M"], T, lam, scale, block)
    assert (idx == np.arange(T)[None]).all()
    o = pisa.attention(q, k, v, st, idx, scale, block)
    ref = scipy.special.softmax(scale * q @ k.T, axis=1) @ v
    assert np.abs(o - ref).max() < 1e-12


# ---------------------------------------------------------------- fact 2
@pytest.mark.parametrize("L,block,k_keep", [(150, 32, 0), (150, 32, 2), (64 * 5 - 9, 64, 1), (64 * 4, 64, 3)])
def test_zeroth_order_exact_for_constant_key_blocks(L, block, k_keep):
    d = 8
    g = np.random.default_rng(7)
    T = -(-L // block)
    centers = g.standard_normal((T, d)) * 2.0
    k = np.repeat(centers, block, axis=0)[:L]          # every key of block j equals centers[j]
    q = g.standard_normal((L, d))
    v = g.standard_normal((L, d))
    scale = 0.7
    st = pisa.block_stats(k, v, block, keep_H=True)
    assert np.abs(st["H"]).max() < 1e-12 and np.abs(st["Hbar"]).max() < 1e-12
    assert np.abs(st["M"]).max() < 1e-12
    idx = _random_idx(T, k_keep, seed=3)
    o = pisa.attention(q, k, v, st, idx, scale, block)
    ref = scipy.special.softmax(scale * q @ k.T, axis=1) @ v
    assert np.abs(o - ref).max() < 1e-12


def test_zeroth_order_term_alone_matches_exact_block_sums():
    # For one constant-key block: alpha * vsum and alpha * n equal the exact sums.
    d, n = 6, 40
    g = np.random.default_rng(1)
    kc = g.standard_normal(d)
    vv = g.standard_normal((n, d))
    qq = g.standard_normal((3, d)) * 0.3
    k = np.tile(kc, (n, 1))
    st = pisa.block_stats(k, vv, 64)
    alpha = np.exp(qq @ st["kbar"][0])
    exact_num = np.exp(qq @ k.T) @ vv
    exact_den = np.exp(qq @ k.T).sum(axis=1)
    assert np.abs(alpha[:, None] * st["vsum"][0] - exact_num).max() < 1e-12
    assert np.abs(alpha * st["n"][0] - exact_den).max() < 1e-12


# ---------------------------------------------------------------- fact 3
def test_first_order_vanishes_from_denominator():
    L, block, d = 203, 32, 8
    q, k, v = _rand(L, d, seed=11, scale=0.8)
    scale = 1 / math.sqrt(d)
    st = pisa.block_stats(k, v, block)
    T = len(st["n"])
    for j, (s, e) in enumerate(pisa.block_ranges(L, block)):
        dev = (k[s:e] - st["kbar"][j]).sum(axis=0)
        assert np.abs(dev).max() <= 1e-12 * np.abs(k).max() * (e - s)
    idx = _random_idx(T, 2, seed=5)
    _, parts = pisa.attention(q, k, v, st, idx, scale, block, return_parts=True, qblocks=range(T))
    rng_ = pisa.block_ranges(L, block)
    for i in range(T):
        s, e = rng_[i]
        m = parts[i]["m"]
        S = set(int(x) for x in idx[i])
        U = [j for j in range(T) if j not in S]
        for r, t in enumerate(range(s, e)):
            qp = scale * q[t]
            exact = sum(math.exp(qp @ k[n] - m[r]) for j in S for n in range(*rng_[j]))
            # brute-force first-order denominator: sum_n alpha_j (1 + q'(k_n - kbar_j))
            first = 0.0
            for j in U:
                a = math.exp(qp @ st["kbar"][j] - m[r])
                for n in range(*rng_[j]):
                    first += a * (1.0 + qp @ (k[n] - st["kbar"][j]))
            assert abs(parts[i]["D"][r] - (exact + first)) < 1e-11 * (exact + first)


# ---------------------------------------------------------------- fact 4
def _brute_force_taylor(q, k, v, block, idx, scale, mode):
    """Scalar loops, no matrices: exact over S_i, Taylor over U_i."""
    L, d = len(q), len(q[0])
    T = -(-L // block)
    ranges = [(j * block, min(L, j * block + block)) for j in range(T)]
    kbar = []
    for s, e in ranges:
        kbar.append([sum(k[n][a] for n in range(s, e)) / (e - s) for a in range(d)])

    def dot(x, y):
        return sum(x[a] * y[a] for a in range(d))

    # global correction vector for a query: (1/T) sum_j' sum_n (q'.(k_n - kbar_j')) v_n
    out = np.zeros((L, d))
    for t in range(L):
        i = t // block
        qp = [scale * x for x in q[t]]
        S = set(int(x) for x in idx[i])
        num = [0.0] * d
        den = 0.0
        for j in range(T):
            s, e = ranges[j]
            if j in S:
                for n in range(s, e):
                    w = math.exp(dot(qp, k[n]))
                    den += w
                    for a in range(d):
                        num[a] += w * v[n][a]
            else:
                alpha = math.exp(dot(qp, kbar[j]))
                for n in range(s, e):
                    first = 0.0
                    if mode == "block":
                        first = dot(qp, [k[n][a] - kbar[j][a] for a in range(d)])
                    den += alpha          # the first-order term adds nothing here
                    for a in range(d):
                        num[a] += alpha * (1.0 + first) * v[n][a]
                if mode == "global":
                    for jj in range(T):
                        s2, e2 = ranges[jj]
                        for n in range(s2, e2):
                            w = alpha * dot(qp, [k[n][a] - kbar[jj][a] for a in range(d)]) / T
                            for a in range(d):
                                num[a] += w * v[n][a]
        out[t] = [x / den for x in num]
    return out


@pytest.mark.parametrize("mode", ["global", "block", "none"])
@pytest.mark.parametrize("L,block,keep", [(43, 8, 2), (40, 8, 0), (24, 8, 3)])
def test_brute_force_taylor(mode, L, block, keep):
    d = 4
    q, k, v = _rand(L, d, seed=L * 3 + keep, scale=0.9)
    scale = 0.6
    st = pisa.block_stats(k, v, block, keep_H=(mode == "block"))
    T = len(st["n"])
    idx = _random_idx(T, keep, seed=L)
    o = pisa.attention(q, k, v, st, idx, scale, block, first_order=mode)
    ref = _brute_force_taylor(q.tolist(), k.tolist(), v.tolist(), block, idx, scale, mode)
    assert np.abs(o - ref).max() < 1e-12


# ------------------------------------------------------- Taylor order slopes
def test_taylor_order_slopes():
    """Block-wise first order errs O(eps^2), zeroth order O(eps) (every block in the tail)."""
    L, block, d = 96, 16, 6
    g = np.random.default_rng(4)
    T = L // block
    centers = g.standard_normal((T, d))
    dev = g.standard_normal((L, d))
    q = g.standard_normal((L, d))
    v = g.standard_normal((L, d))
    idx = np.zeros((T, 0), dtype=np.int64)
    errs = {"block": [], "none": []}
    epss = [0.2, 0.1, 0.05, 0.025]
    for eps in epss:
        k = np.repeat(centers, block, axis=0) + eps * dev
        st = pisa.block_stats(k, v, block, keep_H=True)
        ref = scipy.special.softmax(0.5 * q @ k.T, axis=1) @ v
        for mode in errs:
            o = pisa.attention(q, k, v, st, idx, 0.5, block, first_order=mode)
            errs[mode].append(np.abs(o - ref).max())
    sl = {m: np.polyfit(np.log(epss), np.log(e), 1)[0] for m, e in errs.items()}
    assert 1.8 < sl["block"] < 2.3, sl
    assert 0.8 < sl["none"] < 1.3, sl


# --------------------------------------------------------- spectral norm
def test_spectral_norm_closed_forms():
    g = np.random.default_rng(2)
    u, w = g.standard_normal(9), g.standard_normal(7)
    assert abs(pisa.spectral_norm(np.outer(u, w)) - np.linalg.norm(u) * np.linalg.norm(w)) < 1e-12
    dg = g.standard_normal(8)
    assert abs(pisa.spectral_norm(np.diag(dg)) - np.abs(dg).max()) < 1e-14
    for s in range(5):
        A = np.random.default_rng(s).standard_normal((12, 12))
        sig = pisa.spectral_norm(A)
        fro = np.sqrt((A * A).sum())
        assert fro / math.sqrt(12) <= sig + 1e-12 and sig <= fro + 1e-12
        # independent power iteration on A^T A, run to convergence
        x = np.ones(12)
        prev = 0.0
        for _ in range(100000):
            x = A.T @ (A @ x)
            x /= np.linalg.norm(x)
            est = np.linalg.norm(A @ x)
            if abs(est - prev) < 1e-15 * est:
                break
            prev = est
        assert abs(est - sig) < 1e-10 * sig


def test_block_stats_rank_one_closed_form():
    """Blocks whose key deviations lie along e_a and values along e_b.

    H_j = s_j e_a e_b^T with s_j = sum_n dev_n * val_n, Hbar = mean_j(s_j) e_a e_b^T,
    so M_j = |s_j - mean(s)| exactly; this pins the definition of H_j, the mean
    over all T blocks (partial block included) and the norm.
    """
    d, block, L = 5, 8, 8 * 3 + 5
    g = np.random.default_rng(9)
    T = -(-L // block)
    a_ax, b_ax = 1, 3
    k = np.zeros((L, d))
    v = np.zeros((L, d))
    s_expected = []
    for j in range(T):
        s0, e0 = j * block, min(L, j * block + block)
        n = e0 - s0
        base = g.standard_normal(d)
        dev = g.standard_normal(n)
        dev -= dev.mean()
        val = g.standard_normal(n)
        k[s0:e0] = base
        k[s0:e0, a_ax] += dev
        v[s0:e0, b_ax] = val
        s_expected.append(float((dev * val).sum()))
    st = pisa.block_stats(k, v, block, keep_H=True)
    mean_s = sum(s_expected) / T
    for j in range(T):
        assert abs(st["H"][j][a_ax, b_ax] - s_expected[j]) < 1e-12
        assert abs(st["M"][j] - abs(s_expected[j] - mean_s)) < 1e-12
    assert abs(st["Hbar"][a_ax, b_ax] - mean_s) < 1e-12


def test_block_stats_rank_two_closed_form():
    """Two orthogonal deviation/value pairs per block make H_j - Hbar diagonal.

    Key deviations along e_a and e_c, values along e_b and e_e, with the cross
    sums forced to zero, give H_j = s1_j e_a e_b^T + s2_j e_c e_e^T, so
    M_j = max(|s1_j - mean s1|, |s2_j - mean s2|): the spectral norm, which a
    Frobenius norm would miss.
    """
    d, block, L = 6, 16, 16 * 4 - 3
    g = np.random.default_rng(12)
    T = -(-L // block)
    a_ax, c_ax, b_ax, e_ax = 0, 2, 1, 5
    k = np.zeros((L, d))
    v = np.zeros((L, d))
    s1, s2 = [], []
    for j in range(T):
        s0, e0 = j * block, min(L, j * block + block)
        n = e0 - s0
        dev1, dev2 = g.standard_normal(n), g.standard_normal(n)
        dev1 -= dev1.mean()
        dev2 -= dev2.mean()
        val1, val2 = g.standard_normal(n), g.standard_normal(n)
        val2 -= (val2 @ dev1) / (dev1 @ dev1) * dev1
        val1 -= (val1 @ dev2) / (dev2 @ dev2) * dev2
        k[s0:e0] = g.standard_normal(d)
        k[s0:e0, a_ax] += dev1
        k[s0:e0, c_ax] += dev2
        v[s0:e0, b_ax] = val1
        v[s0:e0, e_ax] = val2
        s1.append(float(dev1 @ val1))
        s2.append(float(dev2 @ val2))
    st = pisa.block_stats(k, v, block)
    m1, m2 = sum(s1) / T, sum(s2) / T
    for j in range(T):
        want = max(abs(s1[j] - m1), abs(s2[j] - m2))
        assert abs(st["M"][j] - want) < 1e-12 * max(1.0, want)


# --------------------------------------------------------------- routing
def _brute_route(q, kbar, M, keep, lam, scale, block):
    L, d = q.shape
    T = kbar.shape[0]
    out = []
    for i in range(T):
        rows = range(i * block, min(L, i * block + block))
        qb = [sum(q[t][a] for t in rows) / len(rows) for a in range(d)]
        sc = [(scale * sum(qb[a] * kbar[j][a] for a in range(d)) + lam * M[j], j) for j in range(T)]
        top = sorted(sc, key=lambda x: (-x[0], x[1]))[:keep]
        out.append(sorted(j for _, j in top))
    return np.array(out, dtype=np.int64).reshape(T, keep)


@pytest.mark.parametrize("lam", [0.0, 0.1, 3.0])
@pytest.mark.parametrize("keep", [0, 1, 3, 7])
def test_route_brute_force(lam, keep):
    L, block, d = 7 * 16 - 5, 16, 6
    q, k, v = _rand(L, d, seed=keep + 10, scale=1.2)
    st = pisa.block_stats(k, v, block)
    idx, _ = pisa.route(q, st["kbar"], st["M"], keep, lam, 0.4, block)
    assert (idx == _brute_route(q, st["kbar"], st["M"], keep, lam, 0.4, block)).all()


def test_route_special_cases():
    L, block, d = 10 * 16, 16, 6
    q, k, v = _rand(L, d, seed=2)
    st = pisa.block_stats(k, v, block)
    T = 10
    # huge lambda: the same top-k of M_j for every query block
    idx, _ = pisa.route(q, st["kbar"], st["M"], 4, 1e9, 0.4, block)
    topM = np.sort(np.argsort(-st["M"], kind="stable")[:4])
    assert (idx == topM[None]).all()
    # lambda 0: top-k of the centroid score alone
    idx0, sc = pisa.route(q, st["kbar"], st["M"], 4, 0.0, 0.4, block)
    qbar = q.reshape(T, block, d).mean(axis=1)
    cs = qbar @ st["kbar"].T
    for i in range(T):
        assert set(idx0[i]) == set(np.argsort(-cs[i], kind="stable")[:4])
    # keep = T selects everything
    idxT, _ = pisa.route(q, st["kbar"], st["M"], T, 0.1, 0.4, block)
    assert (idxT == np.arange(T)[None]).all()


def test_route_ties_go_to_lower_index():
    # duplicate kv blocks give exactly equal scores; the lower index must win
    block, d = 8, 4
    g = np.random.default_rng(0)
    kb = g.standard_normal((3, block, d))
    vb = g.standard_normal((3, block, d))
    k = np.concatenate([kb[0], kb[1], kb[0], kb[2], kb[1]])
    v = np.concatenate([vb[0], vb[1], vb[0], vb[2], vb[1]])
    q = g.standard_normal((5 * block, d))
    st = pisa.block_stats(k, v, block)
    # blocks 0/2 and 1/4 are identical in kbar, but M differs through Hbar only
    # when H differs; both pairs share H as well, so scores tie exactly
    for keep in range(1, 5):
        idx, sc = pisa.route(q, st["kbar"], st["M"], keep, 0.1, 0.5, block)
        assert (idx == _brute_route(q, st["kbar"], st["M"], keep, 0.1, 0.5, block)).all()
    assert sc[0, 0] == sc[0, 2] and sc[0, 1] == sc[0, 4]


# ------------------------------------------------------------ invariances
def _full(q, k, v, block, keep, lam, scale, first_order="global"):
    st = pisa.block_stats(k, v, block, keep_H=(first_order == "block"))
    idx, _ = pisa.route(q, st["kbar"], st["M"], keep, lam, scale, block)
    return idx, pisa.attention(q, k, v, st, idx, scale, block, first_order=first_order)


@pytest.mark.parametrize("first_order", ["global", "block"])
def test_key_shift_invariance(first_order):
    L, block, d = 150, 32, 8
    q, k, v = _rand(L, d, seed=21)
    idx0, o0 = _full(q, k, v, block, 2, 0.1, 0.35, first_order)
    c = np.random.default_rng(3).standard_normal(d)
    idx1, o1 = _full(q, k + c, v, block, 2, 0.1, 0.35, first_order)
    assert (idx0 == idx1).all()
    assert np.abs(o0 - o1).max() < 1e-11


def test_value_shift_and_linearity():
    L, block, d = 150, 32, 8
    q, k, v = _rand(L, d, seed=22)
    scale = 0.35
    st = pisa.block_stats(k, v, block)
    idx, _ = pisa.route(q, st["kbar"], st["M"], 2, 0.1, scale, block)
    o = pisa.attention(q, k, v, st, idx, scale, block)
    c = np.random.default_rng(5).standard_normal(d)
    st_c = pisa.block_stats(k, v + c, block)
    assert np.abs(st_c["Hbar"] - st["Hbar"]).max() < 1e-12
    o_c = pisa.attention(q, k, v + c, st_c, idx, scale, block)
    assert np.abs(o_c - (o + c)).max() < 1e-11
    v2 = np.random.default_rng(6).standard_normal((L, d))
    st2 = pisa.block_stats(k, v2, block)
    o2 = pisa.attention(q, k, v2, st2, idx, scale, block)
    st3 = pisa.block_stats(k, 2.0 * v - 3.0 * v2, block)
    o3 = pisa.attention(q, k, 2.0 * v - 3.0 * v2, st3, idx, scale, block)
    assert np.abs(o3 - (2.0 * o - 3.0 * o2)).max() < 1e-11


def test_permutation_inside_block_and_across_heads():
    L, block, d = 128, 32, 8
    q, k, v = _rand(L, d, seed=23)
    idx0, o0 = _full(q, k, v, block, 2, 0.1, 0.35)
    perm = np.arange(L)
    g = np.random.default_rng(1)
    for j in range(L // block):
        perm[j * block:(j + 1) * block] = g.permutation(np.arange(j * block, (j + 1) * block))
    idx1, o1 = _full(q, k[perm], v[perm], block, 2, 0.1, 0.35)
    assert (idx0 == idx1).all() and np.abs(o0 - o1).max() < 1e-12
    Q = np.stack([_rand(L, d, s)[0] for s in range(3)])[None]
    K = np.stack([_rand(L, d, s)[1] for s in range(3)])[None]
    V = np.stack([_rand(L, d, s)[2] for s in range(3)])[None]
    r = pisa.pisa_reference(Q, K, V, block, 2, 0.1, 0.35)
    rp = pisa.pisa_reference(Q[:, ::-1], K[:, ::-1], V[:, ::-1], block, 2, 0.1, 0.35)
    for h in range(3):
        assert np.array_equal(r[(0, h)]["O"], rp[(0, 2 - h)]["O"])


def test_keep_or_drop_mode_is_renormalised_sparse_attention():
    """tail=False is plain attention restricted to the exact blocks."""
    L, block, d = 96, 16, 6
    q, k, v = _rand(L, d, seed=30)
    st = pisa.block_stats(k, v, block)
    idx = _random_idx(6, 2, seed=2)
    o = pisa.attention(q, k, v, st, idx, 0.5, block, tail=False)
    for i in range(6):
        keys = np.concatenate([np.arange(j * block, (j + 1) * block) for j in idx[i]])
        rows = slice(i * block, (i + 1) * block)
        ref = scipy.special.softmax(0.5 * q[rows] @ k[keys].T, axis=1) @ v[keys]
        assert np.abs(o[rows] - ref).max() < 1e-12


def test_captured_mass_pins():
    """captured_mass (share of the dense softmax mass on S_i, the coverage
    measure of the vector-quantized attention review, Table 6) pinned three
    ways: it is 1 when S_i holds every block; with equal logits the softmax is
    uniform over the L keys, so the share is sum_{j in S_i} n_j / L (a partial
    last block counts its valid keys only); and on random inputs it equals a
    per-token loop of math.exp over every key."""
    g = np.random.default_rng(12)
    L, block, d = 64 * 5 + 23, 64, 8
    T = -(-L // block)
    q, k = g.standard_normal((L, d)), g.standard_normal((L, d))
    scale = 1 / math.sqrt(d)
    idx_all = np.tile(np.arange(T), (T, 1))
    cm = pisa.captured_mass(q, k, idx_all, scale, block, range(T))
    for i in range(T):
        assert np.allclose(cm[i], 1.0, atol=1e-12)
    # equal logits: q = 0 (every logit 0); the partial block 5 holds 23 keys
    idx = np.array([[0, 5], [1, 2], [3, 5], [0, 4], [2, 3], [1, 5]])
    cm = pisa.captured_mass(np.zeros((L, d)), k, idx, scale, block, range(T))
    n = np.array([64, 64, 64, 64, 64, 23])
    for i in range(T):
        assert np.allclose(cm[i], n[idx[i]].sum() / L, atol=1e-13), i
    # brute force on random inputs (a scale large enough for a peaked softmax)
    cm = pisa.captured_mass(q, k, idx, 1.3, block, [0, 5])
    for i in (0, 5):
        s, e = i * block, min(i * block + block, L)
        keep = set()
        for j in idx[i]:
            keep.update(range(j * block, min(j * block + block, L)))
        for r, t in enumerate(range(s, e)):
            ws = [math.exp(1.3 * float(q[t] @ k[u])) for u in range(L)]
            want = sum(ws[u] for u in keep) / sum(ws)
            assert abs(cm[i][r] - want) < 1e-12
    # and it is what the exact part of PISA sees: the keep-or-drop output
    # times the captured share equals the dense numerator's S_i part over D_dense
    v = g.standard_normal((L, d))
    st = pisa.block_stats(k, v, block)
    od = pisa.attention(q, k, v, st, idx, scale, block, tail=False, qblocks=[2])[2]
    cm = pisa.captured_mass(q, k, idx, scale, block, [2])[2]
    s, e = 2 * block, 3 * block
    lg = scale * q[s:e] @ k.T
    p = np.exp(lg - lg.max(axis=1, keepdims=True))
    mask = np.zeros(L, bool)
    for j in idx[2]:
        mask[j * block:min(j * block + block, L)] = True
    want = (p[:, mask] @ v[mask]) / p.sum(axis=1, keepdims=True)
    assert np.allclose(od * cm[:, None], want, atol=1e-12)


def test_dense_attention_and_block_ranges():
    """dense_attention (the reference of the dense control and of the
    discriminating gates) is textbook softmax attention: equal to scipy's
    softmax times V, row subsets included, and invariant to a logit shift of
    1000 (max subtraction). block_ranges cuts L into ceil(L / block) blocks,
    the last one partial."""
    g = np.random.default_rng(3)
    L, d = 150, 8
    q, k, v = g.standard_normal((L, d)), g.standard_normal((L, d)), g.standard_normal((L, d))
    ref = scipy.special.softmax(0.4 * q @ k.T, axis=1) @ v
    assert np.abs(pisa.dense_attention(q, k, v, 0.4) - ref).max() < 1e-13
    rows = [0, 7, 149]
    assert np.abs(pisa.dense_attention(q, k, v, 0.4, rows=rows) - ref[rows]).max() < 1e-13
    # a constant added to every logit of a row changes nothing
    e = np.zeros(d)
    e[0] = 1.0
    qs = q + 1000.0 * e
    ks = np.concatenate([k[:, :1] * 0 + 1.0, k[:, 1:]], axis=1)     # k_0 = 1 for every key
    ref_s = scipy.special.softmax(0.4 * (q + 0 * e) @ ks.T, axis=1) @ v
    assert np.abs(pisa.dense_attention(qs, ks, v, 0.4) - ref_s).max() < 1e-9
    assert pisa.block_ranges(150, 64) == [(0, 64), (64, 128), (128, 150)]
    assert pisa.block_ranges(64, 64) == [(0, 64)] and pisa.block_ranges(1, 64) == [(0, 1)]


def test_block_stats_without_spectral_norms_keeps_the_other_statistics():
    """block_stats(..., spectral=False) leaves M out and nothing else changes."""
    g = np.random.default_rng(4)
    k, v = g.standard_normal((64 * 5 + 9, 32)), g.standard_normal((64 * 5 + 9, 32))
    full = pisa.block_stats(k, v, 64)
    part = pisa.block_stats(k, v, 64, spectral=False)
    assert part["M"] is None
    for name in ("kbar", "vsum", "n", "Hbar"):
        assert np.array_equal(full[name], part[name]), name
