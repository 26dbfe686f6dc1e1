"""GPU checks of the per-query-block budgets (paro_route_budget) and of the
attention on CSR lists (paro_attention_csr), against oracle/budget.py.

The need w_i comes from fp32 dot products on the GPU and fp64 in the oracle,
so it is compared with a relative tolerance; the sharing is integer
arithmetic on the integer weights, so the GPU's k_i are compared bit for bit
with the oracle's sharing of the GPU's own integer weights (the sharing
kernel), and separately with the oracle's whole budget (its own weights,
quantised and shared: equal up to a few rows at the largest-remainder cut,
one block apart); the lists are compared like the fixed-k routing (bit-exact
except rows whose swapped blocks are within 1e-5 in oracle score) on the rows
whose k_i agree; attention is fed the oracle's own lists.
"""
import numpy as np
import pytest
import torch

from block_sparse_attention_pisa_amd import paro
from oracle import budget, pisa
from workloads import WORKLOADS, make_inputs

from parity_util import ROUTE_GAP, check_attention, log, run_gpu

pytestmark = pytest.mark.gpu


def _oracle_shares(qn_h, st, scale, K, k_min):
    """The oracle's own budget for one head: its fp64 weights, quantised and
    shared by the oracle (nothing from the GPU)."""
    w_ref = budget.block_weights(qn_h, st["kbar"], scale, 64)
    return w_ref, budget.allocate(budget.quantise_weights(w_ref), K, k_min)


def _check_shares(kk, wq_gpu, w_ref, k_or, K, k_min):
    """k_i of the GPU against (1) the oracle's sharing of the GPU's own
    integer weights, bit for bit (the sharing kernel is integer arithmetic),
    and (2) the oracle's whole budget: weights within 1e-5 relative, the same
    total, and the shares equal except for a few rows that differ by one
    block (the weights are fp32 dot products on the GPU, fp64 in the oracle,
    so a row at the largest-remainder cut can fall on either side)."""
    assert np.array_equal(kk, budget.allocate(wq_gpu, K, k_min))
    rel = np.abs(wq_gpu / budget.WEIGHT_ONE - w_ref) / w_ref
    assert rel.max() < 1e-5, rel.max()
    diff = np.abs(kk.astype(np.int64) - k_or)
    assert kk.sum() == k_or.sum() == min(K, len(k_or) ** 2)
    assert diff.max(initial=0) <= 1 and int((diff > 0).sum()) <= max(2, len(k_or) // 50), diff
    return float(rel.max()), int((diff > 0).sum())


def _csr(lists, stride=None):
    """(offsets [T + 1], idx [stride]) int32 tensors of a list of index arrays."""
    ks = [len(x) for x in lists]
    offs = np.concatenate([[0], np.cumsum(ks)]).astype(np.int32)
    idx = np.zeros(stride or max(1, int(offs[-1])), dtype=np.int32)
    for i, x in enumerate(lists):
        idx[offs[i]:offs[i + 1]] = np.asarray(x, dtype=np.int32)
    return torch.from_numpy(offs), torch.from_numpy(idx)


def _check_lists(got, ref, score):
    excused = 0
    for i, (a, b) in enumerate(zip(got, ref)):
        assert len(a) == len(b)
        assert list(a) == sorted(a) and len(set(a.tolist())) == len(a)
        sa, sb = set(a.tolist()), set(b.tolist())
        if sa == sb:
            continue
        gap = max(score[i, jm] - score[i, je] for je in sa - sb for jm in sb - sa)
        assert gap < ROUTE_GAP, ("routing mismatch", i, gap)
        excused += 1
    return excused


@pytest.mark.parametrize("name,heads,keep_permille,k_min", [
    ("image_4608", [0, 5], 250, 1),
    ("video480p_32760", [0, 11], 125, 2),
    ("tiny_fp32", [0, 1], 250, 0),
])
def test_budget_routing_and_attention(name, heads, keep_permille, k_min):
    w = WORKLOADS[name]
    q, k, v = make_inputs(w, heads=heads)
    T = w.T
    K = -(-keep_permille * T // 1000) * T
    log(f"[budget] {name} heads {heads} k_total {K} k_min {k_min}")
    (qd, kd, vd), stats, _ = run_gpu(q, k, v, 1, w.lam)
    offsets, idx, wq = paro.route_budget(qd, stats[0], stats[3], K, k_min, w.lam)
    offs_h, idx_h, wq_h = offsets.cpu().numpy(), idx.cpu().numpy(), wq.cpu().numpy()
    qn, kn, vn = (x.double().numpy() for x in (q, k, v))
    offs_or = torch.zeros_like(offsets.cpu())
    idx_or = torch.zeros_like(idx.cpu())
    refs = []
    for h in range(len(heads)):
        st = pisa.block_stats(kn[0, h], vn[0, h], 64)
        w_ref, k_or = _oracle_shares(qn[0, h], st, w.scale, K, k_min)
        kk = np.diff(offs_h[0, h])
        assert offs_h[0, h, 0] == 0
        rel, nd = _check_shares(kk, wq_h[0, h], w_ref, k_or, K, k_min)
        ref_lists, score = budget.route_ragged(qn[0, h], st["kbar"], st["M"], k_or, w.lam, w.scale, 64)
        lists = [idx_h[0, h, offs_h[0, h, i]:offs_h[0, h, i + 1]] for i in range(T)]
        same = [i for i in range(T) if kk[i] == k_or[i]]
        ex = _check_lists([lists[i] for i in same], [ref_lists[i] for i in same], score[same])
        log(f"[budget] {name} h{heads[h]}: k_i {kk.min()}..{kk.max()} (sum {kk.sum()}), w rel err {rel:.2g}, "
            f"rows sharing differently from the oracle {nd}, excused rows {ex}")
        offs_or[0, h], idx_or[0, h] = _csr(ref_lists, idx_or.shape[-1])
        refs.append((st, ref_lists))
    # attention on the oracle's own lists
    o = paro.attention_csr(qd, kd, vd, *stats[:3], offs_or.cuda(), idx_or.cuda(), K).float().cpu().numpy()
    for h, (st, ref_lists) in enumerate(refs):
        oref = pisa.attention(qn[0, h], kn[0, h], vn[0, h], st, ref_lists, w.scale, 64)
        mx, mean = check_attention(o[0, h], oref, w.dtype)
        log(f"[budget] {name} h{heads[h]}: attention max {mx:.3g} mean {mean:.3g}")


def test_uniform_budget_is_the_fixed_k_path():
    """k_min = keep and k_total = T keep leave nothing to share: every row
    gets keep, and the CSR route and attention equal the fixed-k ones bit for bit."""
    w = WORKLOADS["image_4608"]
    q, k, v = make_inputs(w, heads=[2])
    (qd, kd, vd), stats, idx = run_gpu(q, k, v, w.k, w.lam)
    offsets, idx_b, _ = paro.route_budget(qd, stats[0], stats[3], w.T * w.k, w.k, w.lam)
    assert torch.equal(offsets.cpu()[0, 0], torch.arange(0, w.T * w.k + 1, w.k, dtype=torch.int32))
    assert torch.equal(idx_b.cpu().reshape(-1), idx.cpu().reshape(-1))
    o1 = paro.attention(qd, kd, vd, *stats[:3], idx, w.k)
    o2 = paro.attention_csr(qd, kd, vd, *stats[:3], offsets, idx_b, w.T * w.k)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))


@pytest.mark.parametrize("per_row", [10, 30])
def test_budget_with_strongly_varying_need(per_row):
    """The varying-need input (workloads.varying_need_inputs: keys of block j
    offset by a random mu_j, so centroid logits vary, and queries pointing
    along one direction with a strength of 0.2, 1 or 5 by block): sharper
    rows spread over fewer blocks, so the sharing is far from uniform. With 30 blocks per row on average (T = 41) the neediest rows
    reach T and what they cannot take is shared again among the others."""
    from workloads import varying_need_inputs
    B, H, L, d = 1, 2, 64 * 40 + 9, 128
    q, k, v = varying_need_inputs(B, H, L, d)
    T, scale = -(-L // 64), 1 / np.sqrt(d)
    K = per_row * T
    (qd, kd, vd), stats, _ = run_gpu(q, k, v, 1, 0.1)
    offsets, idx, wq = paro.route_budget(qd, stats[0], stats[3], K, 1, 0.1)
    offs_h, idx_h, wq_h = offsets.cpu().numpy(), idx.cpu().numpy(), wq.cpu().numpy()
    qn, kn, vn = (x.double().numpy() for x in (q, k, v))
    offs_or = torch.zeros_like(offsets.cpu())
    idx_or = torch.zeros_like(idx.cpu())
    refs = []
    for h in range(H):
        st = pisa.block_stats(kn[0, h], vn[0, h], 64)
        w_ref, k_or = _oracle_shares(qn[0, h], st, scale, K, 1)
        kk = np.diff(offs_h[0, h])
        _, nd = _check_shares(kk, wq_h[0, h], w_ref, k_or, K, 1)
        assert k_or.max() >= 2 * k_or.min() and k_or.sum() == K  # genuinely ragged, the total fixed
        if per_row == 30:
            assert k_or.max() == T and k_or.min() < T      # some rows full, the rest shared again
        ref_lists, score = budget.route_ragged(qn[0, h], st["kbar"], st["M"], k_or, 0.1, scale, 64)
        lists = [idx_h[0, h, offs_h[0, h, i]:offs_h[0, h, i + 1]] for i in range(T)]
        same = [i for i in range(T) if kk[i] == k_or[i]]
        ex = _check_lists([lists[i] for i in same], [ref_lists[i] for i in same], score[same])
        log(f"[budget] varying need h{h}: k_i {kk.min()}..{kk.max()}, rows sharing differently {nd}, excused rows {ex}")
        offs_or[0, h], idx_or[0, h] = _csr(ref_lists, idx_or.shape[-1])
        refs.append((st, ref_lists))
    o = paro.attention_csr(qd, kd, vd, *stats[:3], offs_or.cuda(), idx_or.cuda(), K).float().cpu().numpy()
    for h, (st, ref_lists) in enumerate(refs):
        check_attention(o[0, h], pisa.attention(qn[0, h], kn[0, h], vn[0, h], st, ref_lists, scale, 64), "bf16")


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_csr_attention_on_random_ragged_lists(dtype):
    """Hand-made lists: every row a random count in [0, T] (0 and T included)
    of random distinct blocks, neighbouring rows of one workgroup very
    different, a head stride larger than the total; in all three tail modes
    (in keep-or-drop mode a row with an empty list has nothing to normalise,
    0 / 0, so those rows are left out)."""
    from workloads import random_uniform_inputs
    B, H, L, d = 2, 1, 64 * 21 - 30, 64
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    q, k, v = random_uniform_inputs(B, H, L, d, dtype=tdt, seed=23, scale=0.8)
    T, scale = -(-L // 64), 1 / np.sqrt(d)
    g = np.random.default_rng(5)
    stride = T * T + 7
    offsets = torch.zeros(B, H, T + 1, dtype=torch.int32)
    idx = torch.full((B, H, stride), -1, dtype=torch.int32)
    lists = {}
    for b in range(B):
        for h in range(H):
            ks = g.integers(0, T + 1, T)
            ks[:3] = [0, T, 1]
            pos = 0
            for i in range(T):
                sel = np.sort(g.choice(T, size=int(ks[i]), replace=False))
                lists[(b, h, i)] = sel
                offsets[b, h, i] = pos
                idx[b, h, pos:pos + len(sel)] = torch.from_numpy(sel.astype(np.int32))
                pos += len(sel)
            offsets[b, h, T] = pos
    (qd, kd, vd), stats, _ = run_gpu(q, k, v, 1, 0.1)
    qn, kn, vn = (x.double().numpy() for x in (q, k, v))
    for mode, kw, okw in (("pisa", {}, {}), ("zeroth", {"first_order": False}, {"first_order": "none"}),
                          ("drop", {"drop_tail": True}, {"tail": False})):
        o = paro.attention_csr(qd, kd, vd, *stats[:3], offsets.cuda(), idx.cuda(), stride, **kw).float().cpu().numpy()
        for b in range(B):
            for h in range(H):
                st = pisa.block_stats(kn[b, h], vn[b, h], 64)
                rl = [lists[(b, h, i)] for i in range(T)]
                keep = [i for i in range(T) if mode != "drop" or len(rl[i]) > 0]
                ref = pisa.attention(qn[b, h], kn[b, h], vn[b, h], st, rl, scale, 64, qblocks=keep, **okw)
                rows = [r for i in keep for r in range(64 * i, min(64 * i + 64, L))]
                check_attention(o[b, h, rows], np.concatenate([ref[i] for i in keep]), dtype)
        log(f"[budget] csr random lists {dtype} {mode}: ok")


@pytest.mark.parametrize("total", ["one", "all"])
def test_budget_extremes(total):
    """The smallest and the largest total the ABI accepts (k_min = 0): one
    block in all (one row gets it, every other row is all tail), and T^2
    (every row keeps every block: dense attention). Sharing, lists and
    attention against the oracle."""
    w = WORKLOADS["tiny_fp32"]
    q, k, v = make_inputs(w, heads=[1])
    T = w.T
    K = 1 if total == "one" else T * T
    (qd, kd, vd), stats, _ = run_gpu(q, k, v, 1, w.lam)
    offsets, idx, wq = paro.route_budget(qd, stats[0], stats[3], K, 0, w.lam)
    offs_h, idx_h, wq_h = offsets.cpu().numpy()[0, 0], idx.cpu().numpy()[0, 0], wq.cpu().numpy()[0, 0]
    kk = np.diff(offs_h)
    qn, kn, vn = (x[0, 0].double().numpy() for x in (q, k, v))
    st = pisa.block_stats(kn, vn, 64)
    w_ref, k_or = _oracle_shares(qn, st, w.scale, K, 0)
    assert offs_h[0] == 0
    _check_shares(kk, wq_h, w_ref, k_or, K, 0)
    assert k_or.sum() == K
    assert k_or.max() == 1 if total == "one" else (k_or == T).all()
    ref_lists, score = budget.route_ragged(qn, st["kbar"], st["M"], k_or, w.lam, w.scale, 64)
    same = [i for i in range(T) if kk[i] == k_or[i]]
    _check_lists([idx_h[offs_h[i]:offs_h[i + 1]] for i in same], [ref_lists[i] for i in same], score[same])
    offs_or, idx_or = _csr(ref_lists, idx.shape[-1])
    o = paro.attention_csr(qd, kd, vd, *stats[:3], offs_or[None, None].cuda(), idx_or[None, None].cuda(),
                           K).float().cpu().numpy()[0, 0]
    oref = pisa.attention(qn, kn, vn, st, ref_lists, w.scale, 64)
    mx, mean = check_attention(o, oref, w.dtype)
    log(f"[budget] extremes {total}: k_i {kk.min()}..{kk.max()}, attention max {mx:.3g} mean {mean:.3g}")
    if total == "all":
        dense = pisa.dense_attention(qn, kn, vn, w.scale)
        assert np.abs(o - dense).max() < 1e-5
