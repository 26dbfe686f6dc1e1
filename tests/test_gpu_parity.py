"""GPU parity: the HIP path through the C ABI against the fp64 oracle.

Small cases run whole; the DiT-sized workloads run the GPU over every head
and every query block (the launch configuration the benchmark times) and the
oracle checks sampled heads and query blocks.
"""
import numpy as np
import pytest
import torch

from block_sparse_attention_pisa_amd import paro
from oracle import pisa
from workloads import WORKLOADS, Workload, make_inputs, random_uniform_inputs

from parity_util import (M_ABS_TOL, check_attention, check_route, check_stats, full_parity, log, run_gpu,
                         sample_qblocks, to_dev)

pytestmark = pytest.mark.gpu


def test_tiny_fp32_whole_pipeline():
    s = full_parity(WORKLOADS["tiny_fp32"])
    assert s["max_err"] <= 1e-5


def test_image_4608_all_heads():
    w = WORKLOADS["image_4608"]
    s = full_parity(w, qblocks=lambda T: list(range(T)))
    log("[parity] image summary", s)


def test_video480p_sampled():
    w = WORKLOADS["video480p_32760"]
    s = full_parity(w, heads=[(0, 0), (0, 11)], qblocks=lambda T: sample_qblocks(T, 24))
    log("[parity] 480p summary", s)


def test_video720p_sampled():
    w = WORKLOADS["video720p_75600"]
    s = full_parity(w, heads=[(0, 0), (0, 13), (0, 26), (0, 39)], qblocks=lambda T: sample_qblocks(T, 48))
    log("[parity] 720p summary", s)


def test_video_long_sampled():
    w = WORKLOADS["video_long_118800"]
    s = full_parity(w, heads=[(0, 0), (0, 23)], qblocks=lambda T: sample_qblocks(T, 24))
    log("[parity] long summary", s)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_precompute_every_head_of_a_batch(dtype):
    """Precompute of B = 2 x H = 5 heads over 1700 blocks (ragged last
    block, 17,000 blocks in all): every head against the oracle, so a wrong
    (batch, head) offset anywhere in the three kernels fails, and two calls
    bitwise equal."""
    B, H, L, d = 2, 5, 64 * 1700 - 17, 64
    _, k, v = random_uniform_inputs(B, H, L, d, dtype=dtype, seed=31)
    kd, vd = to_dev(k, v)
    s1 = paro.precompute(kd, vd)
    s2 = paro.precompute(kd, vd)
    torch.cuda.synchronize()
    assert all(torch.equal(a, b) for a, b in zip(s1, s2))
    kn, vn = k.double().numpy(), v.double().numpy()
    worst = {}
    for b in range(B):
        for h in range(H):
            st = pisa.block_stats(kn[b, h], vn[b, h], 64)
            r = check_stats(s1, st, b, h)
            worst = {n: max(worst.get(n, 0.0), x) for n, x in r.items()}
    log("[parity] precompute, every head", dtype, worst)


def _spectral_bounds(k, v, block=64, iters=24, seed=5):
    """Lower and upper bounds on sigma_max(H_j - Hbar) for every block of one
    head, in fp64 on the CPU from the inputs (k, v: [L, d] float64 tensors):
    ||A x|| for x after `iters` power steps on A^T A from a seeded Gaussian
    start (never above sigma_max, and equal to it once converged), and the
    Frobenius norm (never below); plus kbar, vsum and Hbar by their
    definitions (mean and sum over a block's valid tokens, mean of the H_j)."""
    L, d = k.shape
    T = -(-L // block)
    pad = T * block - L
    z = torch.zeros(pad, d, dtype=torch.float64)
    kb = torch.cat([k, z]).reshape(T, block, d)
    vb = torch.cat([v, z]).reshape(T, block, d)
    n = torch.full((T,), block, dtype=torch.float64)
    n[-1] = block - pad
    valid = (torch.arange(block)[None, :] < n[:, None]).to(torch.float64)[:, :, None]
    kbar = kb.sum(dim=1) / n[:, None]
    H = torch.bmm(((kb - kbar[:, None, :]) * valid).transpose(1, 2).contiguous(), vb)
    A = H - H.mean(dim=0, keepdim=True)
    At = A.transpose(1, 2).contiguous()
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(T, d, 1, dtype=torch.float64, generator=g)
    for _ in range(iters):
        x = torch.bmm(At, torch.bmm(A, x))
        x = x / x.norm(dim=1, keepdim=True)
    lower = torch.bmm(A, x)[:, :, 0].norm(dim=1)
    upper = A.flatten(1).norm(dim=1)
    exact = {"kbar": kbar.numpy(), "vsum": vb.sum(dim=1).numpy(), "Hbar": H.mean(dim=0).numpy()}
    return lower.numpy(), upper.numpy(), exact


@pytest.mark.parametrize("name", ["image_4608", "video480p_32760", "video720p_75600", "video_long_118800"])
def test_spectral_norm_of_every_block_within_bounds(name):
    """At the full sizes, for every head: kbar, vsum and Hbar against their
    fp64 definitions (the bars of the sampled tests), and M_j of every block
    between a converged fp64 power-iteration estimate (a lower bound on
    sigma_max) and the Frobenius norm: a Lanczos run that settled on a lower
    singular value anywhere in the launch fails here, even in heads the
    sampled parity tests do not look at."""
    w = WORKLOADS[name]
    q, k, v = make_inputs(w)
    del q
    stats = paro.precompute(k.cuda(), v.cuda())
    M = stats[3].cpu().numpy()
    kbar, vsum, Hbar = (x.double().cpu().numpy() for x in stats[:3])
    tight = 0
    for h in range(w.H):
        lo, up, ex = _spectral_bounds(k[0, h].double(), v[0, h].double())
        for nm, got, tol in (("kbar", kbar[0, h], 2e-6), ("vsum", vsum[0, h], 2e-6), ("Hbar", Hbar[0, h], 2e-5)):
            rel = np.abs(got - ex[nm]).max() / np.abs(ex[nm]).max()
            assert rel < tol, (name, h, nm, rel)
        m = M[0, h]
        assert (m >= lo - M_ABS_TOL).all(), (name, h, int(np.argmax(lo - m)), float((lo - m).max()))
        assert (m <= up + M_ABS_TOL).all(), (name, h, int(np.argmax(m - up)))
        tight += int((np.abs(m - lo) <= M_ABS_TOL).sum())
    log(f"[parity] {name}: kbar, vsum, Hbar of all {w.H} heads; M within [power estimate, Frobenius] "
        f"for all {w.H * w.T} blocks; "
        f"{tight} within {M_ABS_TOL} of the power estimate")


@pytest.mark.parametrize("name", ["video720p_75600", "video_long_118800"])
def test_route_every_row_at_full_size(name):
    """The routing kernel as a unit, at the full sizes and in the launch
    configuration of the step: the workload's queries, kbar from its
    definition and a seeded synthetic M (any M is a valid input; the exact
    one needs an SVD per block), every row of every head against the
    oracle's top-k, differences excused only within the 1e-5 score gap."""
    w = WORKLOADS[name]
    q, k, _ = make_inputs(w)
    T, d = w.T, w.d
    kn = k[0].double()
    pad = T * 64 - w.L
    kb = torch.cat([kn, torch.zeros(w.H, pad, d, dtype=torch.float64)], dim=1).reshape(w.H, T, 64, d)
    n = torch.full((T,), 64.0, dtype=torch.float64)
    n[-1] = 64 - pad
    kbar = (kb.sum(dim=2) / n[None, :, None]).numpy()
    M = np.abs(np.random.default_rng(11).normal(300.0, 20.0, size=(w.H, T)))
    idx = paro.route(q.cuda(), torch.from_numpy(kbar).float()[None].cuda(), torch.from_numpy(M)[None].cuda(),
                     w.k, w.lam).cpu().numpy()
    excused = 0
    for h in range(w.H):
        # the kernel reads kbar in fp32: the oracle scores use the same rounded values
        kb32 = kbar[h].astype(np.float32).astype(np.float64)
        ir, sc = pisa.route(q[0, h].double().numpy(), kb32, M[h], w.k, w.lam, w.scale, 64)
        excused += check_route(idx[0, h], ir, sc)
    log(f"[parity] {name}: routing of all {w.H * T} rows, {excused} excused within the gap")


@pytest.mark.parametrize("fp8", [False, True])
def test_attention_every_head_at_full_size(fp8):
    """The attention kernel as a unit at 720p, every one of the 40 heads (the
    persistent grid spreads them over eight queues and all workgroups): a
    seeded synthetic routing (148 distinct blocks per row) fed to both
    sides, the first, the last and one seeded query block of each head
    against the exact oracle; also with the key-query products on the fp8
    matrix cores, held to the same bf16 bar."""
    w = WORKLOADS["video720p_75600"]
    q, k, v = make_inputs(w)
    T, kk = w.T, w.k
    g = np.random.default_rng(13)
    idx = np.sort(np.argsort(g.random((w.H, T, T), dtype=np.float32), axis=2)[:, :, :kk], axis=2).astype(np.int32)
    qd, kd, vd = to_dev(q, k, v)
    stats = paro.precompute(kd, vd)
    o = paro.attention(qd, kd, vd, *stats[:3], torch.from_numpy(idx)[None].cuda(), kk,
                       qk_fp8=fp8).float().cpu().numpy()
    worst = (0.0, 0.0)
    for h in range(w.H):
        qn, kn, vn = (x[0, h].double().numpy() for x in (q, k, v))
        st = pisa.block_stats(kn, vn, 64, spectral=False)
        qbs = sorted({0, T - 1, int(g.integers(1, T - 1))})
        ref = pisa.attention(qn, kn, vn, st, idx[h], w.scale, 64, qblocks=qbs)
        for i in qbs:
            rows = slice(64 * i, min(64 * i + 64, w.L))
            mx, mean = check_attention(o[0, h, rows], ref[i], "bf16")
            worst = (max(worst[0], mx), max(worst[1], mean))
    log(f"[parity] 720p attention{' (fp8 key-query)' if fp8 else ''}, 3 query blocks of every head, "
        f"synthetic routing: max {worst[0]:.3g} "
        f"mean {worst[1]:.3g}")


def test_long_dense_control_equals_softmax_attention():
    """keep = 100%: the path must reduce to plain softmax attention."""
    w = WORKLOADS["video_long_118800_dense"]
    q, k, v = make_inputs(w, heads=[3])   # one head at full length
    (qd, kd, vd), stats, idx = run_gpu(q, k, v, w.k, w.lam)
    assert (idx.cpu() == torch.arange(w.T, dtype=torch.int32)).all()
    o = paro.attention(qd, kd, vd, *stats[:3], idx, w.k).float().cpu().numpy()[0, 0]
    qn, kn, vn = (x[0, 0].double().numpy() for x in (q, k, v))
    rows = np.concatenate([np.arange(0, 64), np.arange(60000, 60064), np.arange(w.L - 16, w.L)])
    dense = pisa.dense_attention(qn, kn, vn, w.scale, rows=rows)
    mx, mean = check_attention(o[rows], dense, "bf16")
    log(f"[parity] dense control max {mx:.3g} mean {mean:.3g}")


@pytest.mark.parametrize("case", [
    dict(L=37, d=128, keep=1, H=1, B=1),            # one partial block
    dict(L=64, d=128, keep=0, H=2, B=1),            # keep 0: everything in the tail
    dict(L=64 * 7 + 5, d=128, keep=8, H=1, B=2),    # keep = T: dense
    dict(L=64 * 9 - 17, d=64, keep=3, H=3, B=1),    # d = 64, ragged tail
    dict(L=64 * 40 + 1, d=128, keep=5, H=2, B=2),   # last block of one token
])
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_edge_shapes(case, dtype):
    B, H, L, d, keep = case["B"], case["H"], case["L"], case["d"], case["keep"]
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    q, k, v = random_uniform_inputs(B, H, L, d, dtype=tdt, seed=L + d, scale=0.8)
    lam, scale = 0.1, 1 / np.sqrt(d)
    (qd, kd, vd), stats, idx = run_gpu(q, k, v, keep, lam)
    qn, kn, vn = (x.double().numpy() for x in (q, k, v))
    idx_h = idx.cpu().numpy()
    idx_or = torch.empty_like(idx.cpu())
    refs = {}
    for b in range(B):
        for h in range(H):
            st = pisa.block_stats(kn[b, h], vn[b, h], 64)
            ir, sc = pisa.route(qn[b, h], st["kbar"], st["M"], keep, lam, scale, 64)
            check_stats(stats, st, b, h)
            if keep:
                check_route(idx_h[b, h], ir, sc)
            idx_or[b, h] = torch.from_numpy(ir.astype(np.int32))
            refs[(b, h)] = (st, ir)
    o = paro.attention(qd, kd, vd, *stats[:3], idx_or.cuda(), keep).float().cpu().numpy()
    for (b, h), (st, ir) in refs.items():
        oref = pisa.attention(qn[b, h], kn[b, h], vn[b, h], st, ir, scale, 64)
        check_attention(o[b, h], oref, dtype)


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("fp32", 64)])
def test_custom_scale_and_negative_lambda(dtype, d):
    """A softmax scale other than 1/sqrt(d) (it enters the routing score,
    the exact logits, the tail logits and the correction) and a negative
    lambda (routing then prefers blocks of small M_j): statistics, every
    routing row and every query block against the oracle."""
    B, H, L, keep, lam, scale = 1, 2, 64 * 150 + 9, 20, -0.3, 0.05
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    q, k, v = random_uniform_inputs(B, H, L, d, dtype=tdt, seed=77, scale=0.8)
    (qd, kd, vd), stats, idx = run_gpu(q, k, v, keep, lam, scale=scale)
    qn, kn, vn = (x.double().numpy() for x in (q, k, v))
    idx_h = idx.cpu().numpy()
    idx_or = torch.empty_like(idx.cpu())
    refs = {}
    for b in range(B):
        for h in range(H):
            st = pisa.block_stats(kn[b, h], vn[b, h], 64)
            ir, sc = pisa.route(qn[b, h], st["kbar"], st["M"], keep, lam, scale, 64)
            check_stats(stats, st, b, h)
            check_route(idx_h[b, h], ir, sc)
            idx_or[b, h] = torch.from_numpy(ir.astype(np.int32))
            refs[(b, h)] = (st, ir)
    o = paro.attention(qd, kd, vd, *stats[:3], idx_or.cuda(), keep, scale=scale).float().cpu().numpy()
    worst = 0.0
    for (b, h), (st, ir) in refs.items():
        oref = pisa.attention(qn[b, h], kn[b, h], vn[b, h], st, ir, scale, 64)
        mx, mean = check_attention(o[b, h], oref, dtype)
        worst = max(worst, mx)
        log(f"[parity] scale {scale} lambda {lam} {dtype} d={d} head {h}: max {mx:.3g} mean {mean:.3g}")
    # the scale is used: the same call at the default 1/sqrt(d) lands far
    # outside the error this one has against its reference
    o_def = paro.attention(qd, kd, vd, *stats[:3], idx_or.cuda(), keep).float().cpu().numpy()
    assert np.abs(o_def - o).max() > 10 * worst


@pytest.mark.parametrize("case", [
    dict(B=1, H=2, L=64 * 300 + 11, d=64, keep=30, lam=0.1),     # d = 64 over many tiles, ragged tail
    dict(B=2, H=1, L=64 * 600 - 5, d=128, keep=599, lam=0.1),    # keep = T - 1: one tail block per row
    dict(B=1, H=1, L=64 * 200, d=128, keep=25, lam=0.0),         # lambda = 0: routing by q-bar . k-bar alone
    dict(B=1, H=1, L=64 * 200, d=128, keep=25, lam=5.0),         # large lambda: routing by M_j mostly
])
def test_medium_shapes(case):
    """Stats and routing of every row, attention on sampled query blocks, at
    sizes between the edge cases and the DiT workloads."""
    B, H, L, d, keep, lam = (case[x] for x in ("B", "H", "L", "d", "keep", "lam"))
    q, k, v = random_uniform_inputs(B, H, L, d, dtype=torch.bfloat16, seed=L + keep, scale=0.8)
    scale = 1 / np.sqrt(d)
    (qd, kd, vd), stats, idx = run_gpu(q, k, v, keep, lam)
    qn, kn, vn = (x.double().numpy() for x in (q, k, v))
    idx_h = idx.cpu().numpy()
    idx_or = torch.empty_like(idx.cpu())
    refs = {}
    for b in range(B):
        for h in range(H):
            st = pisa.block_stats(kn[b, h], vn[b, h], 64)
            ir, sc = pisa.route(qn[b, h], st["kbar"], st["M"], keep, lam, scale, 64)
            check_stats(stats, st, b, h)
            ex = check_route(idx_h[b, h], ir, sc)
            log(f"[parity] medium {case} b{b}h{h}: excused routing rows {ex}")
            idx_or[b, h] = torch.from_numpy(ir.astype(np.int32))
            refs[(b, h)] = (st, ir)
    o = paro.attention(qd, kd, vd, *stats[:3], idx_or.cuda(), keep).float().cpu().numpy()
    rng_ = pisa.block_ranges(L, 64)
    for (b, h), (st, ir) in refs.items():
        qbs = sample_qblocks(len(rng_), 8)
        oref = pisa.attention(qn[b, h], kn[b, h], vn[b, h], st, ir, scale, 64, qblocks=qbs)
        og = np.concatenate([o[b, h, rng_[i][0]:rng_[i][1]] for i in qbs])
        orr = np.concatenate([oref[i] for i in qbs])
        check_attention(og, orr, "bf16")


@pytest.mark.parametrize("case", ["image_4608", "ragged_d64", "tiny_fp32"])
def test_drop_tail_mode_is_keep_or_drop_attention(case):
    """PARO_TAIL_DROP: stages 2 and 3 off, softmax renormalised over S_i (the
    oracle's tail=False mode), fed the oracle's routing."""
    if case == "ragged_d64":
        B, H, L, d, keep = 1, 2, 64 * 9 - 17, 64, 3
        q, k, v = random_uniform_inputs(B, H, L, d, dtype=torch.bfloat16, seed=91, scale=0.8)
        dtype, scale = "bf16", 1 / np.sqrt(d)
    else:
        w = WORKLOADS[case]
        q, k, v = make_inputs(w)
        B, H, L, keep, dtype, scale = w.B, w.H, w.L, w.k, w.dtype, w.scale
    (qd, kd, vd), stats, _ = run_gpu(q, k, v, keep, 0.1)
    qn, kn, vn = (x.double().numpy() for x in (q, k, v))
    idx_or = torch.empty(B, H, -(-L // 64), keep, dtype=torch.int32)
    refs = {}
    for b in range(B):
        for h in range(H):
            st = pisa.block_stats(kn[b, h], vn[b, h], 64)
            ir, _ = pisa.route(qn[b, h], st["kbar"], st["M"], keep, 0.1, scale, 64)
            idx_or[b, h] = torch.from_numpy(ir.astype(np.int32))
            refs[(b, h)] = (st, ir)
    o = paro.attention(qd, kd, vd, *stats[:3], idx_or.cuda(), keep, drop_tail=True).float().cpu().numpy()
    for (b, h), (st, ir) in refs.items():
        oref = pisa.attention(qn[b, h], kn[b, h], vn[b, h], st, ir, scale, 64, tail=False)
        check_attention(o[b, h], oref, dtype)


@pytest.mark.parametrize("case", ["image_4608", "tiny_fp32"])
def test_zeroth_order_mode(case):
    """PARO_TAIL_ZEROTH: stages 1 and 2 without the first-order correction
    (the oracle's first_order="none" mode); it must differ from the method
    by the correction term."""
    w = WORKLOADS[case]
    q, k, v = make_inputs(w)
    (qd, kd, vd), stats, _ = run_gpu(q, k, v, w.k, w.lam)
    qn, kn, vn = (x.double().numpy() for x in (q, k, v))
    idx_or = torch.empty(w.B, w.H, w.T, w.k, dtype=torch.int32)
    refs = {}
    for b in range(w.B):
        for h in range(w.H):
            st = pisa.block_stats(kn[b, h], vn[b, h], 64)
            ir, _ = pisa.route(qn[b, h], st["kbar"], st["M"], w.k, w.lam, w.scale, 64)
            idx_or[b, h] = torch.from_numpy(ir.astype(np.int32))
            refs[(b, h)] = (st, ir)
    o0 = paro.attention(qd, kd, vd, *stats[:3], idx_or.cuda(), w.k, first_order=False).float().cpu().numpy()
    o1 = paro.attention(qd, kd, vd, *stats[:3], idx_or.cuda(), w.k).float().cpu().numpy()
    for (b, h), (st, ir) in refs.items():
        oref = pisa.attention(qn[b, h], kn[b, h], vn[b, h], st, ir, w.scale, 64, first_order="none")
        check_attention(o0[b, h], oref, w.dtype)
    assert np.abs(o1 - o0).max() > 0.0


def test_rows_past_L_are_not_written():
    """The output is written only for the L valid rows (bytes after it stay untouched)."""
    B, H, L, d = 1, 1, 64 * 3 - 10, 128
    q, k, v = random_uniform_inputs(B, H, L, d, dtype=torch.bfloat16, seed=5)
    qd, kd, vd = (x.cuda() for x in (q, k, v))
    stats = paro.precompute(kd, vd)
    idx = paro.route(qd, stats[0], stats[3], 1, 0.1)
    o = paro.attention(qd, kd, vd, *stats[:3], idx, 1)
    n = B * H * L * d
    buf = torch.full((n + 4096,), 7.0, dtype=torch.bfloat16, device="cuda")
    ov = buf[:n].view(B, H, L, d)
    paro.attention(qd, kd, vd, *stats[:3], idx, 1, out=ov)
    torch.cuda.synchronize()
    assert torch.isfinite(o.float()).all()
    assert (buf[n:] == 7.0).all()
    assert torch.equal(ov, o)


def test_deterministic_bitwise():
    w = WORKLOADS["image_4608"]
    q, k, v = make_inputs(w, heads=[0, 1, 2, 3])
    outs = []
    for _ in range(2):
        (qd, kd, vd), stats, idx = run_gpu(q, k, v, w.k, w.lam)
        o = paro.attention(qd, kd, vd, *stats[:3], idx, w.k)
        torch.cuda.synchronize()
        outs.append([x.cpu() for x in (*stats, idx, o)])
    for a, b in zip(*outs):
        assert torch.equal(a, b)


@pytest.mark.parametrize("keep", [1, 5, 11])
def test_route_exact_ties_and_equal_scores(keep):
    """Duplicated kv blocks tie exactly (lower block index wins); constant keys
    and values make every score equal (the first keep blocks win)."""
    d, nb = 128, 13
    g = np.random.default_rng(keep)
    base = torch.from_numpy(g.standard_normal((4, 64, d)).astype(np.float32))
    order = [0, 1, 0, 2, 3, 1, 2, 0, 3, 3, 1, 2, 0]
    k = torch.cat([base[i] for i in order])[None, None].to(torch.bfloat16)
    v = torch.cat([base[(i + 1) % 4] for i in order])[None, None].to(torch.bfloat16)
    q = torch.from_numpy(g.standard_normal((1, 1, 64 * nb, d)).astype(np.float32)).to(torch.bfloat16)
    for kk, vv in ((k, v), (torch.ones_like(k), torch.ones_like(v))):
        (qd, kd, vd), stats, idx = run_gpu(q, kk, vv, keep, 0.1)
        qn, kn, vn = (x[0, 0].double().numpy() for x in (q, kk, vv))
        st = pisa.block_stats(kn, vn, 64)
        ir, sc = pisa.route(qn, st["kbar"], st["M"], keep, 0.1, 1 / np.sqrt(d), 64)
        assert (idx.cpu().numpy()[0, 0] == ir).all()


@pytest.mark.parametrize("keep", [37, 300, 560])
def test_route_ties_through_the_gathered_search(keep):
    """T = 601 kv blocks made of 15 distinct blocks repeated about 40 times
    each in a shuffled order: every row has tie groups of ~40 exactly equal
    scores, so the threshold search narrows to a few hundred candidate keys
    (gathered into a few registers per lane through the row's LDS slice of
    dots, which for odd T starts 4 bytes into the slice on every other row)
    and then runs out of bits inside a tie, where the lower block indices
    must win."""
    d, nb, nd = 64, 601, 15
    g = np.random.default_rng(keep)
    base = torch.from_numpy(g.standard_normal((nd, 64, d)).astype(np.float32))
    order = g.permutation(np.arange(nb) % nd)
    L = 64 * nb - 17
    k = torch.cat([base[i] for i in order])[:L][None, None].to(torch.bfloat16)
    v = torch.cat([base[(i + 3) % nd] for i in order])[:L][None, None].to(torch.bfloat16)
    q = torch.from_numpy(g.standard_normal((1, 1, L, d)).astype(np.float32)).to(torch.bfloat16)
    (qd, kd, vd), stats, idx = run_gpu(q, k, v, keep, 0.1)
    qn, kn, vn = (x[0, 0].double().numpy() for x in (q, k, v))
    st = pisa.block_stats(kn, vn, 64)
    ir, sc = pisa.route(qn, st["kbar"], st["M"], keep, 0.1, 1 / np.sqrt(d), 64)
    ig = idx.cpu().numpy()[0, 0]
    check_route(ig, ir, sc)
    # the duplicated full blocks tie exactly on the GPU too: within a row, a
    # taken copy of a block means every lower-indexed copy is taken as well
    full = order[: nb - 1]
    for i in range(0, nb, 7):
        taken = set(ig[i].tolist())
        for blk in range(nd):
            copies = [j for j in range(nb - 1) if full[j] == blk]
            flags = [j in taken for j in copies]
            assert flags == sorted(flags, reverse=True), (i, blk)


@pytest.mark.parametrize("keep", [300, 2060])
def test_route_rows_longer_than_register_keys(keep):
    """T = 2100 > 2048 kv blocks: the keys past the first 2048 of a row are
    re-formed each time they are counted. Random keys check the threshold
    search across that boundary; constant keys (every score equal) check that
    the first keep blocks in ascending j win across it."""
    B, H, T, d = 1, 1, 2100, 64
    L = 64 * T - 30
    q, k, v = random_uniform_inputs(B, H, L, d, dtype=torch.bfloat16, seed=keep, scale=0.8)
    lam, scale = 0.1, 1 / np.sqrt(d)
    for kk, vv in ((k, v), (torch.ones_like(k), torch.ones_like(v))):
        (qd, kd, vd), stats, idx = run_gpu(q, kk, vv, keep, lam)
        qn, kn, vn = (x[0, 0].double().numpy() for x in (q, kk, vv))
        st = pisa.block_stats(kn, vn, 64)
        ir, sc = pisa.route(qn, st["kbar"], st["M"], keep, lam, scale, 64)
        check_route(idx.cpu().numpy()[0, 0], ir, sc)


def test_logit_jump_rerun_keeps_every_row_exact():
    """A kv block whose logits sit ~88 nats above the first tile's forces the
    kernel's rerun path for the query blocks that list it; the other blocks of
    the same workgroup must keep their own results."""
    B, H, d, nb = 1, 1, 128, 8
    L = 64 * nb
    g = np.random.default_rng(7)
    e0 = np.zeros(d, dtype=np.float32)
    e0[0] = 1.0
    q = (0.1 * g.standard_normal((L, d)) + e0).astype(np.float32)
    k = (0.5 * g.standard_normal((L, d))).astype(np.float32)
    k[5 * 64:6 * 64] = 1000.0 * e0 + 0.5 * g.standard_normal((64, d))
    v = g.standard_normal((L, d)).astype(np.float32)
    qt, kt, vt = (torch.from_numpy(x)[None, None].to(torch.bfloat16) for x in (q, k, v))
    idx = np.array([[0, 5], [0, 5], [0, 1], [0, 1], [0, 5], [2, 3], [1, 5], [0, 7]], dtype=np.int32)
    qd, kd, vd = (x.cuda() for x in (qt, kt, vt))
    stats = paro.precompute(kd, vd)
    o = paro.attention(qd, kd, vd, *stats[:3], torch.from_numpy(idx)[None, None].cuda(), 2).float().cpu().numpy()
    qn, kn, vn = (x[0, 0].double().numpy() for x in (qt, kt, vt))
    st = pisa.block_stats(kn, vn, 64)
    ref = pisa.attention(qn, kn, vn, st, idx.astype(np.int64), 1 / np.sqrt(d), 64)
    assert np.isfinite(o).all()
    check_attention(o[0, 0], ref, "bf16")


def _drop_mode_case(q, k, v, idx, fp8):
    """GPU keep-or-drop attention (the tail dropped) on the given rows against
    the oracle's tail=False mode; for the fp8 path the oracle runs on the
    e4m3-rounded operands."""
    from parity_util import fp8_operands
    d = q.shape[-1]
    scale = 1 / np.sqrt(d)
    qt, kt, vt = (torch.from_numpy(x)[None, None].to(torch.bfloat16) for x in (q, k, v))
    qd, kd, vd = (x.cuda() for x in (qt, kt, vt))
    stats = paro.precompute(kd, vd)
    keep = idx.shape[1]
    o = paro.attention(qd, kd, vd, *stats[:3], torch.from_numpy(idx)[None, None].cuda(), keep, drop_tail=True,
                       qk_fp8=fp8).float().cpu().numpy()[0, 0]
    qn, kn, vn = (x[0, 0].double().numpy() for x in (qt, kt, vt))
    st = pisa.block_stats(kn, vn, 64)
    if fp8:
        qn, kn, st = fp8_operands(qt[0, 0], kt[0, 0], st["kbar"], st, scale)
    ref = pisa.attention(qn, kn, vn, st, idx.astype(np.int64), scale, 64, tail=False)
    assert np.isfinite(o).all()
    return check_attention(o, ref, "bf16")


@pytest.mark.parametrize("jump", [1000.0, 2000.0])
@pytest.mark.parametrize("fp8", [False, True])
def test_drop_mode_with_a_dropped_block_far_above_the_kept_ones(jump, fp8):
    """Keep-or-drop: block 5's logits sit ~88 (jump 1000) or ~177 (jump 2000)
    nats above every other block's, and the rows with S_i = {0, 1}, {2, 3} or
    {0, 7} leave it out. The softmax reference must come from blocks that
    carry weight only: taken over all centroids of the first chunk, every
    weight of those rows would underflow (exp2 of about -127 or -255) and
    D would be 0."""
    d, nb = 128, 8
    L = 64 * nb
    g = np.random.default_rng(7)
    e0 = np.zeros(d, dtype=np.float32)
    e0[0] = 1.0
    q = (0.1 * g.standard_normal((L, d)) + e0).astype(np.float32)
    k = (0.5 * g.standard_normal((L, d))).astype(np.float32)
    k[5 * 64:6 * 64] = jump * e0 + 0.5 * g.standard_normal((64, d))
    v = g.standard_normal((L, d)).astype(np.float32)
    idx = np.array([[0, 5], [0, 5], [0, 1], [0, 1], [0, 5], [2, 3], [1, 5], [0, 7]], dtype=np.int32)
    mx, mean = _drop_mode_case(q, k, v, idx, fp8)
    log(f"[parity] drop mode, jump {jump}, fp8 {fp8}: max {mx:.3g} mean {mean:.3g}")


@pytest.mark.parametrize("fp8", [False, True])
def test_drop_mode_with_all_logits_far_below_zero(fp8):
    """Keep-or-drop with T = 66 blocks and every logit about -133 nats: rows
    whose S_i has no block in the first centroid chunk (blocks 64 and 65, the
    last one partial) start from the reference 0, so every weight underflows;
    such a row must be caught (D below 2^-64) and recomputed with its exact
    maximum. Rows with a block of the first chunk take their reference from it."""
    d, nb = 128, 66
    L = 64 * nb - 5
    g = np.random.default_rng(9)
    e0 = np.zeros(d, dtype=np.float32)
    e0[0] = 1.0
    q = (0.1 * g.standard_normal((L, d)) + e0).astype(np.float32)
    k = (-1500.0 * e0 + 0.5 * g.standard_normal((L, d))).astype(np.float32)
    v = g.standard_normal((L, d)).astype(np.float32)
    idx = np.array([[64, 65] if i % 2 == 0 else [3, 64] for i in range(nb)], dtype=np.int32)
    mx, mean = _drop_mode_case(q, k, v, idx, fp8)
    log(f"[parity] drop mode, logits far below zero, fp8 {fp8}: max {mx:.3g} mean {mean:.3g}")
