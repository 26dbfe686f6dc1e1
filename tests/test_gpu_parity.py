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

from parity_util import (check_attention, check_route, check_stats, full_parity, log, run_gpu,
                         sample_qblocks)

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
    s = full_parity(w, heads=[(0, 0), (0, 39)], qblocks=lambda T: sample_qblocks(T, 12), diag=False)
    log("[parity] 720p summary", s)


def test_video_long_sampled():
    w = WORKLOADS["video_long_118800"]
    s = full_parity(w, heads=[(0, 23)], qblocks=lambda T: sample_qblocks(T, 8), diag=False)
    log("[parity] long summary", s)


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
