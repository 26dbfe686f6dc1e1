"""GPU checks of the fp8 key-query path (paro_attention_fp8, paro_fp8_rows).

The e4m3 row codes and scales are an integer result of floating point, so
they are compared bit for bit with the CPU quantiser (oracle/quant.py), both
sides rounding the same fp32 values.

The attention output approximates the method: its logits carry e4m3
rounding of q' and k (relative 2^-4 per factor). Two bars:
  * on the DiT workloads, against the exact fp64 oracle at the bf16 bar
    (max 1e-2, mean 1e-3), which the fp8 path meets there;
  * on every shape, against the fp64 oracle applied to the e4m3-rounded
    operands (q' per query row, K and the oracle's own kbar per row, rounded
    exactly as the kernel rounds them), i.e. the definition of what the fp8
    path computes, at the same bf16 bar; on the DiT workloads that
    definition must also sit within a tenth of the smallest gap between
    PISA and dense, zeroth-order or keep-or-drop attention. (Small iid inputs with a few dozen keys do not
    average the e4m3 error out; against the exact oracle they miss the bf16
    bar by design.)
Attention is always fed the oracle's routing.
"""
import numpy as np
import pytest
import torch

from block_sparse_attention_pisa_amd import paro
from oracle import pisa, quant
from workloads import WORKLOADS, random_uniform_inputs

from parity_util import check_attention, fp8_operands, full_parity, log, run_gpu, sample_qblocks

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype,d", [(torch.bfloat16, 128), (torch.bfloat16, 64), (torch.float32, 128),
                                     (torch.float32, 64)])
def test_fp8_rows_bit_exact(dtype, d):
    g = np.random.default_rng(d + (1 if dtype == torch.float32 else 0))
    n = 777
    x = g.standard_normal((n, d)) * 10.0 ** g.uniform(-4, 4, (n, 1))
    x[5] = 0.0
    x[6] = 448.0
    x[7, 3] = -449.0
    x[8] = 2.0 ** -130  # a row of fp32 subnormal-range magnitudes (exactly 0 in bf16)
    xt = torch.from_numpy(x.astype(np.float32)).to(dtype)
    log(f"[fp8] rows {n}x{d} {dtype}")
    codes, sc = paro.fp8_rows(xt.cuda())
    torch.cuda.synchronize()
    ref_c, ref_s = quant.quantize_rows(xt.float().numpy())
    assert np.array_equal(sc.cpu().numpy(), ref_s)
    assert np.array_equal(codes.cpu().numpy(), ref_c)


def test_fp8_image_4608_all_heads():
    s = full_parity(WORKLOADS["image_4608"], qblocks=lambda T: list(range(T)), qk_fp8=True)
    log("[fp8] image summary", s)


def test_fp8_video480p_sampled():
    w = WORKLOADS["video480p_32760"]
    s = full_parity(w, heads=[(0, 0), (0, 11)], qblocks=lambda T: sample_qblocks(T, 24), qk_fp8=True)
    log("[fp8] 480p summary", s)


def test_fp8_video720p_sampled():
    w = WORKLOADS["video720p_75600"]
    s = full_parity(w, heads=[(0, 0), (0, 20), (0, 39)], qblocks=lambda T: sample_qblocks(T, 48), qk_fp8=True)
    log("[fp8] 720p summary", s)


@pytest.mark.parametrize("case", [
    dict(L=37, d=128, keep=1, H=1, B=1),            # one partial block
    dict(L=64, d=128, keep=0, H=2, B=1),            # keep 0: everything in the tail
    dict(L=64 * 7 + 5, d=128, keep=8, H=1, B=2),    # keep = T: dense
    dict(L=64 * 9 - 17, d=64, keep=3, H=3, B=1),    # d = 64, ragged tail
    dict(L=64 * 40 + 1, d=128, keep=5, H=2, B=2),   # last block of one token
])
@pytest.mark.parametrize("mode", ["pisa", "zeroth", "drop"])
def test_fp8_edge_shapes(case, mode):
    B, H, L, d, keep = case["B"], case["H"], case["L"], case["d"], case["keep"]
    drop = mode == "drop"
    if drop and keep == 0:
        pytest.skip("no exact block and the tail dropped: every output is 0/0 (NaN) by definition")
    q, k, v = random_uniform_inputs(B, H, L, d, dtype=torch.bfloat16, seed=L + d, scale=0.8)
    scale = 1 / np.sqrt(d)
    log(f"[fp8] edge {case} mode={mode}")
    (qd, kd, vd), stats, idx = run_gpu(q, k, v, keep, 0.1)
    qn, kn, vn = (x.double().numpy() for x in (q, k, v))
    idx_or = torch.empty_like(idx.cpu())
    refs = {}
    for b in range(B):
        for h in range(H):
            st = pisa.block_stats(kn[b, h], vn[b, h], 64)
            ir, _ = pisa.route(qn[b, h], st["kbar"], st["M"], keep, 0.1, scale, 64)
            idx_or[b, h] = torch.from_numpy(ir.astype(np.int32))
            refs[(b, h)] = (st, ir)
    o = paro.attention(qd, kd, vd, *stats[:3], idx_or.cuda(), keep, drop_tail=drop,
                       first_order=mode != "zeroth", qk_fp8=True)
    o = o.float().cpu().numpy()
    for (b, h), (st, ir) in refs.items():
        qq, kq, stq = fp8_operands(q[b, h], k[b, h], st["kbar"], st, scale)
        oref = pisa.attention(qq, kq, vn[b, h], stq, ir, scale, 64, tail=not drop,
                              first_order="none" if mode == "zeroth" else "global")
        mx, mean = check_attention(o[b, h], oref, "bf16")
        log(f"[fp8] edge b{b}h{h} vs the oracle on e4m3 operands: max {mx:.3g} mean {mean:.3g}")


@pytest.mark.parametrize("case", [
    dict(B=1, H=2, L=64 * 300 + 11, d=64, keep=30),    # d = 64 over many tiles (scale bytes loaded by waves 4-7)
    dict(B=2, H=1, L=64 * 600 - 5, d=128, keep=40),    # 300 items: more than one per persistent workgroup
])
def test_fp8_medium_shapes(case):
    """The fp8 path at sizes between the edge cases and the DiT workloads,
    on sampled query blocks, against the oracle on the e4m3-rounded operands."""
    B, H, L, d, keep = (case[x] for x in ("B", "H", "L", "d", "keep"))
    q, k, v = random_uniform_inputs(B, H, L, d, dtype=torch.bfloat16, seed=L + keep, scale=0.8)
    scale = 1 / np.sqrt(d)
    log(f"[fp8] medium {case}")
    (qd, kd, vd), stats, idx = run_gpu(q, k, v, keep, 0.1)
    qn, kn, vn = (x.double().numpy() for x in (q, k, v))
    idx_or = torch.empty_like(idx.cpu())
    refs = {}
    for b in range(B):
        for h in range(H):
            st = pisa.block_stats(kn[b, h], vn[b, h], 64)
            ir, _ = pisa.route(qn[b, h], st["kbar"], st["M"], keep, 0.1, scale, 64)
            idx_or[b, h] = torch.from_numpy(ir.astype(np.int32))
            refs[(b, h)] = (st, ir)
    o = paro.attention(qd, kd, vd, *stats[:3], idx_or.cuda(), keep, qk_fp8=True).float().cpu().numpy()
    rng_ = pisa.block_ranges(L, 64)
    for (b, h), (st, ir) in refs.items():
        qbs = sample_qblocks(len(rng_), 8)
        qq, kq, stq = fp8_operands(q[b, h], k[b, h], st["kbar"], st, scale)
        oref = pisa.attention(qq, kq, vn[b, h], stq, ir, scale, 64, qblocks=qbs)
        og = np.concatenate([o[b, h, rng_[i][0]:rng_[i][1]] for i in qbs])
        orr = np.concatenate([oref[i] for i in qbs])
        mx, mean = check_attention(og, orr, "bf16")
        log(f"[fp8] medium b{b}h{h} vs the oracle on e4m3 operands: max {mx:.3g} mean {mean:.3g}")


def test_fp8_rejects_fp32():
    q = torch.zeros(1, 1, 64, 64, device="cuda")
    stats = paro.precompute(q, q)
    idx = torch.zeros(1, 1, 1, 1, dtype=torch.int32, device="cuda")
    with pytest.raises(paro.ParoError):
        paro.attention(q, q, q, *stats[:3], idx, 1, qk_fp8=True)
