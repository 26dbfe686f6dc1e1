"""GPU parity of the token reordering (paro_reorder) against the oracle's
tiled order: bit-exact row moves, and the whole PISA path run in tiled order
against the oracle run on the same reordered tokens."""
import numpy as np
import pytest
import torch

from block_sparse_attention_pisa_amd import paro
from oracle import pisa, reorder
from workloads import WORKLOADS, make_inputs, random_uniform_inputs

from parity_util import check_attention, check_route, check_stats, log, run_gpu

pytestmark = pytest.mark.gpu


def _bits(t: torch.Tensor) -> torch.Tensor:
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


@pytest.mark.parametrize("case", [
    dict(B=1, H=3, grid=(1, 64, 64), tile=(1, 8, 8), extra=512, d=128, dtype=torch.bfloat16),
    dict(B=2, H=9, grid=(3, 7, 11), tile=(2, 3, 4), extra=17, d=64, dtype=torch.float32),
    dict(B=1, H=5, grid=(5, 9, 13), tile=(4, 4, 4), extra=0, d=128, dtype=torch.float32),
    dict(B=1, H=8, grid=(21, 10, 16), tile=(2, 4, 8), extra=3, d=64, dtype=torch.bfloat16),
    dict(B=1, H=1, grid=(4, 4, 4), tile=(9, 9, 9), extra=0, d=128, dtype=torch.bfloat16),
    dict(B=1, H=2, grid=(2, 3, 5), tile=(1, 2, 2), extra=1, d=128, dtype=torch.bfloat16),
])
def test_reorder_bit_exact(case):
    grid, tile, extra = case["grid"], case["tile"], case["extra"]
    L = grid[0] * grid[1] * grid[2] + extra
    x, _, _ = random_uniform_inputs(case["B"], case["H"], L, case["d"], dtype=case["dtype"], seed=L)
    perm = torch.from_numpy(reorder.tiled_order(grid, tile, L=L))
    log(f"[reorder] {case['B']}x{case['H']}x{L}x{case['d']} {case['dtype']} grid {grid} tile {tile}")
    xd = x.cuda()
    y = paro.reorder(xd, grid, tile)
    z = paro.reorder(y, grid, tile, inverse=True)
    torch.cuda.synchronize()
    y, z = y.cpu(), z.cpu()
    assert torch.equal(_bits(y), _bits(x[:, :, perm]))
    assert torch.equal(_bits(z), _bits(x))
    # the scatter of an arbitrary tensor puts row i at perm[i]
    w = paro.reorder(xd, grid, tile, inverse=True).cpu()
    ref = torch.empty_like(x)
    ref[:, :, perm] = x
    assert torch.equal(_bits(w), _bits(ref))


def test_reorder_full_720p_bit_exact():
    """The 720p video shape at full size (40 heads), every row checked."""
    w = WORKLOADS["video720p_75600"]
    grid, tile = w.grid, (2, 4, 8)
    x, _, _ = random_uniform_inputs(1, w.H, w.L, w.d, dtype=torch.bfloat16, seed=5)
    perm = torch.from_numpy(reorder.tiled_order(grid, tile, L=w.L))
    log(f"[reorder] {w.name} full size, tile {tile}")
    y = paro.reorder(x.cuda(), grid, tile)
    torch.cuda.synchronize()
    assert torch.equal(_bits(y.cpu()), _bits(x[:, :, perm]))
    z = paro.reorder(y, grid, tile, inverse=True)
    torch.cuda.synchronize()
    assert torch.equal(_bits(z.cpu()), _bits(x))


@pytest.mark.parametrize("name,tile,heads", [
    ("image_4608", (1, 8, 8), [0, 7]),
    ("tiny_fp32", (2, 4, 8), [0, 1]),
])
def test_pisa_path_in_tiled_order(name, tile, heads):
    """Reorder on the GPU, run the three calls on the reordered tokens, move O
    back; the oracle runs on the same reordered tokens (its own permutation)
    and its O is moved back by the oracle's inverse. Attention takes the
    oracle's routing, as in the other parity tests."""
    w = WORKLOADS[name]
    q, k, v = make_inputs(w, heads=heads)
    perm = reorder.tiled_order(w.grid, tile, L=w.L)
    log(f"[reorder] path {name} tile {tile} heads {heads}")
    qd, kd, vd = (paro.reorder(t.cuda(), w.grid, tile) for t in (q, k, v))
    (qd, kd, vd), stats, idx = run_gpu(qd.cpu(), kd.cpu(), vd.cpu(), w.k, w.lam)
    for t, src in ((qd, q), (kd, k), (vd, v)):
        assert torch.equal(_bits(t.cpu()), _bits(src[:, :, torch.from_numpy(perm)]))
    qn, kn, vn = (reorder.apply_order(t.double().numpy(), perm) for t in (q, k, v))
    idx_h = idx.cpu().numpy()
    idx_or = torch.empty_like(idx.cpu())
    refs = []
    for hi in range(len(heads)):
        st = pisa.block_stats(kn[0, hi], vn[0, hi], w.block)
        ir, sc = pisa.route(qn[0, hi], st["kbar"], st["M"], w.k, w.lam, w.scale, w.block)
        check_stats(stats, st, 0, hi)
        check_route(idx_h[0, hi], ir, sc)
        idx_or[0, hi] = torch.from_numpy(ir.astype(np.int32))
        refs.append((st, ir))
    o_t = paro.attention(qd, kd, vd, stats[0], stats[1], stats[2], idx_or.cuda(), w.k)
    o = paro.reorder(o_t, w.grid, tile, inverse=True).float().cpu().numpy()
    for hi, (st, ir) in enumerate(refs):
        oref = pisa.attention(qn[0, hi], kn[0, hi], vn[0, hi], st, ir, w.scale, w.block)
        mx, mean = check_attention(o[0, hi], reorder.undo_order(oref, perm, axis=0), w.dtype)
        log(f"[reorder] path {name} head {heads[hi]}: max {mx:.3g} mean {mean:.3g}")
