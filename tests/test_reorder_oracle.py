"""Pins of the token-order oracle (CPU only).

The order is the tiled raster order read from "PAROAttention: Pattern-Aware
ReOrdering for Efficient Sparse and Quantized Attention in Visual Generation
Models" (abstract: reorder tokens so visual attention becomes block-wise).
Pins: small orders worked out by hand, bijection, the cases that reduce to
the identity, the box property of full tiles, the place of tokens after the
grid, and the permutation equivariance of dense softmax attention.
"""

import math

import numpy as np
import pytest

from oracle import pisa, reorder


def test_hand_worked_orders():
    # 4x4 image, 2x2 tiles: boxes in raster order, tokens of a box in raster order
    assert reorder.tiled_order((1, 4, 4), (1, 2, 2)).tolist() == [
        0, 1, 4, 5, 2, 3, 6, 7, 8, 9, 12, 13, 10, 11, 14, 15]
    # 3x5 image, 2x2 tiles: the right column and the bottom row are cut short
    assert reorder.tiled_order((1, 3, 5), (1, 2, 2)).tolist() == [
        0, 1, 5, 6, 2, 3, 7, 8, 4, 9, 10, 11, 12, 13, 14]
    # 2x2x2 video, tiles spanning both frames: (t, y, x) -> 4t + 2y + x
    assert reorder.tiled_order((2, 2, 2), (2, 1, 2)).tolist() == [0, 1, 4, 5, 2, 3, 6, 7]
    # three text tokens after a 2x2 image keep their places
    assert reorder.tiled_order((1, 2, 2), (1, 1, 2), L=7).tolist() == [0, 1, 2, 3, 4, 5, 6]
    assert reorder.tiled_order((1, 2, 2), (1, 2, 1), L=7).tolist() == [0, 2, 1, 3, 4, 5, 6]


@pytest.mark.parametrize("grid,tile,extra", [
    ((3, 7, 11), (2, 3, 4), 0), ((5, 9, 13), (4, 4, 4), 17), ((1, 33, 20), (1, 8, 8), 64),
    ((21, 10, 16), (2, 4, 8), 3), ((4, 4, 4), (9, 9, 9), 0), ((2, 5, 3), (1, 1, 1), 5),
])
def test_order_is_a_permutation(grid, tile, extra):
    N = grid[0] * grid[1] * grid[2]
    p = reorder.tiled_order(grid, tile, L=N + extra)
    assert sorted(p.tolist()) == list(range(N + extra))
    assert p[N:].tolist() == list(range(N, N + extra))


@pytest.mark.parametrize("grid", [(3, 5, 7), (1, 8, 8), (4, 1, 9)])
def test_identity_cases(grid):
    N = grid[0] * grid[1] * grid[2]
    ident = list(range(N))
    assert reorder.tiled_order(grid, (1, 1, 1)).tolist() == ident
    assert reorder.tiled_order(grid, (1, 1, grid[2])).tolist() == ident    # whole rows
    assert reorder.tiled_order(grid, (1, grid[1], grid[2])).tolist() == ident  # whole frames
    assert reorder.tiled_order(grid, grid).tolist() == ident
    assert reorder.tiled_order(grid, (50, 50, 50)).tolist() == ident


@pytest.mark.parametrize("grid,tile", [((4, 8, 16), (2, 4, 8)), ((8, 8, 8), (4, 4, 4)), ((1, 16, 24), (1, 8, 8))])
def test_full_tiles_are_aligned_boxes(grid, tile):
    Gt, Gy, Gx = grid
    vol = tile[0] * tile[1] * tile[2]
    p = reorder.tiled_order(grid, tile)
    coords = np.stack(np.unravel_index(p, grid), axis=1)
    for r in range(0, len(p), vol):
        c = coords[r:r + vol]
        lo, hi = c.min(axis=0), c.max(axis=0)
        assert (hi - lo + 1).tolist() == list(tile)
        assert all(lo[a] % tile[a] == 0 for a in range(3))
        # the tokens of a box come in raster order
        assert (np.diff(p[r:r + vol]) > 0).all()


def test_apply_and_undo_are_inverse():
    g = np.random.default_rng(0)
    p = reorder.tiled_order((3, 6, 10), (2, 4, 4), L=190)
    x = g.standard_normal((2, 3, 190, 5))
    y = reorder.apply_order(x, p)
    assert np.array_equal(y[:, :, 7], x[:, :, p[7]])
    assert np.array_equal(reorder.undo_order(y, p), x)


def test_dense_attention_is_order_equivariant():
    """softmax attention commutes with a permutation of the tokens, so a
    reordered whole path at keep = T comes back to raster dense attention."""
    g = np.random.default_rng(1)
    grid, L, d = (2, 6, 9), 108 + 20, 8
    q, k, v = (g.standard_normal((L, d)) for _ in range(3))
    p = reorder.tiled_order(grid, (2, 4, 4), L=L)
    scale = 1 / math.sqrt(d)
    ref = pisa.dense_attention(q, k, v, scale)
    Q, K, V = (reorder.apply_order(x, p, axis=0) for x in (q, k, v))
    T = -(-L // 16)
    out = pisa.pisa_reference(Q[None, None], K[None, None], V[None, None], 16, T, 0.1, scale)[(0, 0)]["O"]
    assert np.abs(reorder.undo_order(out, p, axis=0) - ref).max() < 1e-12


def test_tiled_order_lowers_pisa_error_on_smooth_keys():
    """Diagnostic for the purpose of the order: with spatially smooth keys
    (the Fourier-feature workload), compact 3D tiles make better blocks than
    raster rows, so PISA at the same density lands closer to dense."""
    from workloads.dit import WORKLOADS, make_inputs
    w = WORKLOADS["video480p_32760"].with_(grid=(8, 16, 32), H=1, name="small")
    q, k, v = (x.double().numpy()[0, 0] for x in make_inputs(w))
    keep = -(-125 * w.T // 1000)
    errs = {}
    for tile in [(1, 1, 1), (2, 4, 8)]:
        p = reorder.tiled_order(w.grid, tile, L=w.L)
        Q, K, V = (reorder.apply_order(x, p, axis=0) for x in (q, k, v))
        o = pisa.pisa_reference(Q[None, None], K[None, None], V[None, None], 64, keep, w.lam, w.scale)[(0, 0)]["O"]
        dense = pisa.dense_attention(Q, K, V, w.scale)
        errs[tile] = np.abs(o - dense).max()
    assert errs[(2, 4, 8)] < 0.75 * errs[(1, 1, 1)], errs
