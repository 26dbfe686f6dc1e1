"""Plain CPU oracle of the tiled token order (geometric token reordering).

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module. The
product path never imports it and shares no code with it.

Source: "PAROAttention: Pattern-Aware ReOrdering for Efficient Sparse and
Quantized Attention in Visual Generation Models" (abstract): tokens of a
visual latent are reordered so that attention, which aggregates locally,
becomes a block-wise pattern before sparsification; and the vector-quantised
attention review ("Adaptive Vector Quantized Attention", supplementary
analysis), whose ablation finds token order matters (a space-filling order
slightly better than raster, a random order clearly worse).

The pages give no concrete permutation. The reading taken here is the
plainest locality-preserving one: cut the (t, y, x) grid into boxes of
tile_t x tile_y x tile_x tokens (boxes at the far edges are cut short), list
the boxes in raster order (x fastest), and list the tokens of each box in
raster order. Tokens after the grid (text tokens) keep their places.

Written as an enumeration (nested loops over boxes, then over the tokens of a
box), which is checked by eye against the definition above.
"""

from __future__ import annotations

import numpy as np

__all__ = ["tiled_order", "apply_order", "undo_order"]


def tiled_order(grid, tile, L: int | None = None) -> np.ndarray:
    """perm[i] = raster index of the token placed at position i.

    grid = (Gt, Gy, Gx) holds the first Gt*Gy*Gx of the L tokens in raster
    order (x fastest); tile = (tt, ty, tx), each >= 1. Positions >= Gt*Gy*Gx
    map to themselves.
    """
    Gt, Gy, Gx = (int(g) for g in grid)
    tt, ty, tx = (int(s) for s in tile)
    assert min(Gt, Gy, Gx, tt, ty, tx) >= 1
    N = Gt * Gy * Gx
    L = N if L is None else int(L)
    assert L >= N
    order = []
    for t0 in range(0, Gt, tt):
        for y0 in range(0, Gy, ty):
            for x0 in range(0, Gx, tx):
                for t in range(t0, min(t0 + tt, Gt)):
                    for y in range(y0, min(y0 + ty, Gy)):
                        for x in range(x0, min(x0 + tx, Gx)):
                            order.append((t * Gy + y) * Gx + x)
    order.extend(range(N, L))
    return np.asarray(order, dtype=np.int64)


def apply_order(x: np.ndarray, perm: np.ndarray, axis: int = -2) -> np.ndarray:
    """Tokens of x (along axis) in the new order: out[..., i, :] = x[..., perm[i], :]."""
    return np.take(x, perm, axis=axis)


def undo_order(y: np.ndarray, perm: np.ndarray, axis: int = -2) -> np.ndarray:
    """Inverse of apply_order: out[..., perm[i], :] = y[..., i, :]."""
    out = np.empty_like(y)
    idx = [slice(None)] * y.ndim
    idx[axis] = perm
    out[tuple(idx)] = y
    return out
