"""The method's argument measured on the oracle (CPU, fp64): on one seeded
head of the tiny synthetic workload (1024 tokens, 16 blocks), at 2, 4 and 8
exact blocks, the error against dense attention orders as

    per-block first order < global first order (the method)
                          < zeroth-order tail only < tail dropped.

PISA page, section 1 (keep-or-drop loses the tail's mass), section 2 (the
first-order term, with the per-block H_j rejected for its memory cost and
replaced by the global mean) and section 3 (the hybrid beats both).
The GPU counterpart is tests/test_gpu_ablation.py."""
import numpy as np

from oracle import pisa
from workloads import WORKLOADS, make_inputs


def test_error_order_of_tail_variants():
    w = WORKLOADS["tiny_fp32"]
    q, k, v = make_inputs(w, heads=[0])
    q, k, v = (x.double().numpy()[0, 0] for x in (q, k, v))
    st = pisa.block_stats(k, v, w.block, keep_H=True)
    T = st["kbar"].shape[0]
    dense = pisa.dense_attention(q, k, v, w.scale)
    nd = np.linalg.norm(dense)
    variants = (("block", {"first_order": "block"}), ("global", {}), ("zeroth", {"first_order": "none"}),
                ("drop", {"tail": False}))
    for kk in (2, 4, 8):
        idx, _ = pisa.route(q, st["kbar"], st["M"], kk, w.lam, w.scale, w.block)
        err = [np.linalg.norm(pisa.attention(q, k, v, st, idx, w.scale, w.block, **kw) - dense) / nd
               for _, kw in variants]
        assert all(a < b for a, b in zip(err, err[1:])), (kk, T, dict(zip((n for n, _ in variants), err)))
