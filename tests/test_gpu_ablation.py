"""The method against its two ablations on the GPU: keep-or-drop (the tail
dropped) and the zeroth-order tail without the first-order correction.

Errors are taken against dense softmax attention computed in float64 on the
CPU. The PISA page (sections 1 and 3) argues that at equal density the
hybrid with both tail terms is closer to dense than the zeroth-order tail
alone, and both are closer than dropping the tail. Checked here at three
densities, together with the limit k = T, where every variant is dense
attention. The ablations approach dense as the density grows; the method's
own error need not, and on these synthetic inputs it stays roughly flat (so
does the oracle's with the per-block first-order term: what remains is the
higher-order remainder of the blocks left in the tail), so that is not
asserted for it. A property test of the method on our synthetic inputs,
not an oracle parity test (those are in test_gpu_parity.py)."""
import pytest
import torch

from block_sparse_attention_pisa_amd import paro
from workloads import WORKLOADS, make_inputs

from parity_util import log

pytestmark = pytest.mark.gpu

MODES = (("pisa", {}), ("zeroth", {"first_order": False}), ("drop", {"drop_tail": True}))


def _dense(q, k, v, scale):
    """softmax(scale q k^T) v per head, float64 on the CPU."""
    q, k, v = (x.double() for x in (q, k, v))
    s = torch.matmul(q, k.transpose(-1, -2).contiguous()) * scale
    return torch.matmul(torch.softmax(s, dim=-1), v)


@pytest.mark.parametrize("name,heads", [("image_4608", [0, 5, 11]), ("tiny_fp32", [0, 1])])
def test_error_order_and_density(name, heads):
    w = WORKLOADS[name]
    q, k, v = make_inputs(w, heads=heads)
    ref = _dense(q, k, v, w.scale)
    nref = float(ref.norm())
    qd, kd, vd = (x.cuda() for x in (q, k, v))
    stats = paro.precompute(kd, vd)
    T = w.T
    keeps = sorted({-(-pm * T // 1000) for pm in (125, 250, 500)} | {T})
    err = {}
    for kk in keeps:
        idx = paro.route(qd, stats[0], stats[3], kk, w.lam)
        for mode, kw in MODES:
            o = paro.attention(qd, kd, vd, stats[0], stats[1], stats[2], idx, kk, **kw)
            err[(kk, mode)] = float((o.double().cpu() - ref).norm()) / nref
        log(f"[ablation] {name} k={kk}/{T}: " + " ".join(f"{m} {err[(kk, m)]:.4g}" for m, _ in MODES))
    floor = 1e-2 if w.dtype == "bf16" else 1e-5   # output rounding of the dense result
    for kk in keeps[:-1]:
        assert err[(kk, "pisa")] < err[(kk, "zeroth")] < err[(kk, "drop")], (kk, err)
    for mode, _ in MODES:
        assert err[(T, mode)] < floor, (mode, err[(T, mode)])
    for mode in ("zeroth", "drop"):
        e = [err[(kk, mode)] for kk in keeps]
        assert all(a > b for a, b in zip(e, e[1:])), (mode, e)
