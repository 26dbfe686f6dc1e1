"""Stream semantics and graph capture of the whole path.

The ABI enqueues every kernel on the caller's stream and never allocates,
sets memory or synchronizes, so the calls follow stream order and can be
recorded into a HIP graph. Both are checked bit for bit against the same
calls made eagerly on the default stream: precompute, routing, attention
(bf16 and fp8 key-query products), budgeted routing with CSR attention, and
the token reordering.
"""
import ctypes

import pytest
import torch

from block_sparse_attention_pisa_amd import paro
from workloads import WORKLOADS, make_inputs

from parity_util import log

pytestmark = pytest.mark.gpu


TILE = (1, 8, 8)   # one 64-token block per 8 x 8 patch of the image latent


def _buffers(w, qd, kd):
    dev = qd.device
    p = paro.problem(qd)
    K = w.k * w.T
    return dict(
        stats=paro.alloc_stats(kd),
        idx=torch.empty(w.B, w.H, w.T, w.k, dtype=torch.int32, device=dev),
        out=torch.empty_like(qd), out8=torch.empty_like(qd), outc=torch.empty_like(qd),
        ws=torch.empty(max(16, paro.attention_workspace_bytes(p)), dtype=torch.uint8, device=dev),
        ws8=torch.empty(max(16, paro.attention_fp8_workspace_bytes(p)), dtype=torch.uint8, device=dev),
        budget=(torch.empty(w.B, w.H, w.T + 1, dtype=torch.int32, device=dev),
                torch.zeros(w.B, w.H, K, dtype=torch.int32, device=dev),
                torch.empty(w.B, w.H, w.T, dtype=torch.int64, device=dev),
                torch.empty(max(16, int(paro.lib().paro_route_budget_workspace_bytes(ctypes.byref(p)))),
                            dtype=torch.uint8, device=dev)),
        qt=torch.empty_like(qd), qback=torch.empty_like(qd))


def _step(w, qd, kd, vd, b):
    """precompute, route, attention (bf16 and fp8), budgeted routing with CSR
    attention, and a reorder round trip of q"""
    st = b["stats"]
    paro.precompute(kd, vd, out=st)
    paro.route(qd, st[0], st[3], w.k, w.lam, out=b["idx"])
    paro.attention(qd, kd, vd, st[0], st[1], st[2], b["idx"], w.k, out=b["out"], workspace=b["ws"])
    paro.attention(qd, kd, vd, st[0], st[1], st[2], b["idx"], w.k, out=b["out8"], workspace=b["ws8"], qk_fp8=True)
    offs, lists, _, _ = b["budget"]
    paro.route_budget(qd, st[0], st[3], w.k * w.T, 1, w.lam, out=b["budget"])
    paro.attention_csr(qd, kd, vd, st[0], st[1], st[2], offs, lists, w.k * w.T, out=b["outc"], workspace=b["ws"])
    paro.reorder(qd, w.grid, TILE, out=b["qt"])
    paro.reorder(b["qt"], w.grid, TILE, inverse=True, out=b["qback"])


def _outputs(b):
    return [*b["stats"][:4], b["idx"], b["out"], b["out8"], b["outc"], *b["budget"][:3], b["qt"], b["qback"]]


def _results(b):
    return [t.clone() for t in _outputs(b)]


def _clobber(b):
    for t in _outputs(b):
        if t.is_floating_point():
            t.fill_(float("nan"))
        else:
            t.fill_(-7)


def _same(a, b):
    return all(torch.equal(x, y) for x, y in zip(a, b))


def test_side_stream_and_graph_replays_match_eager():
    w = WORKLOADS["image_4608"]
    q, k, v = make_inputs(w)
    qd, kd, vd = (x.cuda() for x in (q, k, v))

    # eager reference on the default stream
    ref_bufs = _buffers(w, qd, kd)
    _step(w, qd, kd, vd, ref_bufs)
    torch.cuda.synchronize()
    ref = _results(ref_bufs)

    # side stream: the inputs are written on it after a long delay, so a
    # launch on any other stream would read them before they are there
    s = torch.cuda.Stream()
    q2, k2, v2 = (torch.zeros_like(x) for x in (qd, kd, vd))
    bufs = _buffers(w, qd, kd)
    _clobber(bufs)
    busy = torch.randn(2048, 2048, device="cuda")
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for _ in range(20):
            busy = busy @ busy
            busy = busy / busy.norm()
        for dst, src in ((q2, qd), (k2, kd), (v2, vd)):
            dst.copy_(src)
        _step(w, q2, k2, v2, bufs)
    s.synchronize()
    assert _same(_results(bufs), ref), "results on a side stream differ from the default stream's"
    assert torch.equal(ref[-1], qd)   # the reorder round trip gives q back
    log("[streams] side stream: bitwise equal")

    # graph: captured once on a side stream, replayed three times; between
    # replays the outputs are clobbered and an eager step runs on other
    # buffers, and every replay must reproduce the eager result
    gbufs = _buffers(w, qd, kd)
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        _step(w, q2, k2, v2, gbufs)     # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _step(w, q2, k2, v2, gbufs)
    torch.cuda.synchronize()
    other = _buffers(w, qd, kd)
    for r in range(3):
        _clobber(gbufs)
        _step(w, qd, kd, vd, other)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert _same(_results(gbufs), ref), f"graph replay {r} differs from the eager result"
        assert _same(_results(other), ref)
    log("[streams] graph: 3 replays bitwise equal")
