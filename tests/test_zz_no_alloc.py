"""paro_attention_noalloc (the attention with its workspace in the library's
static device scratch, for callers that cannot allocate) against
paro_attention_mode with a caller workspace, through the C ABI: two calls
in a row, the second on a smaller problem, each bit for bit equal to the
entry point it varies (same kernels, same inputs), in all three tail modes;
then an fp32 problem (no workspace) and the size limit.
"""
import ctypes

import pytest
import torch

from block_sparse_attention_pisa_amd import paro
from workloads import WORKLOADS, make_inputs

from parity_util import log

pytestmark = pytest.mark.gpu


def _path(w, heads):
    q, k, v = make_inputs(w, heads=heads)
    qd, kd, vd = (x.cuda() for x in (q, k, v))
    kbar, vsum, Hbar, M = paro.precompute(kd, vd)
    idx = paro.route(qd, kbar, M, w.k, w.lam)
    return qd, kd, vd, kbar, vsum, Hbar, idx, w.k


def _raw_noalloc(qd, kd, vd, kbar, vsum, Hbar, idx, keep, mode, out):
    p = paro.problem(qd)
    return paro.lib().paro_attention_noalloc(
        ctypes.byref(p), qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), kbar.data_ptr(), vsum.data_ptr(),
        Hbar.data_ptr(), idx.data_ptr() if keep > 0 else None, keep, mode, out.data_ptr(),
        torch.cuda.current_stream().cuda_stream)


def test_noalloc_matches_the_workspace_entry_point():
    cases = [("video720p_75600", None), ("image_4608", [0, 3, 7])]
    for name, heads in cases:
        w = WORKLOADS[name]
        args = _path(w, heads)
        need = paro.attention_workspace_bytes(paro.problem(args[0]))
        log(f"[noalloc] {name} heads {heads}: workspace {need} bytes of {paro.NOALLOC_SCRATCH_BYTES}")
        assert 0 < need <= paro.NOALLOC_SCRATCH_BYTES
        for mode, kw in ((0, {}), (1, {"drop_tail": True}), (2, {"first_order": False})):
            ref = paro.attention(*args, **kw)
            o = torch.full_like(args[0], float("nan"))
            assert _raw_noalloc(*args, mode, o) == 0
            torch.cuda.synchronize()
            assert torch.equal(o.view(torch.int16), ref.view(torch.int16)), (name, mode)
    # an fp32 problem needs no scratch
    w = WORKLOADS["tiny_fp32"]
    args = _path(w, None)
    ref = paro.attention(*args)
    o = paro.attention_noalloc(*args, out=torch.empty_like(args[0]))
    torch.cuda.synchronize()
    assert torch.equal(o, ref)


def test_noalloc_rejects_problems_past_the_scratch():
    """A problem whose workspace exceeds the scratch returns PARO_ERR_WORKSPACE
    and launches nothing (the output keeps its contents)."""
    B, H, L, d = 1, 60, 64 * 1100, 128        # 2 * 60 * 1100 * 128 * 2 bytes = 33.8 MB > 32 MiB
    q = torch.zeros(B, H, L, d, dtype=torch.bfloat16, device="cuda")
    T = L // 64
    st = (torch.zeros(B, H, T, d, device="cuda"), torch.zeros(B, H, T, d, device="cuda"),
          torch.zeros(B, H, d, d, device="cuda"))
    idx = torch.zeros(B, H, T, 1, dtype=torch.int32, device="cuda")
    assert paro.attention_workspace_bytes(paro.problem(q)) > paro.NOALLOC_SCRATCH_BYTES
    o = torch.full_like(q, 3.0)
    assert _raw_noalloc(q, q, q, *st, idx, 1, 0, o) == -5
    torch.cuda.synchronize()
    assert bool((o == 3.0).all())
