"""Guard bands and run-to-run determinism of every output buffer.

Each output is handed to the library as a view into a larger buffer whose
bytes before and after the view hold a sentinel pattern; after the call the
sentinels must be untouched (no write outside the documented extent of any
output: kbar, vsum, Hbar, M, idx, O, the budget offsets, lists and weights,
the reordered tensor), and outputs must be bitwise identical across runs
(the kernels use no float atomics; every reduction has a fixed order).
"""
import numpy as np
import pytest
import torch

from block_sparse_attention_pisa_amd import paro
from workloads import WORKLOADS, make_inputs, random_uniform_inputs

from parity_util import log

pytestmark = pytest.mark.gpu

GUARD = 4096  # bytes of sentinel on each side (keeps every view 16-byte aligned)
SENTINEL = 0xA5


def guarded(shape, dtype):
    """(buffer, view): a contiguous view of `shape` with GUARD sentinel bytes before and after it."""
    n = int(np.prod(shape)) * torch.empty((), dtype=dtype).element_size()
    raw = torch.full((n + 2 * GUARD,), SENTINEL, dtype=torch.uint8, device="cuda")
    view = raw[GUARD:GUARD + n].view(dtype).view(*shape)
    return raw, view


def intact(raw, name):
    n = raw.numel() - 2 * GUARD
    head, tail = raw[:GUARD].cpu(), raw[GUARD + n:].cpu()
    assert (head == SENTINEL).all(), f"{name}: bytes before the output were written"
    assert (tail == SENTINEL).all(), f"{name}: bytes after the output were written"


def bits(t):
    return t.contiguous().view(torch.uint8).cpu()


@pytest.mark.parametrize("case", ["image", "ragged_d64"])
def test_guard_bands_and_determinism(case):
    if case == "image":
        w = WORKLOADS["image_4608"]
        q, k, v = make_inputs(w, heads=[0, 1, 2])
        keep = w.k
    else:
        q, k, v = random_uniform_inputs(2, 3, 64 * 9 - 17, 64, dtype=torch.bfloat16, seed=3, scale=0.8)
        keep = 3
    B, H, L, d = q.shape
    T = -(-L // 64)
    log(f"[guards] {case} {tuple(q.shape)} keep {keep}")
    qd, kd, vd = (x.cuda() for x in (q, k, v))
    runs = []
    for rep in range(2):
        g_kbar, kbar = guarded((B, H, T, d), torch.float32)
        g_vsum, vsum = guarded((B, H, T, d), torch.float32)
        g_hbar, Hbar = guarded((B, H, d, d), torch.float32)
        g_m, M = guarded((B, H, T), torch.float64)
        ws = torch.empty(max(16, paro.workspace_bytes(paro.problem(kd))), dtype=torch.uint8, device="cuda")
        paro.precompute(kd, vd, out=(kbar, vsum, Hbar, M, ws))
        g_idx, idx = guarded((B, H, T, keep), torch.int32)
        paro.route(qd, kbar, M, keep, 0.1, out=idx)
        g_o, o = guarded((B, H, L, d), torch.bfloat16)
        paro.attention(qd, kd, vd, kbar, vsum, Hbar, idx, keep, out=o)
        g_o8, o8 = guarded((B, H, L, d), torch.bfloat16)
        paro.attention(qd, kd, vd, kbar, vsum, Hbar, idx, keep, out=o8, qk_fp8=True)
        K = T * keep + T // 2
        g_off, offs = guarded((B, H, T + 1), torch.int32)
        g_li, lists = guarded((B, H, K), torch.int32)
        g_wq, wq = guarded((B, H, T), torch.int64)
        wsb = torch.empty(max(16, int(paro.lib().paro_route_budget_workspace_bytes(
            paro.ctypes.byref(paro.problem(qd))))), dtype=torch.uint8, device="cuda")
        paro.route_budget(qd, kbar, M, K, 1, 0.1, out=(offs, lists, wq, wsb))
        g_oc, oc = guarded((B, H, L, d), torch.bfloat16)
        paro.attention_csr(qd, kd, vd, kbar, vsum, Hbar, offs, lists, K, out=oc)
        g_r, r = guarded((B, H, L, d), torch.bfloat16)
        grid, tile = ((1, 64, 64), (1, 8, 8)) if case == "image" else ((1, 13, 43), (1, 4, 8))
        paro.reorder(qd, grid, tile, out=r)
        torch.cuda.synchronize()
        for raw, name in ((g_kbar, "kbar"), (g_vsum, "vsum"), (g_hbar, "Hbar"), (g_m, "M"), (g_idx, "idx"),
                          (g_o, "O"), (g_o8, "O fp8"), (g_off, "offsets"), (g_li, "budget lists"),
                          (g_wq, "budget weights"), (g_oc, "O csr"), (g_r, "reorder")):
            intact(raw, name)
        assert int(offs[..., -1].min()) == K and int(offs[..., -1].max()) == K
        runs.append([bits(x) for x in (kbar, vsum, Hbar, M, idx, o, o8, offs, lists, wq, oc, r)])
    for a, b, name in zip(*runs, ("kbar", "vsum", "Hbar", "M", "idx", "O", "O fp8", "offsets", "lists", "weights",
                                  "O csr", "reorder")):
        assert torch.equal(a, b), f"{name} differs between two runs"
