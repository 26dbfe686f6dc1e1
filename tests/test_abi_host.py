"""C ABI checks that need no GPU: exported symbols, helpers and host-side validation.

Validation runs before any HIP call, so rejected arguments return their error
code here (a launch attempted without a device would give PARO_ERR_HIP instead).
"""
import ctypes
import os
import re
import subprocess

import pytest

from block_sparse_attention_pisa_amd import paro

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "paro.h")

pytestmark = pytest.mark.skipif(not os.path.exists(paro.LIB_PATH), reason="libparo.so not built")

FAKE = 0x10000  # an aligned non-null address that validation never dereferences


def _declared():
    src = open(HEADER).read()
    return sorted(set(re.findall(r"\b(paro_[a-z_0-9]+)\s*\(", src)))


def test_header_symbols_exported():
    names = _declared()
    assert set(names) == set(paro.EXPORTED)
    out = subprocess.run(["nm", "-D", "--defined-only", paro.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (paro_\w+)", out))
    for n in names:
        assert n in exported, n
    L = paro.lib()
    for n in names:
        assert hasattr(L, n)


def test_helpers():
    L = paro.lib()
    assert L.paro_version() == 100
    assert L.paro_num_blocks(75600, 64) == 1182
    assert L.paro_num_blocks(64, 64) == 1 and L.paro_num_blocks(65, 64) == 2
    assert L.paro_num_blocks(0, 64) == -1
    for c in range(-7, 1):
        assert len(L.paro_status_string(c)) > 0
    assert L.paro_status_string(-99) == b"unknown status"


def _p(**kw):
    d = dict(B=1, H=2, L=1000, d=128, block=64, dtype=0, scale=0.088)
    d.update(kw)
    return paro.ParoProblem(**d)


def test_workspace_bytes():
    L = paro.lib()
    p = _p()
    n = L.paro_precompute_workspace_bytes(ctypes.byref(p))
    assert n > 0 and n % (128 * 128 * 4) == 0
    assert L.paro_precompute_workspace_bytes(ctypes.byref(_p(d=96))) == 0


@pytest.mark.parametrize("kw,code", [
    (dict(d=96), -2), (dict(block=32), -2), (dict(L=0), -2), (dict(B=0), -2), (dict(H=-1), -2),
    (dict(dtype=7), -3), (dict(scale=0.0), -7), (dict(scale=float("nan")), -7),
    (dict(L=64 * 16384 + 1), -2), (dict(B=300, H=300), -2),
    (dict(B=16, H=1, L=64 * 16384, d=128), -2),   # B*H*L*d = 2^31 elements: past the 32-bit bound
])
def test_problem_validation(kw, code):
    L = paro.lib()
    p = _p(**kw)
    ws = 1 << 30
    assert L.paro_precompute(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, ws, None) == code
    assert L.paro_route(ctypes.byref(p), FAKE, FAKE, FAKE, 2, 0.1, FAKE, None) == code
    assert L.paro_attention(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 2, FAKE, FAKE, ws, None) == code


def test_element_count_bound():
    """B*H*L*d must stay below 2^31: one element less per tensor passes the
    shape checks (the call then stops at the workspace size, before any launch)."""
    L = paro.lib()
    big = _p(B=16, H=1, L=64 * 16384, d=128)
    assert L.paro_precompute_workspace_bytes(ctypes.byref(big)) == 0
    ok = _p(B=16, H=1, L=64 * 16384 - 1, d=128)
    ws = L.paro_precompute_workspace_bytes(ctypes.byref(ok))
    assert ws > 0
    assert L.paro_precompute(ctypes.byref(ok), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, ws - 1, None) == -5
    assert L.paro_precompute(ctypes.byref(big), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 40, None) == -2
    assert L.paro_route(ctypes.byref(big), FAKE, FAKE, FAKE, 2, 0.1, FAKE, None) == -2
    assert L.paro_reorder(ctypes.byref(big), ctypes.byref(_g(1, 1, 1, 1, 1, 1)), 0, FAKE, FAKE + 16, None) == -2


def test_pointer_and_argument_validation():
    L = paro.lib()
    p = _p()
    pp = ctypes.byref(p)
    ws = L.paro_precompute_workspace_bytes(pp)
    assert L.paro_precompute(None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, ws, None) == -1
    assert L.paro_precompute(pp, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, ws, None) == -1
    assert L.paro_precompute(pp, FAKE + 8, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, ws, None) == -4
    assert L.paro_precompute(pp, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, ws - 1, None) == -5
    T = L.paro_num_blocks(1000, 64)
    assert L.paro_route(pp, FAKE, FAKE, FAKE, T + 1, 0.1, FAKE, None) == -2
    assert L.paro_route(pp, FAKE, FAKE, FAKE, -1, 0.1, FAKE, None) == -2
    assert L.paro_route(pp, FAKE, FAKE, FAKE, 2, float("inf"), FAKE, None) == -7
    assert L.paro_route(pp, FAKE, FAKE, FAKE, 2, 0.1, None, None) == -1
    assert L.paro_route(pp, FAKE, FAKE + 4, FAKE, 2, 0.1, FAKE, None) == -4
    wa = L.paro_attention_workspace_bytes(pp)
    assert wa == 2 * 1 * 2 * T * 128 * 2 + 512   # bf16 copies of kbar and vsum, 8 item-queue counters
    assert L.paro_attention_workspace_bytes(ctypes.byref(_p(dtype=1))) == 0
    assert L.paro_attention(pp, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, 2, FAKE, FAKE, wa, None) == -1
    assert L.paro_attention(pp, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, T + 1, FAKE, FAKE, wa, None) == -2
    assert L.paro_attention(pp, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 2, FAKE + 2, FAKE, wa, None) == -4
    assert L.paro_attention(pp, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 2, FAKE, FAKE, wa - 1, None) == -5
    assert L.paro_attention(pp, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 2, FAKE, None, wa, None) == -1
    assert L.paro_attention_mode(pp, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 2, 3, FAKE, FAKE, wa, None) == -7
    assert L.paro_attention_mode(pp, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 2, -1, FAKE, FAKE, wa, None) == -7
    assert L.paro_attention_mode(pp, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, T + 1, 1, FAKE, FAKE, wa, None) == -2


def test_binding_refuses_host_tensors():
    import torch
    q = torch.zeros(1, 1, 64, 64)
    with pytest.raises(ValueError):
        paro.precompute(q, q)


def _g(t, y, x, tt, ty, tx):
    return paro.ParoGrid(t, y, x, tt, ty, tx)


@pytest.mark.parametrize("grid,tile,extra", [
    ((3, 7, 11), (2, 3, 4), 0), ((5, 9, 13), (4, 4, 4), 17), ((1, 33, 20), (1, 8, 8), 64),
    ((21, 10, 16), (2, 4, 8), 3), ((4, 4, 4), (9, 9, 9), 0), ((2, 5, 3), (1, 1, 1), 5),
    ((21, 45, 80), (2, 4, 8), 0), ((1, 64, 64), (1, 8, 8), 512), ((7, 1, 1), (3, 1, 1), 2),
])
def test_reorder_source_matches_oracle_order(grid, tile, extra):
    """The library's arithmetic position -> source map (the one the reorder
    kernel evaluates) equals the oracle's box-by-box enumeration."""
    from oracle import reorder
    N = grid[0] * grid[1] * grid[2]
    L = N + extra
    ref = reorder.tiled_order(grid, tile, L=L)
    lib = paro.lib()
    g = _g(*grid, *tile)
    got = [lib.paro_reorder_source(ctypes.byref(g), L, i) for i in range(L)]
    assert got == ref.tolist()


def test_reorder_validation():
    L = paro.lib()
    p = _p(L=1000)
    pp = ctypes.byref(p)
    ok = _g(2, 10, 50, 2, 4, 8)
    assert L.paro_reorder_source(ctypes.byref(ok), 1000, 999) == 999
    assert L.paro_reorder_source(ctypes.byref(ok), 1000, 1000) == -1
    assert L.paro_reorder_source(ctypes.byref(_g(2, 10, 51, 2, 4, 8)), 1000, 0) == -1
    assert L.paro_reorder_source(None, 1000, 0) == -1
    assert L.paro_reorder(pp, None, 0, FAKE, FAKE + 16, None) == -1
    assert L.paro_reorder(pp, ctypes.byref(_g(2, 10, 51, 2, 4, 8)), 0, FAKE, FAKE + 16, None) == -2
    assert L.paro_reorder(pp, ctypes.byref(_g(0, 10, 50, 2, 4, 8)), 0, FAKE, FAKE + 16, None) == -2
    assert L.paro_reorder(pp, ctypes.byref(_g(2, 10, 50, 2, 0, 8)), 0, FAKE, FAKE + 16, None) == -2
    assert L.paro_reorder(pp, ctypes.byref(ok), 2, FAKE, FAKE + 16, None) == -7
    assert L.paro_reorder(pp, ctypes.byref(ok), 0, FAKE, FAKE, None) == -7
    assert L.paro_reorder(pp, ctypes.byref(ok), 1, None, FAKE, None) == -1
    assert L.paro_reorder(pp, ctypes.byref(ok), 1, FAKE, FAKE + 4, None) == -4
    assert L.paro_reorder(ctypes.byref(_p(d=96)), ctypes.byref(ok), 0, FAKE, FAKE + 16, None) == -2


def test_fp8_entry_points_validation():
    L = paro.lib()
    p = _p()
    pp = ctypes.byref(p)
    T = L.paro_num_blocks(1000, 64)
    wf = L.paro_attention_fp8_workspace_bytes(pp)
    # e4m3 K [2][1000][128] + its scales + e4m3 kbar [2][16][128] + scales + bf16 vsum + 8 item-queue
    # counters, 256-byte aligned regions
    up = lambda x: (x + 255) // 256 * 256
    assert wf == up(2 * 1000 * 128) + up(2 * 1000) + up(2 * T * 128) + up(2 * T) + up(2 * T * 128 * 2) + 512
    assert L.paro_attention_fp8_workspace_bytes(ctypes.byref(_p(dtype=1))) == 0
    args = (FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE)
    assert L.paro_attention_fp8(ctypes.byref(_p(dtype=1)), *args, 2, 0, FAKE, FAKE, wf, None) == -3
    assert L.paro_attention_fp8(pp, *args, T + 1, 0, FAKE, FAKE, wf, None) == -2
    assert L.paro_attention_fp8(pp, *args, 2, 3, FAKE, FAKE, wf, None) == -7
    assert L.paro_attention_fp8(pp, *args, 2, 0, FAKE, None, wf, None) == -1
    assert L.paro_attention_fp8(pp, *args, 2, 0, FAKE, FAKE, wf - 1, None) == -5
    assert L.paro_attention_fp8(pp, *args, 2, 0, FAKE + 4, FAKE, wf, None) == -4
    assert L.paro_fp8_rows(FAKE, 7, 10, 128, FAKE, FAKE, None) == -3
    assert L.paro_fp8_rows(FAKE, 0, 10, 96, FAKE, FAKE, None) == -2
    assert L.paro_fp8_rows(FAKE, 0, 0, 128, FAKE, FAKE, None) == -2
    assert L.paro_fp8_rows(FAKE, 0, 10, 128, FAKE, None, None) == -1
    assert L.paro_fp8_rows(FAKE + 8, 0, 10, 128, FAKE, FAKE, None) == -4


def test_budget_entry_points_validation():
    L = paro.lib()
    p = _p()
    pp = ctypes.byref(p)
    T = L.paro_num_blocks(1000, 64)
    wb = L.paro_route_budget_workspace_bytes(pp)
    assert wb == 2 * T * 128 * 4   # qbar, fp32
    rb = lambda K, kmin, lam=0.1, w=FAKE, ws=wb: L.paro_route_budget(pp, FAKE, FAKE, FAKE, K, kmin, lam, w, FAKE,
                                                                       FAKE, FAKE, ws, None)
    assert rb(T * 2 - 1, 2) == -2          # below the per-row floor
    assert rb(T * T + 1, 1) == -2          # above T^2
    assert rb(T, -1) == -2
    assert rb(0, 0) == -2
    assert rb(T * 3, 1, lam=float("nan")) == -7
    assert rb(T * 3, 1, w=None) == -1
    assert rb(T * 3, 1, ws=wb - 1) == -5
    wa = L.paro_attention_workspace_bytes(pp)
    ac = lambda stride, mode=0, offs=FAKE: L.paro_attention_csr(pp, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, offs, FAKE,
                                                                 stride, mode, FAKE, FAKE, wa, None)
    assert ac(-1) == -2
    assert ac(10, mode=3) == -7
    assert ac(10, offs=None) == -1


def test_noalloc_validation():
    """paro_attention_noalloc validates like paro_attention_mode and refuses a
    problem whose workspace would not fit its static scratch, before any HIP call."""
    L = paro.lib()
    args = (FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE)
    p = _p()
    T = L.paro_num_blocks(1000, 64)
    na = lambda pr, keep=2, mode=0, o=FAKE: L.paro_attention_noalloc(ctypes.byref(pr), *args, keep, mode, o, None)
    assert na(p, keep=T + 1) == -2
    assert na(p, mode=3) == -7
    assert na(p, o=None) == -1
    assert na(p, o=FAKE + 4) == -4
    assert na(_p(d=96)) == -2
    big = _p(B=1, H=60, L=64 * 1100)        # 2 * 60 * 1100 * 128 * 2 bytes > 32 MiB
    assert L.paro_attention_workspace_bytes(ctypes.byref(big)) > paro.NOALLOC_SCRATCH_BYTES
    assert na(big) == -5
    fits = _p(B=1, H=40, L=75600)           # the 720p video shape: 24.2 MB
    assert L.paro_attention_workspace_bytes(ctypes.byref(fits)) <= paro.NOALLOC_SCRATCH_BYTES
