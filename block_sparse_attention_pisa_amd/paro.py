"""Thin ctypes binding of libparo (include/paro.h).

Argument marshalling only: every step of the PISA path runs in the HIP
kernels of libparo.so. PyTorch supplies device memory and the current
stream. There is no fallback: without the built library every call raises.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libparo.so")

PARO_OK = 0
PARO_DTYPE_BF16 = 0
PARO_DTYPE_FP32 = 1
BLOCK = 64

STATUS = {
    0: "PARO_OK", -1: "PARO_ERR_NULL", -2: "PARO_ERR_SHAPE", -3: "PARO_ERR_DTYPE",
    -4: "PARO_ERR_ALIGN", -5: "PARO_ERR_WORKSPACE", -6: "PARO_ERR_HIP", -7: "PARO_ERR_ARG",
}

EXPORTED = (
    "paro_precompute", "paro_precompute_workspace_bytes", "paro_route", "paro_attention",
    "paro_attention_mode", "paro_attention_workspace_bytes", "paro_attention_fp8",
    "paro_attention_fp8_workspace_bytes", "paro_fp8_rows", "paro_route_budget",
    "paro_route_budget_workspace_bytes", "paro_attention_csr", "paro_reorder",
    "paro_reorder_source", "paro_num_blocks", "paro_status_string", "paro_version",
    "paro_attention_noalloc",
)
NOALLOC_SCRATCH_BYTES = 32 << 20   # PARO_NOALLOC_SCRATCH_BYTES
REORDER_GATHER = 0
REORDER_SCATTER = 1


class ParoProblem(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int32), ("H", ctypes.c_int32), ("L", ctypes.c_int32),
        ("d", ctypes.c_int32), ("block", ctypes.c_int32), ("dtype", ctypes.c_int32),
        ("scale", ctypes.c_double),
    ]


class ParoGrid(ctypes.Structure):
    _fields_ = [
        ("t", ctypes.c_int32), ("y", ctypes.c_int32), ("x", ctypes.c_int32),
        ("tile_t", ctypes.c_int32), ("tile_y", ctypes.c_int32), ("tile_x", ctypes.c_int32),
    ]


class ParoError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        msg = lib().paro_status_string(code).decode() if _LIB is not None else ""
        super().__init__(f"{where}: {STATUS.get(code, code)} ({msg})")


_LIB = None


def lib() -> ctypes.CDLL:
    """Load libparo.so once; raise if it has not been built."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m block_sparse_attention_pisa_amd.build` "
                "(there is no CPU fallback)")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, sz, dbl = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t, ctypes.c_double
        pp = ctypes.POINTER(ParoProblem)
        L.paro_precompute.argtypes = [pp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.paro_precompute.restype = ctypes.c_int
        L.paro_precompute_workspace_bytes.argtypes = [pp]
        L.paro_precompute_workspace_bytes.restype = sz
        L.paro_route.argtypes = [pp, vp, vp, vp, i32, dbl, vp, vp]
        L.paro_route.restype = ctypes.c_int
        L.paro_attention.argtypes = [pp, vp, vp, vp, vp, vp, vp, vp, i32, vp, vp, sz, vp]
        L.paro_attention.restype = ctypes.c_int
        L.paro_attention_mode.argtypes = [pp, vp, vp, vp, vp, vp, vp, vp, i32, i32, vp, vp, sz, vp]
        L.paro_attention_mode.restype = ctypes.c_int
        L.paro_attention_noalloc.argtypes = [pp, vp, vp, vp, vp, vp, vp, vp, i32, i32, vp, vp]
        L.paro_attention_noalloc.restype = ctypes.c_int
        L.paro_attention_workspace_bytes.argtypes = [pp]
        L.paro_attention_workspace_bytes.restype = sz
        L.paro_attention_fp8.argtypes = [pp, vp, vp, vp, vp, vp, vp, vp, i32, i32, vp, vp, sz, vp]
        L.paro_attention_fp8.restype = ctypes.c_int
        L.paro_attention_fp8_workspace_bytes.argtypes = [pp]
        L.paro_attention_fp8_workspace_bytes.restype = sz
        L.paro_fp8_rows.argtypes = [vp, i32, ctypes.c_int64, i32, vp, vp, vp]
        L.paro_fp8_rows.restype = ctypes.c_int
        L.paro_route_budget.argtypes = [pp, vp, vp, vp, i32, i32, dbl, vp, vp, vp, vp, sz, vp]
        L.paro_route_budget.restype = ctypes.c_int
        L.paro_route_budget_workspace_bytes.argtypes = [pp]
        L.paro_route_budget_workspace_bytes.restype = sz
        L.paro_attention_csr.argtypes = [pp, vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, vp, vp, sz, vp]
        L.paro_attention_csr.restype = ctypes.c_int
        gp = ctypes.POINTER(ParoGrid)
        L.paro_reorder.argtypes = [pp, gp, i32, vp, vp, vp]
        L.paro_reorder.restype = ctypes.c_int
        L.paro_reorder_source.argtypes = [gp, i32, i32]
        L.paro_reorder_source.restype = i32
        L.paro_num_blocks.argtypes = [i32, i32]
        L.paro_num_blocks.restype = i32
        L.paro_status_string.argtypes = [ctypes.c_int]
        L.paro_status_string.restype = ctypes.c_char_p
        L.paro_version.argtypes = []
        L.paro_version.restype = ctypes.c_int
        _LIB = L
    return _LIB


def _check(rc: int, where: str):
    if rc != PARO_OK:
        raise ParoError(rc, where)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return PARO_DTYPE_BF16
    if t.dtype == torch.float32:
        return PARO_DTYPE_FP32
    raise TypeError(f"unsupported dtype {t.dtype} (bf16 or fp32)")


def problem(q: torch.Tensor, scale: float | None = None, block: int = BLOCK) -> ParoProblem:
    """Problem descriptor for a [B, H, L, d] tensor."""
    if q.dim() != 4:
        raise ValueError("expected a [B, H, L, d] tensor")
    B, H, L, d = q.shape
    s = 1.0 / math.sqrt(d) if scale is None else float(scale)
    return ParoProblem(B, H, L, d, block, _dtype_code(q), s)


def _dev(t: torch.Tensor, name: str, dtype=None) -> int:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    return t.data_ptr()


def _shape(t: torch.Tensor, name: str, shape, ref: torch.Tensor | None = None) -> None:
    """Shape (and device) check done before any call into the library: the C
    ABI receives bare pointers and cannot check buffer sizes itself."""
    if tuple(t.shape) != tuple(int(x) for x in shape):
        raise ValueError(f"{name} must have shape {tuple(int(x) for x in shape)}, got {tuple(t.shape)}")
    if ref is not None and t.device != ref.device:
        raise ValueError(f"{name} is on {t.device}, expected {ref.device}")


def _bytes_at_least(t: torch.Tensor, name: str, need: int) -> int:
    n = t.numel() * t.element_size()
    if n < need:
        raise ValueError(f"{name} holds {n} bytes, the call needs {need}")
    return n


def _dims(q: torch.Tensor):
    """(B, H, L, d, T) of a [B, H, L, d] tensor."""
    if q.dim() != 4:
        raise ValueError(f"expected a [B, H, L, d] tensor, got shape {tuple(q.shape)}")
    B, H, L, d = q.shape
    return B, H, L, d, -(-L // BLOCK)


def _stats_shapes(ref: torch.Tensor, kbar, vsum, Hbar, M) -> None:
    B, H, L, d, T = _dims(ref)
    if kbar is not None:
        _shape(kbar, "kbar", (B, H, T, d), ref)
    if vsum is not None:
        _shape(vsum, "vsum", (B, H, T, d), ref)
    if Hbar is not None:
        _shape(Hbar, "Hbar", (B, H, d, d), ref)
    if M is not None:
        _shape(M, "M", (B, H, T), ref)


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def num_blocks(L: int, block: int = BLOCK) -> int:
    return int(lib().paro_num_blocks(L, block))


def workspace_bytes(p: ParoProblem) -> int:
    return int(lib().paro_precompute_workspace_bytes(ctypes.byref(p)))


def alloc_stats(k: torch.Tensor, block: int = BLOCK):
    """Allocate (kbar, vsum, Hbar, M, workspace) for a [B, H, L, d] key tensor."""
    B, H, L, d = k.shape
    T = -(-L // block)
    dev = k.device
    p = problem(k, block=block)
    ws = torch.empty(max(16, workspace_bytes(p)), dtype=torch.uint8, device=dev)
    return (torch.empty(B, H, T, d, dtype=torch.float32, device=dev),
            torch.empty(B, H, T, d, dtype=torch.float32, device=dev),
            torch.empty(B, H, d, d, dtype=torch.float32, device=dev),
            torch.empty(B, H, T, dtype=torch.float64, device=dev),
            ws)


def precompute(k: torch.Tensor, v: torch.Tensor, out=None, scale: float | None = None):
    """Block statistics (kbar, vsum, Hbar, M) of [B, H, L, d] keys and values."""
    p = problem(k, scale)
    kbar, vsum, Hbar, M, ws = alloc_stats(k) if out is None else out
    _shape(v, "v", k.shape, k)
    _stats_shapes(k, kbar, vsum, Hbar, M)
    _bytes_at_least(ws, "workspace", workspace_bytes(p))
    _check(lib().paro_precompute(
        ctypes.byref(p), _dev(k, "k"), _dev(v, "v", k.dtype), _dev(kbar, "kbar", torch.float32),
        _dev(vsum, "vsum", torch.float32), _dev(Hbar, "Hbar", torch.float32),
        _dev(M, "M", torch.float64), _dev(ws, "workspace"), ws.numel() * ws.element_size(),
        _stream()), "paro_precompute")
    return kbar, vsum, Hbar, M


def route(q: torch.Tensor, kbar: torch.Tensor, M: torch.Tensor, keep_k: int, lam: float,
          scale: float | None = None, out: torch.Tensor | None = None) -> torch.Tensor:
    """Top-keep_k kv-block indices [B, H, T, keep_k] (int32, ascending per row)."""
    p = problem(q, scale)
    B, H, L, d, T = _dims(q)
    if not 0 <= keep_k <= T:
        raise ValueError(f"keep_k must be in [0, {T}], got {keep_k}")
    _stats_shapes(q, kbar, None, None, M)
    idx = torch.empty(B, H, T, keep_k, dtype=torch.int32, device=q.device) if out is None else out
    _shape(idx, "idx", (B, H, T, keep_k), q)
    ptr = _dev(idx, "idx", torch.int32) if keep_k > 0 else None
    _check(lib().paro_route(ctypes.byref(p), _dev(q, "q"), _dev(kbar, "kbar", torch.float32),
                            _dev(M, "M", torch.float64), int(keep_k), float(lam), ptr, _stream()),
           "paro_route")
    return idx


TAIL_PISA, TAIL_DROP, TAIL_ZEROTH = 0, 1, 2


def attention_workspace_bytes(p: ParoProblem) -> int:
    return int(lib().paro_attention_workspace_bytes(ctypes.byref(p)))


def attention_fp8_workspace_bytes(p: ParoProblem) -> int:
    return int(lib().paro_attention_fp8_workspace_bytes(ctypes.byref(p)))


def fp8_rows(x: torch.Tensor):
    """e4m3 rows of x [..., d] (bf16 or fp32, d in {64, 128}) with one
    power-of-two scale per row: returns (codes uint8 [..., d], scales uint8
    [...], the E8M0 codes e + 127)."""
    d = x.shape[-1]
    n = x.numel() // d
    codes = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    sc = torch.empty(x.shape[:-1], dtype=torch.uint8, device=x.device)
    _check(lib().paro_fp8_rows(_dev(x, "x"), _dtype_code(x), n, d, _dev(codes, "codes"), _dev(sc, "scales"),
                               _stream()), "paro_fp8_rows")
    return codes, sc


def attention(q, k, v, kbar, vsum, Hbar, idx, keep_k: int, scale: float | None = None,
              out: torch.Tensor | None = None, drop_tail: bool = False,
              first_order: bool = True, workspace: torch.Tensor | None = None,
              qk_fp8: bool = False) -> torch.Tensor:
    """Piecewise attention output [B, H, L, d] in the dtype of q.

    drop_tail=True drops U_i instead of approximating it (keep-or-drop
    sparse attention, the exact phase alone); first_order=False keeps the
    zeroth-order tail but leaves out the first-order correction. workspace:
    a device byte buffer of at least attention_workspace_bytes (allocated
    here when not given). qk_fp8=True (bf16 only) takes the key-query
    products on the fp8 matrix cores (paro_attention_fp8)."""
    p = problem(q, scale)
    B, H, L, d, T = _dims(q)
    if not 0 <= keep_k <= T:
        raise ValueError(f"keep_k must be in [0, {T}], got {keep_k}")
    _shape(k, "k", q.shape, q)
    _shape(v, "v", q.shape, q)
    _stats_shapes(q, kbar, vsum, Hbar, None)
    if keep_k > 0:
        _shape(idx, "idx", (B, H, T, keep_k), q)
    o = torch.empty_like(q) if out is None else out
    _shape(o, "out", q.shape, q)
    mode = TAIL_DROP if drop_tail else (TAIL_PISA if first_order else TAIL_ZEROTH)
    if qk_fp8:
        nws = attention_fp8_workspace_bytes(p)
        if workspace is None:
            workspace = torch.empty(max(16, nws), dtype=torch.uint8, device=q.device)
        _bytes_at_least(workspace, "workspace", nws)
        ptr = _dev(idx, "idx", torch.int32) if keep_k > 0 else None
        _check(lib().paro_attention_fp8(
            ctypes.byref(p), _dev(q, "q"), _dev(k, "k", q.dtype), _dev(v, "v", q.dtype),
            _dev(kbar, "kbar", torch.float32), _dev(vsum, "vsum", torch.float32),
            _dev(Hbar, "Hbar", torch.float32), ptr, int(keep_k), mode, _dev(o, "o", q.dtype),
            _dev(workspace, "workspace"), workspace.numel() * workspace.element_size(), _stream()),
            "paro_attention_fp8")
        return o
    nws = attention_workspace_bytes(p)
    if nws > 0 and workspace is None:
        workspace = torch.empty(nws, dtype=torch.uint8, device=q.device)
    wbytes = _bytes_at_least(workspace, "workspace", nws) if workspace is not None else 0
    wptr = _dev(workspace, "workspace") if nws > 0 else None
    ptr = _dev(idx, "idx", torch.int32) if keep_k > 0 else None
    _check(lib().paro_attention_mode(
        ctypes.byref(p), _dev(q, "q"), _dev(k, "k", q.dtype), _dev(v, "v", q.dtype),
        _dev(kbar, "kbar", torch.float32), _dev(vsum, "vsum", torch.float32),
        _dev(Hbar, "Hbar", torch.float32), ptr, int(keep_k), mode,
        _dev(o, "o", q.dtype), wptr, wbytes, _stream()), "paro_attention_mode")
    return o


def attention_noalloc(q, k, v, kbar, vsum, Hbar, idx, keep_k: int, out: torch.Tensor, scale: float | None = None,
                      drop_tail: bool = False, first_order: bool = True) -> torch.Tensor:
    """paro_attention_noalloc: the attention with its workspace in the
    library's static device scratch (nothing allocated by the library or
    here: the caller passes `out`). Calls that overlap on one GPU race on
    that scratch."""
    p = problem(q, scale)
    B, H, L, d, T = _dims(q)
    if not 0 <= keep_k <= T:
        raise ValueError(f"keep_k must be in [0, {T}], got {keep_k}")
    _shape(k, "k", q.shape, q)
    _shape(v, "v", q.shape, q)
    _stats_shapes(q, kbar, vsum, Hbar, None)
    if keep_k > 0:
        _shape(idx, "idx", (B, H, T, keep_k), q)
    _shape(out, "out", q.shape, q)
    mode = TAIL_DROP if drop_tail else (TAIL_PISA if first_order else TAIL_ZEROTH)
    ptr = _dev(idx, "idx", torch.int32) if keep_k > 0 else None
    _check(lib().paro_attention_noalloc(
        ctypes.byref(p), _dev(q, "q"), _dev(k, "k", q.dtype), _dev(v, "v", q.dtype),
        _dev(kbar, "kbar", torch.float32), _dev(vsum, "vsum", torch.float32),
        _dev(Hbar, "Hbar", torch.float32), ptr, int(keep_k), mode, _dev(out, "out", q.dtype), _stream()),
        "paro_attention_noalloc")
    return out


def route_budget(q, kbar, M, k_total: int, k_min: int = 1, lam: float = 0.1, scale: float | None = None,
                 out=None):
    """Per-query-block budgets: returns (offsets [B, H, T + 1] int32, idx [B, H, k_total] int32,
    weights [B, H, T] int64 = w * 2^16). Row i of head h is idx[h][offsets[h][i]:offsets[h][i + 1]].
    out: optional (offsets, idx, weights, workspace) buffers of those shapes (and at least
    paro_route_budget_workspace_bytes bytes of workspace)."""
    p = problem(q, scale)
    B, H, L, d, T = _dims(q)
    _stats_shapes(q, kbar, None, None, M)
    nws = int(lib().paro_route_budget_workspace_bytes(ctypes.byref(p)))
    if out is None:
        offsets = torch.empty(B, H, T + 1, dtype=torch.int32, device=q.device)
        idx = torch.zeros(B, H, max(1, k_total), dtype=torch.int32, device=q.device)
        wq = torch.empty(B, H, T, dtype=torch.int64, device=q.device)
        ws = torch.empty(max(16, nws), dtype=torch.uint8, device=q.device)
    else:
        offsets, idx, wq, ws = out
    _shape(offsets, "offsets", (B, H, T + 1), q)
    _shape(idx, "idx", (B, H, max(1, k_total)), q)
    _shape(wq, "weights", (B, H, T), q)
    _bytes_at_least(ws, "workspace", nws)
    _check(lib().paro_route_budget(ctypes.byref(p), _dev(q, "q"), _dev(kbar, "kbar", torch.float32),
                                   _dev(M, "M", torch.float64), int(k_total), int(k_min), float(lam),
                                   _dev(wq, "weights", torch.int64),
                                   _dev(offsets, "offsets", torch.int32), _dev(idx, "idx", torch.int32),
                                   _dev(ws, "workspace"), ws.numel() * ws.element_size(), _stream()),
           "paro_route_budget")
    return offsets, idx, wq


def attention_csr(q, k, v, kbar, vsum, Hbar, offsets, idx, k_stride: int, scale: float | None = None,
                  out: torch.Tensor | None = None, drop_tail: bool = False, first_order: bool = True,
                  workspace: torch.Tensor | None = None) -> torch.Tensor:
    """paro_attention_csr: exact lists of any lengths (offsets [B, H, T + 1], idx [B, H, k_stride])."""
    p = problem(q, scale)
    B, H, L, d, T = _dims(q)
    _shape(k, "k", q.shape, q)
    _shape(v, "v", q.shape, q)
    _stats_shapes(q, kbar, vsum, Hbar, None)
    _shape(offsets, "offsets", (B, H, T + 1), q)
    if k_stride < 0:
        raise ValueError(f"k_stride must be >= 0, got {k_stride}")
    _shape(idx, "idx", (B, H, k_stride), q)
    o = torch.empty_like(q) if out is None else out
    _shape(o, "out", q.shape, q)
    nws = attention_workspace_bytes(p)
    if nws > 0 and workspace is None:
        workspace = torch.empty(nws, dtype=torch.uint8, device=q.device)
    wbytes = _bytes_at_least(workspace, "workspace", nws) if workspace is not None else 0
    wptr = _dev(workspace, "workspace") if nws > 0 else None
    mode = TAIL_DROP if drop_tail else (TAIL_PISA if first_order else TAIL_ZEROTH)
    _check(lib().paro_attention_csr(
        ctypes.byref(p), _dev(q, "q"), _dev(k, "k", q.dtype), _dev(v, "v", q.dtype),
        _dev(kbar, "kbar", torch.float32), _dev(vsum, "vsum", torch.float32), _dev(Hbar, "Hbar", torch.float32),
        _dev(offsets, "offsets", torch.int32), _dev(idx, "idx", torch.int32), int(k_stride), mode,
        _dev(o, "o", q.dtype), wptr, wbytes, _stream()), "paro_attention_csr")
    return o


def keep_to_k(keep: float, T: int) -> int:
    """Kept fraction -> block count, k = ceil(keep * T) (integer-exact for permille fractions)."""
    return min(T, max(0, -(-round(keep * 1000) * T // 1000)))


def grid_spec(grid, tile) -> ParoGrid:
    """paro_grid for a (t, y, x) latent grid cut into (tile_t, tile_y, tile_x) boxes."""
    (t, y, x), (tt, ty, tx) = grid, tile
    return ParoGrid(int(t), int(y), int(x), int(tt), int(ty), int(tx))


def reorder(x: torch.Tensor, grid, tile, inverse: bool = False,
            out: torch.Tensor | None = None) -> torch.Tensor:
    """Token rows of x [B, H, L, d] in the tiled order of the (t, y, x) grid
    (inverse=False), or back to raster order (inverse=True). The first
    t*y*x tokens are the grid in raster order; later tokens keep their places."""
    p = problem(x)
    g = grid_spec(grid, tile)
    y = torch.empty_like(x) if out is None else out
    if y.shape != x.shape or y.dtype != x.dtype:
        raise ValueError("out must match x in shape and dtype")
    _check(lib().paro_reorder(ctypes.byref(p), ctypes.byref(g),
                              REORDER_SCATTER if inverse else REORDER_GATHER,
                              _dev(x, "x"), _dev(y, "out"), _stream()), "paro_reorder")
    return y


def reorder_source(grid, tile, L: int, i: int) -> int:
    """Raster index of the token at tiled position i (host-side, no GPU), -1 on bad input."""
    return int(lib().paro_reorder_source(ctypes.byref(grid_spec(grid, tile)), int(L), int(i)))


def pisa_attention(q, k, v, keep_k: int | None = None, keep: float | None = None, lam: float = 0.1,
                   scale: float | None = None, grid=None, tile=None) -> torch.Tensor:
    """Whole path: precompute, route and fused attention on the current stream.

    With grid and tile, the tokens are first moved into the tiled order of
    the latent grid (geometric reordering before blocking) and the output is
    moved back to the raster order of the inputs."""
    if (grid is None) != (tile is None):
        raise ValueError("grid and tile go together")
    if grid is not None:
        q, k, v = (reorder(t, grid, tile) for t in (q, k, v))
    T = -(-q.shape[2] // BLOCK)
    if keep_k is None:
        keep_k = keep_to_k(0.125 if keep is None else keep, T)
    kbar, vsum, Hbar, M = precompute(k, v, scale=scale)
    idx = route(q, kbar, M, keep_k, lam, scale=scale)
    o = attention(q, k, v, kbar, vsum, Hbar, idx, keep_k, scale=scale)
    return o if grid is None else reorder(o, grid, tile, inverse=True)
