"""The Python binding checks every buffer's shape (and the workspace size)
before it calls into the library: the C ABI takes bare pointers and cannot
see a short buffer, which would become an out-of-bounds device access.

These run on the CPU: every call here must fail in the shape check, which
comes before any pointer is taken (a host tensor that passed the shape
checks would fail later with a different message, "must be a device
tensor"), so nothing is launched.
"""
import os

import pytest
import torch

from block_sparse_attention_pisa_amd import paro

pytestmark = pytest.mark.skipif(not os.path.exists(paro.LIB_PATH), reason="libparo.so not built")

B, H, L, d = 1, 2, 200, 64
T = -(-L // 64)


def _qkv():
    q = torch.zeros(B, H, L, d, dtype=torch.bfloat16)
    return q, q.clone(), q.clone()


def _stats():
    return (torch.zeros(B, H, T, d), torch.zeros(B, H, T, d), torch.zeros(B, H, d, d),
            torch.zeros(B, H, T, dtype=torch.float64))


def _ws(n):
    return torch.zeros(n, dtype=torch.uint8)


def test_precompute_shapes():
    q, k, v = _qkv()
    kbar, vsum, Hbar, M = _stats()
    ws = _ws(paro.workspace_bytes(paro.problem(k)))
    with pytest.raises(ValueError, match="v must have shape"):
        paro.precompute(k, v[:, :, :-1])
    for i, (name, bad) in enumerate((("kbar", torch.zeros(B, H, T - 1, d)), ("vsum", torch.zeros(B, H, T, 2 * d)),
                                     ("Hbar", torch.zeros(B, H, d, d - 1)),
                                     ("M", torch.zeros(B, H, T + 1, dtype=torch.float64)))):
        out = [kbar, vsum, Hbar, M, ws]
        out[i] = bad
        with pytest.raises(ValueError, match=f"{name} must have shape"):
            paro.precompute(k, v, out=tuple(out))
    with pytest.raises(ValueError, match="workspace holds"):
        paro.precompute(k, v, out=(kbar, vsum, Hbar, M, _ws(16)))
    with pytest.raises(ValueError, match="expected a \\[B, H, L, d\\] tensor"):
        paro.precompute(k[0], v[0])


def test_route_shapes():
    q, _, _ = _qkv()
    kbar, _, _, M = _stats()
    with pytest.raises(ValueError, match="keep_k must be in"):
        paro.route(q, kbar, M, T + 1, 0.1)
    with pytest.raises(ValueError, match="kbar must have shape"):
        paro.route(q, kbar[:, :1], M, 2, 0.1)
    with pytest.raises(ValueError, match="M must have shape"):
        paro.route(q, kbar, M[..., :-1], 2, 0.1)
    with pytest.raises(ValueError, match="idx must have shape"):
        paro.route(q, kbar, M, 2, 0.1, out=torch.zeros(B, H, T, 1, dtype=torch.int32))


def test_attention_shapes():
    q, k, v = _qkv()
    kbar, vsum, Hbar, _ = _stats()
    idx = torch.zeros(B, H, T, 2, dtype=torch.int32)
    with pytest.raises(ValueError, match="k must have shape"):
        paro.attention(q, k[:, :1], v, kbar, vsum, Hbar, idx, 2)
    with pytest.raises(ValueError, match="v must have shape"):
        paro.attention(q, k, v[..., :32], kbar, vsum, Hbar, idx, 2)
    with pytest.raises(ValueError, match="vsum must have shape"):
        paro.attention(q, k, v, kbar, vsum[:, :, :-1], Hbar, idx, 2)
    with pytest.raises(ValueError, match="idx must have shape"):
        paro.attention(q, k, v, kbar, vsum, Hbar, idx[..., :1], 2)   # fewer than keep_k columns
    with pytest.raises(ValueError, match="idx must have shape"):
        paro.attention(q, k, v, kbar, vsum, Hbar, idx, 3)
    with pytest.raises(ValueError, match="keep_k must be in"):
        paro.attention(q, k, v, kbar, vsum, Hbar, idx, -1)
    with pytest.raises(ValueError, match="out must have shape"):
        paro.attention(q, k, v, kbar, vsum, Hbar, idx, 2, out=torch.zeros(B, H, L - 1, d, dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="workspace holds"):
        paro.attention(q, k, v, kbar, vsum, Hbar, idx, 2, workspace=_ws(16))
    with pytest.raises(ValueError, match="workspace holds"):
        paro.attention(q, k, v, kbar, vsum, Hbar, idx, 2, workspace=_ws(16), qk_fp8=True)


def test_csr_and_budget_shapes():
    q, k, v = _qkv()
    kbar, vsum, Hbar, M = _stats()
    offs = torch.zeros(B, H, T + 1, dtype=torch.int32)
    idx = torch.zeros(B, H, 7, dtype=torch.int32)
    with pytest.raises(ValueError, match="offsets must have shape"):
        paro.attention_csr(q, k, v, kbar, vsum, Hbar, offs[..., :-1], idx, 7)
    with pytest.raises(ValueError, match="idx must have shape"):
        paro.attention_csr(q, k, v, kbar, vsum, Hbar, offs, idx, 8)    # stride larger than the buffer
    with pytest.raises(ValueError, match="k_stride must be"):
        paro.attention_csr(q, k, v, kbar, vsum, Hbar, offs, idx, -1)
    with pytest.raises(ValueError, match="kbar must have shape"):
        paro.route_budget(q, kbar[..., :8], M, 2 * T)
