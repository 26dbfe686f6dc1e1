"""The whole path at the largest problem the ABI accepts: T = PARO_MAX_BLOCKS
kv blocks (about a million tokens, a ragged last block).

At that size the attention kernel runs its largest LDS configuration (512
membership words, a union list of 16384 entries, 256 centroid chunks) and the
route kernel its smallest row groups (R = 2), both untouched by the smaller
workloads. The full oracle is too slow there, so the test uses inputs whose
result is known in closed form: every key is the same vector k0, and k0 and
V hold small integers, so that every product and sum the kernels form is
exact in fp32. Then

  * every block statistic is exact: kbar_j = k0, vsum_j = the block sums of V,
    H_j = 0, Hbar = 0 and M_j = 0 (PISA page, section 2, with the zeroth-order
    term exact for constant-key blocks);
  * all routing scores of a row are equal, so S_i = the first k blocks (ties
    go to the lower index);
  * each query's logits are all equal, so dense softmax attention is the plain
    mean of V over all L tokens, and PISA (exact part plus an exact
    zeroth-order tail) reproduces it.
"""
import pytest
import torch

from block_sparse_attention_pisa_amd import paro

from parity_util import ATTN_TOL, log

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("fp8", [False, True])
def test_max_blocks_uniform_logits(d, fp8):
    """d = 128 is the largest LDS footprint of the attention kernel (three
    staging buffers plus the lists of 16384 blocks). The fp8 key-query path
    rounds q to e4m3, but with every key equal all logits of a row stay
    equal, so its result is the same mean of V."""
    T, keep = 16384, 5
    L = 64 * T - 7
    g = torch.Generator().manual_seed(11)
    q = torch.randn(1, 1, L, d, generator=g).to(torch.bfloat16)
    k0 = torch.randint(-2, 3, (d,), generator=g).to(torch.bfloat16)
    k = k0.expand(1, 1, L, d).contiguous()
    v = torch.randint(-2, 3, (1, 1, L, d), generator=g).to(torch.bfloat16)
    log(f"[limits] T={T} L={L} d={d} keep={keep} fp8={fp8}")
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    kbar, vsum, Hbar, M = paro.precompute(kd, vd)
    idx = paro.route(qd, kbar, M, keep, 0.1)
    o = paro.attention(qd, kd, vd, kbar, vsum, Hbar, idx, keep, qk_fp8=fp8)
    torch.cuda.synchronize()

    # statistics
    assert torch.equal(kbar[0, 0].cpu(), k0.float().expand(T, d))
    vb = torch.nn.functional.pad(v[0, 0].double(), (0, 0, 0, 7)).view(T, 64, d).sum(1)
    assert torch.equal(vsum[0, 0].cpu().double(), vb)
    assert float(Hbar.abs().max()) == 0.0
    assert float(M.abs().max()) == 0.0
    # routing: all scores tie, so every row keeps blocks 0 .. keep - 1
    assert torch.equal(idx[0, 0].cpu(), torch.arange(keep, dtype=torch.int32).expand(T, keep))
    # attention: the mean of V for every query row
    ref = v[0, 0].double().mean(0)
    err = (o[0, 0].cpu().double() - ref).abs()
    tmax, tmean = ATTN_TOL["bf16"]
    log(f"[limits] attention max {float(err.max()):.3g} mean {float(err.mean()):.3g}")
    assert float(err.max()) <= tmax and float(err.mean()) <= tmean
