"""Helpers shared by the GPU parity tests: run the HIP path, run the oracle, compare."""
from __future__ import annotations

import math
import sys

import numpy as np
import torch

from block_sparse_attention_pisa_amd import paro
from oracle import pisa

# acceptance thresholds
ROUTE_GAP = 1e-5          # score gap under which a different top-k choice is excused
M_ABS_TOL = 2e-5          # |M_gpu - M_oracle|
ATTN_TOL = {"bf16": (1e-2, 1e-3), "fp32": (1e-5, 1e-5)}   # (max abs, mean abs)


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev(*ts):
    return [t.cuda() for t in ts]


def sample_qblocks(T: int, n: int = 24):
    if T <= n:
        return list(range(T))
    s = sorted(set(np.linspace(0, T - 1, n).round().astype(int).tolist()) | {T - 1, T - 2, 1})
    return s


def check_stats(gpu_stats, st, b, h, rtol=2e-6):
    """GPU precompute of one (b, h) against the oracle's fp64 statistics."""
    kbar, vsum, Hbar, M = (x[b, h].double().cpu().numpy() for x in gpu_stats)
    def rel(a, ref):
        return np.abs(a - ref).max() / max(1e-30, np.abs(ref).max())
    r_k, r_v, r_h = rel(kbar, st["kbar"]), rel(vsum, st["vsum"]), rel(Hbar, st["Hbar"])
    dM = np.abs(M - st["M"]).max()
    assert r_k < rtol, ("kbar", r_k)
    assert r_v < rtol, ("vsum", r_v)
    assert r_h < 2e-5, ("Hbar", r_h)
    assert dM <= M_ABS_TOL, ("M", dM, float(np.abs(st["M"]).max()))
    return dict(kbar=r_k, vsum=r_v, Hbar=r_h, M=dM)


def check_route(idx_gpu: np.ndarray, idx_ref: np.ndarray, score: np.ndarray, rows=None):
    """Bit-exact routing except rows whose swapped blocks are within ROUTE_GAP in oracle score."""
    rows = range(idx_ref.shape[0]) if rows is None else rows
    excused = 0
    for i in rows:
        a, b = set(idx_gpu[i].tolist()), set(idx_ref[i].tolist())
        assert list(idx_gpu[i]) == sorted(idx_gpu[i].tolist()), ("not ascending", i)
        assert len(a) == len(idx_gpu[i]), ("duplicate", i)
        if a == b:
            continue
        extra, missing = a - b, b - a
        gap = max(score[i, jm] - score[i, je] for je in extra for jm in missing)
        assert gap < ROUTE_GAP, ("routing mismatch", i, sorted(extra), sorted(missing), gap)
        excused += 1
    return excused


def check_attention(o_gpu: np.ndarray, o_ref: np.ndarray, dtype: str):
    err = np.abs(o_gpu - o_ref)
    mx, mean = float(err.max()), float(err.mean())
    tmax, tmean = ATTN_TOL[dtype]
    assert mx <= tmax and mean <= tmean, (dtype, mx, mean)
    return mx, mean


def run_gpu(q, k, v, keep_k, lam, scale=None):
    qd, kd, vd = to_dev(q, k, v)
    stats = paro.precompute(kd, vd, scale=scale)
    idx = paro.route(qd, stats[0], stats[3], keep_k, lam, scale=scale)
    torch.cuda.synchronize()
    return (qd, kd, vd), stats, idx


GATE = 0.1   # GPU-vs-oracle max error, as a share of the smallest gap between PISA and the alternatives


def fp8_operands(q, k, kbar, st, scale):
    """The operands the fp8 key-query path multiplies, as fp64 arrays of one
    (b, h): q' = bf16(q) * fp32(scale log2 e) rounded per query row (returned
    divided back by that factor), K rows and kbar rows rounded per row. kbar
    is the oracle's own fp64 centroid, taken to fp32 first (the precision the
    path stores it in); nothing here comes from the GPU."""
    from oracle import quant
    cl2 = np.float32(scale * 1.4426950408889634)
    x = q.float().numpy() * cl2
    qq = quant.dequantize_rows(*quant.quantize_rows(x)) / np.float64(cl2)
    kq = quant.dequantize_rows(*quant.quantize_rows(k.float().numpy()))
    stq = dict(st)
    stq["kbar"] = quant.dequantize_rows(*quant.quantize_rows(np.asarray(kbar, dtype=np.float64).astype(np.float32)))
    return qq, kq, stq


def full_parity(w, heads=None, qblocks=None, diag=True, qk_fp8=False, gate=GATE):
    """Run every stage on the GPU for workload w and compare with the oracle.

    heads: (b, h) pairs the oracle checks (all by default); qblocks: query
    blocks the oracle evaluates (all by default). The GPU always runs every
    head and query block, in the launch configuration the benchmark times.
    qk_fp8: the attention takes the fp8 key-query path.

    Two bars on the attention, both fed the oracle's routing:
      * against the exact fp64 oracle: the bf16 / fp32 tolerance;
      * (diag, when U_i is not empty) the discriminating gate: the GPU's
        largest error against the oracle's definition of what it computes
        (the exact oracle; for fp8 the oracle on the e4m3-rounded operands)
        must stay below `gate` times the smallest of the oracle's own gaps
        max |PISA - dense|, max |PISA - zeroth-order tail| and
        max |PISA - keep-or-drop| over the same rows, so that a kernel that
        silently computed one of those instead fails.
    """
    from workloads import make_inputs
    q, k, v = make_inputs(w)
    log(f"[parity] {w.name}: inputs {tuple(q.shape)} {q.dtype} keep_k={w.k} lam={w.lam} fp8={qk_fp8}")
    (qd, kd, vd), stats, idx = run_gpu(q, k, v, w.k, w.lam)
    idx_h = idx.cpu().numpy()
    pairs = [(b, h) for b in range(w.B) for h in range(w.H)] if heads is None else heads
    qn, kn, vn = (x.double().numpy() for x in (q, k, v))
    # oracle routing fed to the GPU attention
    ref = {}
    idx_or = torch.from_numpy(idx_h.copy())
    for b, h in pairs:
        st = pisa.block_stats(kn[b, h], vn[b, h], w.block)
        ir, sc = pisa.route(qn[b, h], st["kbar"], st["M"], w.k, w.lam, w.scale, w.block)
        ref[(b, h)] = (st, ir, sc)
        idx_or[b, h] = torch.from_numpy(ir.astype(np.int32))
    o = paro.attention(qd, kd, vd, stats[0], stats[1], stats[2], idx_or.cuda(), w.k,
                       qk_fp8=qk_fp8).float().cpu().numpy()
    summary = {"excused_rows": 0, "max_err": 0.0, "mean_err": 0.0, "gate_ratio": 0.0}
    errs = []
    rng_ = pisa.block_ranges(w.L, w.block)
    for b, h in pairs:
        st, ir, sc = ref[(b, h)]
        s = check_stats(stats, st, b, h)
        ex = check_route(idx_h[b, h], ir, sc)
        summary["excused_rows"] += ex
        T = st["kbar"].shape[0]
        qbs = list(range(T)) if qblocks is None else qblocks(T)
        oref = pisa.attention(qn[b, h], kn[b, h], vn[b, h], st, ir, w.scale, w.block, qblocks=qbs)
        og = np.concatenate([o[b, h, rng_[i][0]:rng_[i][1]] for i in qbs])
        orr = np.concatenate([oref[i] for i in qbs])
        mx, mean = check_attention(og, orr, w.dtype)
        errs.append(np.abs(og - orr))
        summary["max_err"] = max(summary["max_err"], mx)
        msg = ""
        if diag and w.k < T:
            rows = np.concatenate([np.arange(*rng_[i]) for i in qbs])
            dense = pisa.dense_attention(qn[b, h], kn[b, h], vn[b, h], w.scale, rows=rows)
            oz = pisa.attention(qn[b, h], kn[b, h], vn[b, h], st, ir, w.scale, w.block, qblocks=qbs,
                                first_order="none")
            od = pisa.attention(qn[b, h], kn[b, h], vn[b, h], st, ir, w.scale, w.block, qblocks=qbs, tail=False)
            gaps = {"dense": float(np.abs(orr - dense).max()),
                    "zeroth": float(np.abs(orr - np.concatenate([oz[i] for i in qbs])).max()),
                    "drop": float(np.abs(orr - np.concatenate([od[i] for i in qbs])).max())}
            if qk_fp8:
                qq, kq, stq = fp8_operands(q[b, h], k[b, h], st["kbar"], st, w.scale)
                odef = pisa.attention(qq, kq, vn[b, h], stq, ir, w.scale, w.block, qblocks=qbs)
                e_def = float(np.abs(og - np.concatenate([odef[i] for i in qbs])).max())
            else:
                e_def = mx
            gmin = min(gaps.values())
            # a kernel computing dense, zeroth-order or keep-or-drop attention by mistake fails here
            assert e_def <= gate * gmin, ("indistinct from an alternative", e_def, gaps)
            summary["gate_ratio"] = max(summary["gate_ratio"], e_def / gmin)
            for kx, vx in gaps.items():
                summary.setdefault(f"pisa_vs_{kx}_max", []).append(vx)
            msg = f" gaps {gaps} err/gap {e_def / gmin:.3g}"
        log(f"[parity] {w.name} b{b}h{h}: stats {s} excused {ex} attn max {mx:.3g} mean {mean:.3g}{msg}")
    summary["mean_err"] = float(np.concatenate([e.ravel() for e in errs]).mean())
    return summary
