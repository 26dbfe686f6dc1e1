#!/usr/bin/env python3
"""Benchmark of the PISA hot path on one MI355X.

One step = paro_precompute + paro_route + paro_attention over one batch of
synthetic DiT-shaped input already resident in HBM. The default workload is
the 720p video shape (B=1, 40 heads, 75,600 tokens, d=128, bf16, 12.5% of
the kv-blocks exact). Prints one JSON line:
  value      dense-equivalent TFLOP/s = 4 B H L^2 d / step time
  roofline   the attention kernel against the bf16 MFMA peak, from its
             algorithmic FLOPs (exact blocks + zeroth-order terms of U_i +
             correction) over its mean launch time measured with HIP events
  exact_phase   the same attention kernel on the all-exact (keep = 100%)
                control of the long-video shape, against the bf16 MFMA peak
  fp8           the same step with the key-query products on the fp8 matrix
                cores (paro_attention_fp8): step time, dense-equivalent
                TFLOP/s, and the attention against the mixed peak (the
                key-query half of the FLOPs at the fp8 rate, the rest at the
                bf16 rate); reported beside the bf16 headline, never as it
  budget        per-query-block budgets: paro_route_budget with the same
                total (keep_k T blocks per head, at least one per row) and
                paro_attention_csr on its lists; times and the spread of k_i
  reorder       the geometric token reordering (paro_reorder) of one
                [B, H, L, d] tensor into the tiled order and back, against
                the HBM peak (one read and one write of every row)
  cpu_baseline  the fp64 oracle on a bounded sample of the same workload
  other_configs the image (4.6k tokens), 480p and long-video shapes: step,
                per-phase and cold times, attention against the bf16 peak
  measured_peaks  practical peaks of this GPU (MFMA chains, streaming read,
                device copy); the headline fractions are also given against them
  precompute_kernels  per-kernel times of one step (torch.profiler): block
                statistics against the HBM peak, the spectral kernel against
                the fp32 VALU peak (nominal 8 Lanczos steps per block)
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_FP8_TFLOPS = 5000.0      # MI355X dense fp8 MFMA
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
PEAK_FP32_VALU_TFLOPS = 78.6   # MI355X fp32 vector FMA without packed-fp32 instructions (the build disables them)
PEAK_FP32_MFMA_TFLOPS = 157.3  # MI355X dense fp32 MFMA
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attention_traffic_video720p_75600.json")
ATTN_SRCS = [os.path.join(ROOT, "block_sparse_attention_pisa_amd", "csrc", f)
             for f in ("paro_attention.hip", "paro_common.h")]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="video720p_75600")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-exact-phase", action="store_true",
                    help="skip the all-exact control run that isolates the exact phase")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the 480p and long-video steps (the other shapes of the metric)")
    ap.add_argument("--no-ablation", action="store_true",
                    help="skip the error-against-dense table of the method and its ablations")
    ap.add_argument("--no-peaks", action="store_true", help="skip the measured practical peaks")
    ap.add_argument("--no-split", action="store_true", help="skip the per-kernel profiler split of one step")
    ap.add_argument("--cpu-qblocks", type=int, default=48, help="query blocks per head in the oracle sample")
    ap.add_argument("--cpu-heads", type=int, default=1)
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="only run a device-to-device copy of this many MiB (scales the HBM byte counters)")
    return ap.parse_args()


def attention_flops(w, idx_cpu, with_exact: bool = False):
    """Algorithmic FLOPs of one attention launch.

    Exact part 4 d sum_i n_i sum_{j in S_i} n_j (QK^T and PV), zeroth-order
    part 4 d sum_i n_i |U_i| (one centroid logit and one value-sum product
    per tail block), correction 2 d^2 L per head (q' Hbar).
    """
    import numpy as np
    T, L, d, blk = w.T, w.L, w.d, w.block
    n = np.full(T, blk, dtype=np.int64)
    n[-1] = L - blk * (T - 1)
    per_head = 0.0
    idx = idx_cpu.reshape(-1, T, w.k) if w.k else None
    heads = w.B * w.H
    total = 0.0
    exact_total = 0.0
    for h in range(heads):
        if w.k:
            sel_tokens = n[idx[h]].sum(axis=1)           # sum_{j in S_i} n_j per row i
        else:
            sel_tokens = np.zeros(T, dtype=np.int64)
        exact = 4.0 * d * float((n * sel_tokens).sum())
        tail = 4.0 * d * float((n * (T - w.k)).sum())
        corr = 2.0 * d * d * L if w.k < T else 0.0
        total += exact + tail + corr
        exact_total += exact
    return (total, exact_total) if with_exact else total


def exact_phase_entry(reps: int = 5):
    """The exact phase alone: the same attention kernel on the keep = 100% control
    of the long-video shape (every kv-block exact, no tail, no correction), so
    every MFMA is stage-1 work. FLOPs 4 d sum_i n_i L per head."""
    import torch
    from block_sparse_attention_pisa_amd import paro
    from workloads import WORKLOADS, make_inputs
    w = WORKLOADS["video_long_118800_dense"]
    q, k, v = make_inputs(w)
    qd, kd, vd = (x.to("cuda:0") for x in (q, k, v))
    del q, k, v
    stats = paro.precompute(kd, vd)
    idx = paro.route(qd, stats[0], stats[3], w.k, w.lam)
    out = torch.empty_like(qd)
    attn_ws = torch.empty(max(16, paro.attention_workspace_bytes(paro.problem(qd))), dtype=torch.uint8,
                          device=qd.device)
    stream = torch.cuda.current_stream()
    paro.attention(qd, kd, vd, *stats[:3], idx, w.k, out=out, workspace=attn_ws)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record(stream)
    for _ in range(reps):
        paro.attention(qd, kd, vd, *stats[:3], idx, w.k, out=out, workspace=attn_ws)
    ev[1].record(stream)
    torch.cuda.synchronize()
    ms = ev[0].elapsed_time(ev[1]) / reps
    flops = 4.0 * w.B * w.H * w.L * w.L * w.d
    tf = flops / (ms * 1e-3) / 1e12
    return {"workload": w.name, "keep_k": w.k, "T": w.T, "ms": round(ms, 3), "achieved": round(tf, 2),
            "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(tf / PEAK_BF16_TFLOPS, 4)}


def traffic_entry():
    """HBM bytes per attention launch from committed counter runs, if the kernel is unchanged."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
        sha = hashlib.sha256(b"".join(open(f, "rb").read() for f in ATTN_SRCS)).hexdigest()
        if rec.get("source_sha256") != sha:
            return None
        return rec["hbm_bytes_per_launch"]
    except Exception:
        return None


def reorder_entry(w, x, out, reps: int = 5):
    """paro_reorder of x [B, H, L, d] into the tiled order of the workload's
    latent grid (gather) and back (scatter); algorithmic bytes = one read and
    one write of the tensor."""
    import torch
    from block_sparse_attention_pisa_amd import paro
    tile = (1, 8, 8) if w.grid[0] == 1 else (2, 4, 8)
    stream = torch.cuda.current_stream()
    nbytes = 2.0 * x.numel() * x.element_size()
    res = {"tile_txy": list(tile), "bytes_per_call": nbytes}
    for name, inv in (("gather", False), ("scatter", True)):
        paro.reorder(x, w.grid, tile, inverse=inv, out=out)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record(stream)
        for _ in range(reps):
            paro.reorder(x, w.grid, tile, inverse=inv, out=out)
        ev[1].record(stream)
        torch.cuda.synchronize()
        ms = ev[0].elapsed_time(ev[1]) / reps
        gbs = nbytes / (ms * 1e-3) / 1e9
        res[name] = {"ms": round(ms, 4), "GBs": round(gbs, 1), "frac_of_hbm_peak": round(gbs / PEAK_HBM_GBS, 4)}
    return res


def fp8_entry(w, qd, kd, vd, stats, idx, out, attn_flops, exact_flops, reps: int = 3):
    """The step with paro_attention_fp8: q', K and kbar in e4m3 for the
    key-query products. Half of the exact and of the tail FLOPs are
    key-query products (fp8 rate), the other half and the correction run at
    the bf16 rate; the mixed-peak time is their sum at those rates."""
    import torch
    from block_sparse_attention_pisa_amd import paro
    stream = torch.cuda.current_stream()
    ws8 = torch.empty(paro.attention_fp8_workspace_bytes(paro.problem(qd)), dtype=torch.uint8, device=qd.device)

    def attn(drop=False):
        paro.attention(qd, kd, vd, stats[0], stats[1], stats[2], idx, w.k, out=out, drop_tail=drop, qk_fp8=True,
                       workspace=ws8)

    def step():
        paro.precompute(kd, vd, out=stats)
        paro.route(qd, stats[0], stats[3], w.k, w.lam, out=idx)
        attn()

    def timed(fn):
        fn()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record(stream)
        for _ in range(reps):
            fn()
        ev[1].record(stream)
        torch.cuda.synchronize()
        return ev[0].elapsed_time(ev[1]) / reps

    step_ms = timed(step)
    attn_ms = timed(attn)
    drop_ms = timed(lambda: attn(True))
    dense_flops = 4.0 * w.B * w.H * w.L * w.L * w.d
    qk = (attn_flops - 2.0 * w.d * w.d * w.L * w.B * w.H) / 2.0   # key-query half of exact + tail
    ideal_attn = qk / (PEAK_FP8_TFLOPS * 1e12) + (attn_flops - qk) / (PEAK_BF16_TFLOPS * 1e12)
    ideal_exact = exact_flops / 2.0 / (PEAK_FP8_TFLOPS * 1e12) + exact_flops / 2.0 / (PEAK_BF16_TFLOPS * 1e12)
    return {
        "ms_per_step": round(step_ms, 4),
        "value": round(dense_flops / (step_ms * 1e-3) / 1e12, 2), "unit": "TFLOP/s (dense-equivalent)",
        "attention_ms": round(attn_ms, 4),
        "attention_achieved": round(attn_flops / (attn_ms * 1e-3) / 1e12, 2),
        "attention_frac_of_mixed_peak": round(ideal_attn * 1e3 / attn_ms, 4),
        "exact_phase_ms": round(drop_ms, 4),
        "exact_phase_frac_of_mixed_peak": round(ideal_exact * 1e3 / drop_ms, 4),
        "note": "q', K and kbar rounded to e4m3 (per-row power-of-two scales); parity-tested at the bf16 bar",
    }


def budget_entry(w, qd, kd, vd, stats, out, reps: int = 3):
    """paro_route_budget (the fixed-k total, k_min = 1) and paro_attention_csr."""
    import torch
    from block_sparse_attention_pisa_amd import paro
    stream = torch.cuda.current_stream()
    K = w.k * w.T
    res = {}

    def timed(fn):
        fn()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record(stream)
        for _ in range(reps):
            r = fn()
        ev[1].record(stream)
        torch.cuda.synchronize()
        return ev[0].elapsed_time(ev[1]) / reps, r

    route_ms, (offsets, idx, _) = timed(lambda: paro.route_budget(qd, stats[0], stats[3], K, 1, w.lam))
    attn_ms, _ = timed(lambda: paro.attention_csr(qd, kd, vd, stats[0], stats[1], stats[2], offsets, idx, K, out=out))
    kk = torch.diff(offsets.to(torch.int64), dim=-1)
    return {"k_total_per_head": K, "k_min": 1, "route_ms": round(route_ms, 4), "attention_ms": round(attn_ms, 4),
            "k_i_min": int(kk.min()), "k_i_max": int(kk.max())}


def configs_entry(names=("image_4608", "video480p_32760", "video_long_118800"), steps: int = 11,
                  warm_s: float = 0.1):
    """The other DiT shapes (the 4.6k-token image, and the 32k and 119k-token
    videos the metric spans), timed like the headline step: precompute +
    route + attention on one stream, inputs resident, HIP events around each
    phase (medians of `steps`) after warm-up steps worth about `warm_s`
    seconds (at least two): a step of a millisecond or less run after a few
    warm-up steps finds the shader clock below its steady-state rate. Cold:
    the median of 3 steps each after a 512 MB write that evicts L2 and
    MALL."""
    import torch
    from block_sparse_attention_pisa_amd import paro
    from workloads import WORKLOADS, make_inputs
    stream = torch.cuda.current_stream()
    out = {}
    for name in names:
        w = WORKLOADS[name]
        q, k, v = make_inputs(w)
        qd, kd, vd = (x.cuda() for x in (q, k, v))
        del q, k, v
        stats = paro.alloc_stats(kd)
        idx = torch.empty(w.B, w.H, w.T, w.k, dtype=torch.int32, device="cuda")
        o = torch.empty_like(qd)
        ws = torch.empty(max(16, paro.attention_workspace_bytes(paro.problem(qd))), dtype=torch.uint8, device="cuda")

        def step(ev=None):
            if ev:
                ev[0].record(stream)
            paro.precompute(kd, vd, out=stats)
            if ev:
                ev[1].record(stream)
            paro.route(qd, stats[0], stats[3], w.k, w.lam, out=idx)
            if ev:
                ev[2].record(stream)
            paro.attention(qd, kd, vd, stats[0], stats[1], stats[2], idx, w.k, out=o, workspace=ws)
            if ev:
                ev[3].record(stream)

        t_warm, n_warm = time.perf_counter(), 0
        while n_warm < 2 or time.perf_counter() - t_warm < warm_s:
            step()
            n_warm += 1
            if n_warm % 4 == 0:
                torch.cuda.synchronize()
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
        for e in evs:
            step(e)
        torch.cuda.synchronize()

        def med(a, b):
            return sorted(e[a].elapsed_time(e[b]) for e in evs)[steps // 2]
        ms, pre, rou, att = med(0, 3), med(0, 1), med(1, 2), med(2, 3)
        flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
        cold = []
        for i in range(3):
            flush.fill_(i & 255)
            cev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            cev[0].record(stream)
            step()
            cev[1].record(stream)
            torch.cuda.synchronize()
            cold.append(cev[0].elapsed_time(cev[1]))
        del flush
        flops = attention_flops(w, idx.cpu().numpy())
        kv_bytes = 2.0 * w.B * w.H * w.L * w.d * 2
        out[name] = {"L": w.L, "H": w.H, "keep_k": w.k, "T": w.T, "median_ms_per_step": round(ms, 4),
                     "dense_equiv_TFLOPs": round(4.0 * w.B * w.H * w.L * w.L * w.d / (ms * 1e-3) / 1e12, 1),
                     "phases_ms": {"precompute": round(pre, 4), "route": round(rou, 4), "attention": round(att, 4)},
                     "attention_ms": round(att, 4),
                     "attention_TFLOPs": round(flops / (att * 1e-3) / 1e12, 1),
                     "attention_frac_of_bf16_peak": round(flops / (att * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                     "precompute_frac_of_hbm_peak": round(kv_bytes / (pre * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                     "cold_ms_per_step": round(sorted(cold)[1], 4),
                     "warmup_steps": n_warm, "timed_steps": steps}
        del qd, kd, vd, stats, idx, o, ws
        torch.cuda.empty_cache()
    return out


def ablation_entry(name: str = "video480p_32760", permille=(50, 100, 125, 250, 500), tile=(2, 4, 8)):
    """Error against dense attention of the method and its two ablations,
    the zeroth-order tail alone and keep-or-drop, as a function of density
    (the paradigm contrast of the PISA page, sections 1 and 3), and of the
    method run on tokens moved into compact (t, y, x) boxes first (the
    geometric reordering of the PAROAttention page) or with the same total of
    exact blocks per head shared out by need (per-query-block budgets, the
    ALLOT review page). Dense attention is the
    fp32 pipeline on the same bf16 values with every block exact (keep_k = T
    leaves no tail). Error: relative Frobenius norm over all heads and rows,
    in fp32 on the device."""
    import torch
    from block_sparse_attention_pisa_amd import paro
    from workloads import WORKLOADS, make_inputs
    w = WORKLOADS[name]
    T = w.T
    q, k, v = make_inputs(w)
    q32, k32, v32 = (x.float().cuda() for x in (q, k, v))
    st32 = paro.precompute(k32, v32)
    dense = paro.attention(q32, k32, v32, st32[0], st32[1], st32[2],
                           paro.route(q32, st32[0], st32[3], T, w.lam), T)
    del q32, k32, v32, st32
    nd = float(dense.norm())
    qd, kd, vd = (x.cuda() for x in (q, k, v))
    stats = paro.precompute(kd, vd)
    qt, kt, vt = (paro.reorder(x, w.grid, tile) for x in (qd, kd, vd))
    stats_t = paro.precompute(kt, vt)
    tname = "pisa_tiled_" + "x".join(map(str, tile))
    rows = []
    for pm in permille:
        kk = -(-pm * T // 1000)
        idx = paro.route(qd, stats[0], stats[3], kk, w.lam)
        r = {"keep_permille": pm, "k": kk,
             "captured_mass": round(captured_mass(qd, kd, idx, w.scale, list(range(0, T, 8)) + [T - 1]), 4)}
        for mode, kw in (("pisa", {}), ("zeroth", {"first_order": False}), ("drop", {"drop_tail": True})):
            o = paro.attention(qd, kd, vd, stats[0], stats[1], stats[2], idx, kk, **kw)
            r[mode] = round(float((o.float() - dense).norm()) / nd, 6)
        idx_t = paro.route(qt, stats_t[0], stats_t[3], kk, w.lam)
        o_t = paro.attention(qt, kt, vt, stats_t[0], stats_t[1], stats_t[2], idx_t, kk)
        o = paro.reorder(o_t, w.grid, tile, inverse=True)
        r[tname] = round(float((o.float() - dense).norm()) / nd, 6)
        # the same total per head, shared out by need (per-query-block budgets)
        kt_ = kk * T
        offs, idx_b, _ = paro.route_budget(qd, stats[0], stats[3], kt_, 1, w.lam)
        o = paro.attention_csr(qd, kd, vd, stats[0], stats[1], stats[2], offs, idx_b, kt_)
        r["pisa_budget"] = round(float((o.float() - dense).norm()) / nd, 6)
        rows.append(r)
    full = paro.attention(qd, kd, vd, stats[0], stats[1], stats[2], paro.route(qd, stats[0], stats[3], T, w.lam), T)
    floor = round(float((full.float() - dense).norm()) / nd, 6)
    torch.cuda.synchronize()
    return {"workload": name, "error": "relative Frobenius norm of O - O_dense over all heads",
            "dense_reference": "fp32 path, every block exact", "bf16_dense_floor": floor,
            "captured_mass": "mean share of the dense softmax mass on S_i, every 8th query block of every head",
            "rows": rows}


def peaks_entry(reps: int = 3):
    """Practical peaks of this GPU, measured with the helper kernels of
    libparo_peaks.so (include/paro_peaks.h) and a device copy: dense bf16
    MFMA chains from registers (8 independent 32x32x16 chains per wave,
    2 waves per SIMD), a streaming read of 4 GiB, and a 2 GiB
    device-to-device copy (bytes read + written)."""
    import ctypes

    import torch
    from block_sparse_attention_pisa_amd import build as _b
    lib = ctypes.CDLL(_b.LIB_PEAKS)
    lib.paro_peak_mfma_bf16.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]
    lib.paro_peak_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32, ctypes.c_void_p,
                                   ctypes.c_void_p]
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream
    nwg, iters = 256 * 2, 4000
    sink = torch.zeros(1 << 14, dtype=torch.float32, device="cuda")

    def timed(fn):
        fn()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record(stream)
        for _ in range(reps):
            fn()
        ev[1].record(stream)
        torch.cuda.synchronize()
        return ev[0].elapsed_time(ev[1]) / reps

    def mfma():
        assert lib.paro_peak_mfma_bf16(nwg, iters, sink.data_ptr(), sp) == 0
    ms = timed(mfma)
    mfma_tf = nwg * 4 * iters * 8 * 32768.0 / (ms * 1e-3) / 1e12
    buf = torch.empty(4 << 30, dtype=torch.uint8, device="cuda")
    buf.fill_(1)

    def read():
        assert lib.paro_peak_read(buf.data_ptr(), buf.numel(), 256 * 16, sink.data_ptr(), sp) == 0
    ms_r = timed(read)
    read_gbs = buf.numel() / (ms_r * 1e-3) / 1e9
    src, dst = buf[:2 << 30], buf[2 << 30:]
    ms_c = timed(lambda: dst.copy_(src))
    copy_gbs = 2.0 * src.numel() / (ms_c * 1e-3) / 1e9
    del buf, src, dst
    torch.cuda.empty_cache()
    return {"bf16_mfma_TFLOPs": round(mfma_tf, 1), "hbm_read_GBs": round(read_gbs, 1),
            "hbm_copy_GBs": round(copy_gbs, 1),
            "method": "register-operand MFMA chains (512 workgroups x 4 waves x 8 chains); 4 GiB streaming "
                      "read; 2 GiB device copy counted as read + write"}


def kernel_split_entry(step, names, steps: int = 3):
    """Mean device time per launch of each kernel of the step, from a
    torch.profiler trace of `steps` steps (kernel names matched by
    substring). None when the profiler records no device activity."""
    import torch
    try:
        from torch.profiler import ProfilerActivity, profile
        with profile(activities=[ProfilerActivity.CUDA]) as prof:
            for _ in range(steps):
                step()
            torch.cuda.synchronize()
        acc = {}
        for e in prof.events():
            if e.device_type != torch.autograd.DeviceType.CUDA:
                continue
            for key, pat in names.items():
                if pat in e.name:
                    t = e.device_time if hasattr(e, "device_time") else e.cuda_time
                    acc.setdefault(key, []).append(t)
        if not acc:
            return None
        return {k: round(sum(v) / len(v) / 1e3, 4) for k, v in acc.items()}
    except Exception as ex:  # the profiler is a measurement aid only
        return {"error": str(ex)[:200]}


def captured_mass(qd, kd, idx, scale: float, qblocks):
    """Mean share of the dense softmax mass that falls on the exact blocks S_i
    (the coverage measure of the vector-quantized attention review, Table 6),
    over the rows of the sampled query blocks of every head; fp32 logits on
    the device."""
    import torch
    B, H, L, d = qd.shape
    T = idx.shape[2]
    kblock = torch.arange(L, device=qd.device) // 64
    tot, cnt = 0.0, 0
    for b in range(B):
        for h in range(H):
            rows = torch.cat([torch.arange(64 * i, min(64 * i + 64, L), device=qd.device) for i in qblocks])
            lg = (qd[b, h, rows].float() @ kd[b, h].float().t().contiguous()) * scale
            p = torch.softmax(lg, dim=-1)
            member = torch.zeros(T, T, dtype=torch.bool, device=qd.device)
            member.scatter_(1, idx[b, h].long(), True)
            mask = member[rows // 64][:, kblock]
            share = (p * mask).sum(-1)
            tot += float(share.sum())
            cnt += share.numel()
    return tot / cnt


def budget_ablation_entry(H: int = 8, L: int = 64 * 512, d: int = 128, permille=(50, 100, 125, 250)):
    """Per-query-block budgets where they matter: error against dense
    attention of the method with a fixed k per query block and with the same
    total shared out by need (paro_route_budget, at least one block per row),
    on the varying-need input (workloads.varying_need_inputs: some query
    blocks attend sharply, others broadly). Dense = the fp32 path with every
    block exact; error = relative Frobenius norm over all heads and rows."""
    import torch
    from block_sparse_attention_pisa_amd import paro
    from workloads import varying_need_inputs
    q, k, v = varying_need_inputs(1, H, L, d)
    T = -(-L // 64)
    q32, k32, v32 = (x.float().cuda() for x in (q, k, v))
    st32 = paro.precompute(k32, v32)
    dense = paro.attention(q32, k32, v32, st32[0], st32[1], st32[2], paro.route(q32, st32[0], st32[3], T, 0.1), T)
    del q32, k32, v32, st32
    nd = float(dense.norm())
    qd, kd, vd = (x.cuda() for x in (q, k, v))
    stats = paro.precompute(kd, vd)
    rows = []
    for pm in permille:
        kk = -(-pm * T // 1000)
        idx = paro.route(qd, stats[0], stats[3], kk, 0.1)
        o = paro.attention(qd, kd, vd, stats[0], stats[1], stats[2], idx, kk)
        e_fixed = float((o.float() - dense).norm()) / nd
        offs, idx_b, _ = paro.route_budget(qd, stats[0], stats[3], kk * T, 1, 0.1)
        o = paro.attention_csr(qd, kd, vd, stats[0], stats[1], stats[2], offs, idx_b, kk * T)
        e_budget = float((o.float() - dense).norm()) / nd
        # keep-or-drop (tail dropped) with the same two allocations
        o = paro.attention(qd, kd, vd, stats[0], stats[1], stats[2], idx, kk, drop_tail=True)
        d_fixed = float((o.float() - dense).norm()) / nd
        o = paro.attention_csr(qd, kd, vd, stats[0], stats[1], stats[2], offs, idx_b, kk * T, drop_tail=True)
        d_budget = float((o.float() - dense).norm()) / nd
        ki = torch.diff(offs.to(torch.int64), dim=-1)
        rows.append({"keep_permille": pm, "k": kk, "fixed_k": round(e_fixed, 6), "budget": round(e_budget, 6),
                     "drop_fixed_k": round(d_fixed, 6), "drop_budget": round(d_budget, 6),
                     "k_i_min": int(ki.min()), "k_i_max": int(ki.max())})
    torch.cuda.synchronize()
    return {"workload": f"varying need, B=1, H={H}, L={L}, d={d}, bf16", "total_per_head": "k T (same as fixed k)",
            "error": "relative Frobenius norm of O - O_dense over all heads", "rows": rows}


def cpu_baseline(w, q, k, v, nq: int, nheads: int):
    """Time the fp64 oracle on host cores on a bounded sample of the workload.

    Per sampled head: block statistics and routing in full, attention on nq
    evenly spaced query blocks (plus the last); the head time is extrapolated
    to all T query blocks, and the rate is the dense-equivalent FLOPs of a
    head over that time.
    """
    import numpy as np
    from oracle import pisa
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [os.cpu_count()])
    except Exception:
        cores = os.cpu_count()
    T = w.T
    qbs = sorted(set(np.linspace(0, T - 1, nq).round().astype(int).tolist()) | {T - 1})
    total_s = 0.0
    for h in range(nheads):
        qh, kh, vh = (x[0, h].double().numpy() for x in (q, k, v))
        t0 = time.perf_counter()
        st = pisa.block_stats(kh, vh, w.block)
        idx, _ = pisa.route(qh, st["kbar"], st["M"], w.k, w.lam, w.scale, w.block)
        t1 = time.perf_counter()
        pisa.attention(qh, kh, vh, st, idx, w.scale, w.block, qblocks=qbs)
        t2 = time.perf_counter()
        total_s += (t1 - t0) + (t2 - t1) * T / len(qbs)
    per_head_s = total_s / nheads
    flops_head = 4.0 * w.L * w.L * w.d
    return {
        "value": flops_head / per_head_s / 1e12,
        "unit": "TFLOP/s",
        "cores": int(cores),
        "kind": "oracle",
        "sample": (f"{nheads} head(s) of {w.name}: precompute + routing in full, attention on "
                   f"{len(qbs)} of {T} query blocks, extrapolated to the whole head "
                   f"({per_head_s:.1f} s per head, {per_head_s * w.B * w.H:.0f} s for the whole step)"),
    }


def main():
    a = parse()
    if a.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {a.gpus}); the kernels shard by "
              "(batch, head) with no communication, so multi-GPU runs are not part of this build.",
              file=sys.stderr)
        sys.exit(2)
    import torch
    if a.copy_calibration_mib:
        n = a.copy_calibration_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n}), flush=True)
        return
    from block_sparse_attention_pisa_amd import paro
    from workloads import WORKLOADS, make_inputs

    w = WORKLOADS[a.workload]
    t_gen = time.perf_counter()
    q, k, v = make_inputs(w)
    t_gen = time.perf_counter() - t_gen
    dev = torch.device("cuda:0")
    qd, kd, vd = (x.to(dev) for x in (q, k, v))
    stats = paro.alloc_stats(kd)
    idx = torch.empty(w.B, w.H, w.T, w.k, dtype=torch.int32, device=dev)
    out = torch.empty_like(qd)
    attn_ws = torch.empty(max(16, paro.attention_workspace_bytes(paro.problem(qd))), dtype=torch.uint8,
                          device=dev)
    stream = torch.cuda.current_stream()

    def step(ev=None):
        if ev:
            ev[0].record(stream)
        paro.precompute(kd, vd, out=stats)
        if ev:
            ev[1].record(stream)
        paro.route(qd, stats[0], stats[3], w.k, w.lam, out=idx)
        if ev:
            ev[2].record(stream)
        paro.attention(qd, kd, vd, stats[0], stats[1], stats[2], idx, w.k, out=out, workspace=attn_ws)
        if ev:
            ev[3].record(stream)

    for _ in range(a.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(a.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(a.steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    pre = [e[0].elapsed_time(e[1]) for e in evs]
    rou = [e[1].elapsed_time(e[2]) for e in evs]
    att = [e[2].elapsed_time(e[3]) for e in evs]
    per_step = [e[0].elapsed_time(e[3]) for e in evs]

    def median(x):
        x = sorted(x)
        n = len(x)
        return x[n // 2] if n % 2 else 0.5 * (x[n // 2 - 1] + x[n // 2])
    ms_step = wall * 1e3 / a.steps
    dense_flops = 4.0 * w.B * w.H * w.L * w.L * w.d
    value = dense_flops / (ms_step * 1e-3) / 1e12

    idx_cpu = idx.cpu().numpy()
    attn_flops, exact_flops = attention_flops(w, idx_cpu, with_exact=True)
    split = None if a.no_split else kernel_split_entry(step, {
        "block_stats": "k_block_stats", "hbar_reduce": "k_hbar_reduce", "spectral": "k_block_spectral",
        "route": "k_route", "centroids_bf16": "k_centroids_bf16", "attention": "k_attn_bf16"})

    # the exact phase on this workload: the same kernel with U_i dropped
    # (keep-or-drop mode), exact FLOPs over its time
    ex_ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    paro.attention(qd, kd, vd, stats[0], stats[1], stats[2], idx, w.k, out=out, drop_tail=True,
                   workspace=attn_ws)
    ex_ev[0].record(stream)
    for _ in range(3):
        paro.attention(qd, kd, vd, stats[0], stats[1], stats[2], idx, w.k, out=out, drop_tail=True,
                   workspace=attn_ws)
    ex_ev[1].record(stream)
    torch.cuda.synchronize()
    ex_ms = ex_ev[0].elapsed_time(ex_ev[1]) / 3
    ex_tf = exact_flops / (ex_ms * 1e-3) / 1e12
    reorder = reorder_entry(w, qd, out)
    budget = budget_entry(w, qd, kd, vd, stats, out)
    fp8 = fp8_entry(w, qd, kd, vd, stats, idx, out, attn_flops, exact_flops) if w.dtype == "bf16" else None

    # cold steps: L2 and MALL flushed by a 512 MB write before each step
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    cold = []
    for i in range(3):
        flush.fill_(i & 255)
        cev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        cev[0].record(stream)
        step()
        cev[1].record(stream)
        torch.cuda.synchronize()
        cold.append(cev[0].elapsed_time(cev[1]))
    del flush
    attn_ms = sum(att) / len(att)
    achieved = attn_flops / (attn_ms * 1e-3) / 1e12
    traffic = traffic_entry()
    kv_bytes = 2.0 * w.B * w.H * w.L * w.d * (2 if w.dtype == "bf16" else 4)
    pre_ms = sum(pre) / len(pre)
    # routing reads Q once plus kbar (fp32) and M (fp64), and writes idx (int32)
    route_bytes = kv_bytes / 2 + w.B * w.H * w.T * (4.0 * w.d + 8.0 + 4.0 * w.k)
    route_ms = sum(rou) / len(rou)

    res = {
        "metric": "dense-equiv TFLOP/s + ms/call, 32k-119k-token DiT attention, 12.5% density",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded Fourier-feature Q/K, N(0,1) V; no trained weights)",
        "config": {**w.describe(), "parallelism": "none (1 GPU)"},
        "phases_ms": {"precompute": round(pre_ms, 4), "route": round(route_ms, 4),
                      "attention": round(attn_ms, 4)},
        "median_ms": {"step": round(median(per_step), 4), "precompute": round(median(pre), 4),
                      "route": round(median(rou), 4), "attention": round(median(att), 4)},
        "precompute_hbm": {"algorithmic_GBs": round(kv_bytes / (pre_ms * 1e-3) / 1e9, 1),
                           "frac_of_peak": round(kv_bytes / (pre_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)},
        "route_hbm": {"algorithmic_GBs": round(route_bytes / (route_ms * 1e-3) / 1e9, 1),
                      "frac_of_peak": round(route_bytes / (route_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)},
        # the centroid dots q_bar . k_bar (2 B H T^2 d FLOPs on fp32 MFMA)
        # over the whole routing time
        "route_fp32_mfma": {"dots_flops": 2.0 * w.B * w.H * w.T * w.T * w.d,
                            "TFLOPs": round(2.0 * w.B * w.H * w.T * w.T * w.d / (route_ms * 1e-3) / 1e12, 2),
                            "frac_of_peak": round(2.0 * w.B * w.H * w.T * w.T * w.d / (route_ms * 1e-3) / 1e12 /
                                                  PEAK_FP32_MFMA_TFLOPS, 4)},
        "roofline": {
            "kernel": "k_attn_bf16 (paro_attention)",
            "bound": "mfma",
            "achieved": round(achieved, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
            "traffic": traffic,
            "algorithmic_flops_per_launch": attn_flops,
        },
        "exact_phase_tail_dropped": {"workload": w.name + " (tail dropped)", "ms": round(ex_ms, 3),
                             "algorithmic_flops": exact_flops, "achieved": round(ex_tf, 2),
                             "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                             "frac": round(ex_tf / PEAK_BF16_TFLOPS, 4)},
        "fp8": fp8,
        "budget": budget,
        "reorder": reorder,
        "cold_ms_per_step": round(sorted(cold)[1], 4),
        "input_generation_s": round(t_gen, 1),
    }
    if split and "error" not in split:
        pk = {"kernels_ms_per_launch": split}
        if "block_stats" in split:
            gbs = kv_bytes / (split["block_stats"] * 1e-3) / 1e9
            pk["block_stats"] = {"algorithmic_GBs": round(gbs, 1), "frac_of_hbm_peak": round(gbs / PEAK_HBM_GBS, 4)}
        if "spectral" in split:
            # nominal work: 8 Lanczos steps of A^T A per block (A x and A^T y, 2 d^2 FMAs each)
            fl = 8 * 4.0 * w.d * w.d * w.B * w.H * w.T
            tf = fl / (split["spectral"] * 1e-3) / 1e12
            pk["spectral"] = {"nominal_flops": fl, "TFLOPs": round(tf, 2),
                              "frac_of_fp32_valu_peak": round(tf / PEAK_FP32_VALU_TFLOPS, 4),
                              "note": "fp32 VALU peak without packed-fp32 instructions (78.6 TFLOP/s)"}
        res["precompute_kernels"] = pk
    elif split:
        res["precompute_kernels"] = split
    if not a.no_peaks:
        peaks = peaks_entry()
        res["measured_peaks"] = peaks
        res["roofline"]["frac_of_measured_peak"] = round(achieved / peaks["bf16_mfma_TFLOPs"], 4)
        res["precompute_hbm"]["frac_of_measured_read"] = round(kv_bytes / (pre_ms * 1e-3) / 1e9 /
                                                              peaks["hbm_read_GBs"], 4)
        res["route_hbm"]["frac_of_measured_read"] = round(route_bytes / (route_ms * 1e-3) / 1e9 /
                                                         peaks["hbm_read_GBs"], 4)
    if not a.no_exact_phase:
        del qd, kd, vd, stats, idx, out
        torch.cuda.empty_cache()
        res["exact_phase"] = exact_phase_entry()
    if not a.no_ablation:
        res["ablation"] = ablation_entry()
        res["budget_ablation"] = budget_ablation_entry()
    if not a.no_configs:
        res["other_configs"] = configs_entry()
    if not a.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w, q, k, v, a.cpu_qblocks, a.cpu_heads)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
