#!/usr/bin/env python3
"""Benchmark of the fused attention backward on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

A step is one whole backward call (preprocess + dK/dV kernel + dQ kernel) on inputs already
resident in HBM.  The default workload is the 2x2048x32x128 fp16 causal MHA backward.
Prints one JSON line: causal-adjusted TFLOP/s (2.5 x forward flops over the exact unmasked
pairs), its fraction of the 2.5 PFLOP/s dense fp16/bf16 MFMA peak, per-kernel times from HIP
events recorded on the launch stream, the dominant kernel's roofline, a cold-cache per-call
median, and the CPU oracle timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import statistics
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from attention_backward_amd import synth  # noqa: E402

PEAK_MFMA_TFLOPS = 2500.0  # MI355X dense fp16/bf16
PEAK_HBM_GBS = 8000.0
LOG2E = 1.4426950408889634
METRIC = "attn-bwd TFLOP/s (causal-adjusted) + % of MI355X fp16/bf16 MFMA peak"


def carries_events(args, s: int) -> bool:
    """Whether timed step s records the per-kernel events.  Each event costs the stream a few
    microseconds (a timestamp packet, or a dispatch with timestamps), so only every N-th timed step
    carries them: the kernel durations are still taken inside the timed region, on its stream,
    while the step time carries 1/N of that cost."""
    n = max(1, args.events_every)
    return s % n == n - 1 or (args.steps < n and s == args.steps - 1)


def timed_steps(args) -> list:
    return [s for s in range(args.steps) if carries_events(args, s)]


# HBM traffic of the dominant kernel per launch, from two rocprofv3 counter runs (FETCH_SIZE, then
# WRITE_SIZE, KiB per dispatch), each scaled by what the counter reads for an fp16->f32 copy of
# known size (FETCH_SIZE x 2.000, WRITE_SIZE x 1.000).  Keyed by the hash of the kernel's source
# files at the time: once the sources change, the figure no longer applies and is reported as null.
PROFILED_TRAFFIC = {
    ("dense_dkdv", "mha_causal_b2_s2048_h32_d128_fp16"): dict(
        fetch_kib=116276.0, write_kib=65536.0, fetch_scale=2.000, write_scale=1.000,
        files=("dense_dkdv.hip", "common.h"), sha="0c0f4fd76aca1bff"),
    ("dense_dkdv", "gqa_causal_b1_t16384_hq32_hkv4_d128_bf16"): dict(
        fetch_kib=2460181.0, write_kib=32768.0, fetch_scale=2.000, write_scale=1.000,
        files=("dense_dkdv.hip", "common.h"), sha="0c0f4fd76aca1bff"),
    ("dense_fwd", "mha_causal_b2_s2048_h32_d128_fp16"): dict(
        fetch_kib=76850.5, write_kib=33280.0, fetch_scale=2.000, write_scale=1.000,
        files=("dense_fwd.hip", "common.h"), sha="740a012af4d2d2b7"),
    ("sparse_dkdv", "sparse_mla_b1_sq4096_skv8192_h64_dqk576_dv512_top2048_bf16"): dict(
        fetch_kib=7178644.6, write_kib=426496.0, fetch_scale=2.000, write_scale=1.000,
        files=("sparse_dkdv.hip", "common.h"), sha="3dcaa90113c98a4e"),
}


def profiled_traffic(kernel, workload):
    """Calibrated HBM bytes per launch if counters were taken on the current kernel source, else None."""
    import hashlib

    rec = PROFILED_TRAFFIC.get((kernel, workload))
    if rec is None:
        return None
    h = hashlib.sha256()
    for f in rec["files"]:
        with open(os.path.join(ROOT, "attention_backward_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    if h.hexdigest()[:16] != rec["sha"]:
        return None
    return round((rec["fetch_kib"] * rec["fetch_scale"] + rec["write_kib"] * rec["write_scale"]) * 1024)


def pairs(w) -> int:
    off = w.Skv - w.Sq
    if w.topk:
        return w.B * w.Hq * w.Sq * w.topk
    i = np.arange(w.Sq, dtype=np.int64)
    hi = np.minimum(w.Skv - 1, i + off) if w.causal else np.full_like(i, w.Skv - 1)
    lo = np.maximum(0, i + off - w.window + 1) if w.window > 0 else np.zeros_like(i)
    return int(np.maximum(0, hi - lo + 1).sum()) * w.B * w.Hq


def _softmax_out(s, ok, vv):
    """Masked base-2 softmax of score rows s (-> O rows and lse), fp32 on the GPU."""
    s = torch.where(ok, s, torch.full_like(s, -math.inf))
    m = s.amax(-1, keepdim=True)
    empty = torch.isinf(m) & (m < 0)
    m = torch.where(empty, torch.zeros_like(m), m)
    p = torch.exp2(s - m)
    tot = p.sum(-1, keepdim=True)
    safe = torch.where(empty, torch.ones_like(tot), tot)
    out = (p @ vv) if vv.dim() == 2 else torch.bmm(p, vv)
    o = torch.where(empty, torch.zeros_like(out), out / safe)
    lse = torch.where(empty, torch.full_like(m, -math.inf), m + torch.log2(safe)).squeeze(-1)
    return o, lse


def gpu_forward_inputs(q, k, v, w, idx=None):
    """Input preparation (not timed): O in the storage dtype and base-2 lse in f32 of the masked
    softmax forward over the drawn inputs, evaluated with torch fp32 matmuls on the GPU."""
    B, Sq, Hq, _ = q.shape
    Skv, Hkv, Dv = k.shape[1], k.shape[2], v.shape[3]
    G = Hq // Hkv
    off = Skv - Sq
    c = w.scale * LOG2E
    o = torch.empty((B, Sq, Hq, Dv), dtype=q.dtype, device=q.device)
    lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=q.device)
    if idx is not None:  # top-k: each query row against its own gathered keys, all G heads at once
        rows = 64
        for b in range(B):
            for g in range(Hkv):
                kk = k[b, :, g].float()
                vv = v[b, :, g].float()
                for i0 in range(0, Sq, rows):
                    i1 = min(Sq, i0 + rows)
                    ix = idx[b, i0:i1, g].long()
                    ok = (ix >= 0) & (ix < Skv)
                    if w.causal:
                        ok &= ix <= torch.arange(i0, i1, device=q.device).unsqueeze(1) + off
                    ixc = torch.where(ok, ix, torch.zeros_like(ix))
                    kt = kk[ixc].transpose(1, 2).contiguous()              # [n, Dqk, topk]
                    vs = vv[ixc].contiguous()                              # [n, topk, Dv]
                    qq = q[b, i0:i1, g * G:(g + 1) * G].float().contiguous()  # [n, G, Dqk]
                    s_ = torch.bmm(qq, kt) * c                             # [n, G, topk]
                    oo, ll = _softmax_out(s_, ok.unsqueeze(1).expand_as(s_), vs)
                    o[b, i0:i1, g * G:(g + 1) * G] = oo.to(q.dtype)
                    lse[b, g * G:(g + 1) * G, i0:i1] = ll.t()
        return o, lse
    rows = 1024
    for b in range(B):
        for h in range(Hq):
            kk = k[b, :, h // G].float()
            kt = kk.t().contiguous()
            vv = v[b, :, h // G].float().contiguous()
            qq = q[b, :, h].float()
            for i0 in range(0, Sq, rows):
                i1 = min(Sq, i0 + rows)
                s_ = (qq[i0:i1] @ kt) * c
                ii = torch.arange(i0, i1, device=q.device).unsqueeze(1)
                jj = torch.arange(Skv, device=q.device).unsqueeze(0)
                ok = torch.ones_like(s_, dtype=torch.bool)
                if w.causal:
                    ok &= jj <= ii + off
                if w.window > 0:
                    ok &= jj > ii + off - w.window
                oo, ll = _softmax_out(s_, ok, vv)
                o[b, i0:i1, h] = oo.to(q.dtype)
                lse[b, h, i0:i1] = ll
    return o, lse


def cpu_baseline(w, inp_cpu, target_s):
    """The f64 CPU oracle, as it stands, on a bounded sample of the workload: the full backward of
    the first nb batches and their first nh heads (nh grown first, then nb, so that the run takes
    about target_s seconds; the whole workload when it fits)."""
    import oracle  # the oracle is test infrastructure; this leg only times it

    threads = int(os.environ.get("OMP_NUM_THREADS", "0")) or len(os.sched_getaffinity(0))

    def run(nb, nh):
        G = w.G
        nkv = max(1, nh // G)
        nh = nkv * G
        sl = lambda t, n: t[:nb, :, :n].contiguous()  # noqa: E731
        args = (sl(inp_cpu["q"], nh), sl(inp_cpu["k"], nkv), sl(inp_cpu["v"], nkv), sl(inp_cpu["o"], nh),
                sl(inp_cpu["dout"], nh), inp_cpu["lse"][:nb, :nh].contiguous())
        t0 = time.perf_counter()
        oracle.bwd(*args, w.scale, w.causal, w.window)
        return time.perf_counter() - t0, nh

    if w.topk:
        return cpu_baseline_topk(w, inp_cpu, target_s, threads)
    dt1, nh1 = run(1, w.G)
    nh = min(w.Hq, max(nh1, int(nh1 * target_s / max(dt1, 1e-3))))
    dt, nh = run(1, nh) if nh > nh1 else (dt1, nh1)
    nb = 1
    if nh == w.Hq and w.B > 1 and dt < target_s / 2:
        nb = min(w.B, max(1, int(target_s / max(dt, 1e-3))))
        if nb > 1:
            dt, nh = run(nb, nh)
    sample = w.with_(B=nb, Hq=nh, Hkv=max(1, nh // w.G))
    flops = 2.5 * pairs(sample) * (2 * w.Dqk + 2 * w.Dv)
    what = "the whole workload" if (nb, nh) == (w.B, w.Hq) else \
        f"batches 0..{nb - 1}, query heads 0..{nh - 1} of {w.Hq} ({nb * nh}/{w.B * w.Hq} of the workload's heads)"
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"full f64 backward of {what}, {dt:.1f} s", "seconds": dt}


def cpu_baseline_topk(w, inp_cpu, target_s, threads):
    """Top-k workload: the oracle's full backward over the last n query rows of batch 0 with all
    heads and every key (the last rows keep their causal diagonal, i + Skv - Sq, unchanged)."""
    import oracle

    def run(n):
        i0 = w.Sq - n
        args = (inp_cpu["q"][:1, i0:].contiguous(), inp_cpu["k"][:1].contiguous(), inp_cpu["v"][:1].contiguous(),
                inp_cpu["o"][:1, i0:].contiguous(), inp_cpu["dout"][:1, i0:].contiguous(),
                inp_cpu["lse"][:1, :, i0:].contiguous())
        t0 = time.perf_counter()
        oracle.bwd(*args, w.scale, w.causal, w.window, inp_cpu["idx"][:1, i0:].contiguous())
        return time.perf_counter() - t0

    n1 = 4
    dt1 = run(n1)
    n = min(w.Sq, max(n1, int(n1 * target_s / max(dt1, 1e-3))))
    dt = run(n) if n > n1 else dt1
    flops = 2.5 * n * w.Hq * w.topk * (2 * w.Dqk + 2 * w.Dv)
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"full f64 backward of batch 0, the last {n} of {w.Sq} query rows with all {w.Hq} heads and "
                      f"their top-{w.topk} lists ({n}/{w.B * w.Sq} of the workload's rows), {dt:.1f} s",
            "seconds": dt}


def gpu_state():
    """Temperature and clock levels of the benchmarked GPU, read from its sysfs files (plain file
    reads, no child process; None where they are unavailable): a throttled clock compresses
    differences."""
    import glob

    try:
        pr = torch.cuda.get_device_properties(0)
        bus = "%04x:%02x:%02x" % (pr.pci_domain_id, pr.pci_bus_id, pr.pci_device_id)
        card = next(c for c in sorted(glob.glob("/sys/class/drm/card*/device")) if bus in os.path.realpath(c))
        out = {}
        for t in sorted(glob.glob(card + "/hwmon/hwmon*/temp*_input")):
            lab = t[: -len("_input")] + "_label"
            name = open(lab).read().strip() if os.path.exists(lab) else os.path.basename(t)
            out[f"temp_{name}_C"] = int(open(t).read()) / 1000
        for f in ("pp_dpm_sclk", "pp_dpm_mclk"):
            if os.path.exists(os.path.join(card, f)):
                cur = [ln for ln in open(os.path.join(card, f)).read().splitlines() if ln.rstrip().endswith("*")]
                out[f] = cur[0].split(":", 1)[1].strip(" *") if cur else None
        return out or None
    except Exception:  # noqa: BLE001 -- a missing reading is reported as null
        return None


def gemm_clock(n: int, reps: int = 20):
    """A plain library GEMM (torch.matmul, fp16, n x n x n, contiguous operands) on three operand
    sets -- zeros, a constant, N(0,1) -- each timed with events: the matrix cores' throughput
    and, under the profiler's GRBM_GUI_ACTIVE counter, their clock as a function of the data."""
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev).manual_seed(0)
    cases = (("zeros", lambda: torch.zeros(n, n, dtype=torch.float16, device=dev)),
             ("constant 1/64", lambda: torch.full((n, n), 1.0 / 64, dtype=torch.float16, device=dev)),
             ("normal(0,1)", lambda: torch.randn(n, n, generator=g, dtype=torch.float16, device=dev)))
    for name, make in cases:
        a, b = make(), make()
        c = torch.empty(n, n, dtype=torch.float16, device=dev)
        for _ in range(3):
            torch.matmul(a, b, out=c)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            torch.matmul(a, b, out=c)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        print(json.dumps({"gemm": f"{n}x{n}x{n} fp16", "operands": name, "ms": round(ms, 4),
                          "tflops": round(2.0 * n ** 3 / (ms * 1e-3) / 1e12, 1)}), flush=True)
        del a, b, c


def calib_copy(args, dev):
    """After timing: one fp16 -> f32 device copy reading --calib-copy-mib MiB, a known-size kernel
    against which profiler byte counters are scaled (a conversion, so it runs an elementwise
    kernel; a same-dtype copy would be a DMA transfer)."""
    if args.calib_copy_mib:
        src = torch.ones(args.calib_copy_mib << 19, dtype=torch.float16, device=dev)
        dst = torch.empty(src.shape, dtype=torch.float32, device=dev)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst


def bench_forward(args, w, ab, with_bwd=False):
    """The forward alone (or forward + backward per step): K back-to-back calls on resident q, k, v
    (and dO); one JSON line.  The roofline is the forward kernel's, from events around it."""
    dev = torch.device("cuda:0")
    inp = synth.make_inputs(w)
    q, k, v, do = (inp[n].to(dev) for n in ("q", "k", "v", "dout"))
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.Hq, w.Sq), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    a = None
    if with_bwd:
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        a = ab.make_args(q, k, v, o, do, lse, dq, dk, dv, scale=w.scale, causal=w.causal, window=w.window)
        need = ab.attn_bwd_workspace_size(a)
        ws = torch.empty(need, dtype=torch.uint8, device=dev)
        a.workspace, a.workspace_bytes = ws.data_ptr(), need

    def step():
        ab.attn_fwd(q, k, v, o, lse, w.scale, causal=w.causal, window=w.window, stream=stream)
        if with_bwd:
            ab.attn_bwd_ex(a)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in timed_steps(args)]
    t0 = time.perf_counter()
    it = iter(ev)
    for s in range(args.steps):
        row = next(it) if carries_events(args, s) else None
        if row:
            row[0].record(stream)
        ab.attn_fwd(q, k, v, o, lse, w.scale, causal=w.causal, window=w.window, stream=stream)
        if row:
            row[1].record(stream)
        if with_bwd:
            ab.attn_bwd_ex(a)
        if row:
            row[2].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = [row[0].elapsed_time(row[1]) * 1e3 for row in ev]
    per_b = [row[1].elapsed_time(row[2]) * 1e3 for row in ev]
    calib_copy(args, dev)
    ms_per_step = wall * 1e3 / args.steps
    npairs = pairs(w)
    fwd_flops = npairs * (2 * w.Dqk + 2 * w.Dv)  # S = Q K^T and O = P V over the unmasked pairs
    flops = fwd_flops * (3.5 if with_bwd else 1.0)  # the backward counted as 2.5 forwards
    value = flops / (ms_per_step * 1e-3) / 1e12
    ktf = fwd_flops / (statistics.fmean(per) * 1e-6) / 1e12
    what = "attn-fwd+bwd" if with_bwd else "attn-fwd"
    result = {
        "metric": what + " TFLOP/s (causal-adjusted) + % of MI355X fp16/bf16 MFMA peak",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "pct_of_mfma_peak": round(100 * value / PEAK_MFMA_TFLOPS, 2),
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic: N(0,1) q,k,v" + (",dO" if with_bwd else "") + " from a seeded PCG64 generator",
        "config": {"workload": w.name + (" (forward + backward)" if with_bwd else " (forward)"), "B": w.B, "Sq": w.Sq, "Skv": w.Skv, "Hq": w.Hq, "Hkv": w.Hkv,
                   "Dqk": w.Dqk, "Dv": w.Dv, "causal": w.causal, "window": w.window, "metric_flops": flops,
                   "pairs": npairs},
        "roofline": {"kernel": "dense_fwd", "bound": "mfma", "achieved": round(ktf, 2), "peak": PEAK_MFMA_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(ktf / PEAK_MFMA_TFLOPS, 4),
                     "traffic": profiled_traffic("dense_fwd", w.name), "traffic_unit": "bytes per launch",
                     "algorithmic_flops_per_launch": fwd_flops},
        "kernels_us_median": {"fwd": round(statistics.median(per), 2)} |
                             ({"bwd_call": round(statistics.median(per_b), 2)} if with_bwd else {}),
    }
    print(json.dumps(result), flush=True)


def varlen_pairs(vw, lens) -> int:
    """Unmasked (query, key, head) pairs of packed sequences: each sequence's dense count."""
    return sum(pairs(synth.Workload("", 1, int(n), int(n), vw.Hq, vw.Hkv, vw.D, vw.D, vw.dtype, vw.causal, vw.window,
                                    0, 0)) for n in lens if n > 0)


def bench_varlen(args, vw, ab):
    """The backward (or with --forward the forward) over packed sequences; one JSON line."""
    dev = torch.device("cuda:0")
    inp = synth.make_varlen_inputs(vw)
    q, k, v, do, cu = (inp[n].to(dev) for n in ("q", "k", "v", "dout", "cu"))
    cul = inp["cu"].tolist()
    lens = np.diff(cul)
    mx = inp["max_seqlen"]
    o = torch.empty_like(q)
    lse = torch.full((1, vw.Hq, vw.T), -math.inf, dtype=torch.float32, device=dev)
    for a_, b_ in zip(cul[:-1], cul[1:]):  # input preparation, not timed: fp32 torch forward per sequence
        if b_ > a_:
            oo, ll = gpu_forward_inputs(q[:, a_:b_].contiguous(), k[:, a_:b_].contiguous(), v[:, a_:b_].contiguous(), vw)
            o[:, a_:b_], lse[:, :, a_:b_] = oo, ll
    stream = torch.cuda.current_stream()
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    a = ab.make_args(q, k, v, o, do, lse, dq, dk, dv, scale=vw.scale, causal=vw.causal, window=vw.window,
                     cu_seqlens=cu, max_seqlen=mx)
    need = ab.attn_bwd_workspace_size(a)
    ws = torch.empty(need, dtype=torch.uint8, device=dev)
    a.workspace, a.workspace_bytes = ws.data_ptr(), need
    o2, lse2 = torch.empty_like(q), torch.empty_like(lse)

    def call():
        if args.forward:
            ab.attn_fwd_varlen(q, k, v, o2, lse2, cu, mx, vw.scale, causal=vw.causal, window=vw.window, stream=stream)
        else:
            ab.attn_bwd_ex(a)

    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    import ctypes

    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in timed_steps(args)]
    for row in ev:
        for e in row:
            e.record(stream)
    torch.cuda.synchronize()
    ev_arrays = [(ctypes.c_void_p * 4)(*[e.cuda_event for e in row]) for row in ev]
    t0 = time.perf_counter()
    j_ = 0
    for s_ in range(args.steps):
        if not carries_events(args, s_):
            a.events = None
            call()
        elif args.forward:
            ev[j_][0].record(stream)
            call()
            ev[j_][1].record(stream)
            j_ += 1
        else:
            a.events = ctypes.cast(ev_arrays[j_], ctypes.c_void_p)
            call()
            j_ += 1
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    a.events = None
    ms_per_step = wall * 1e3 / args.steps
    npairs = varlen_pairs(vw, lens)
    fwd_flops = npairs * 4 * vw.D
    if args.forward:
        per = {"fwd": [row[0].elapsed_time(row[1]) * 1e3 for row in ev]}
        flops, kname, kflops = fwd_flops, "dense_fwd", fwd_flops
    else:
        per = {"dq": [row[0].elapsed_time(row[1]) * 1e3 for row in ev],
               "dkdv": [row[1].elapsed_time(row[2]) * 1e3 for row in ev],
               "landing": [row[2].elapsed_time(row[3]) * 1e3 for row in ev]}
        flops, kname, kflops = 2.5 * fwd_flops, "dense_dkdv", npairs * 8 * vw.D
    kus = statistics.fmean(per["fwd" if args.forward else "dkdv"])
    ktf = kflops / (kus * 1e-6) / 1e12
    value = flops / (ms_per_step * 1e-3) / 1e12
    what = "attn-fwd" if args.forward else "attn-bwd"
    result = {
        "metric": what + " TFLOP/s (causal-adjusted) + % of MI355X fp16/bf16 MFMA peak",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "pct_of_mfma_peak": round(100 * value / PEAK_MFMA_TFLOPS, 2),
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": vw.dtype,
        "data": "synthetic: seeded unequal lengths, N(0,1) q,k,v,dO from a seeded PCG64 generator; "
                "O and lse from an fp32 forward per sequence",
        "config": {"workload": vw.name + (" (forward)" if args.forward else ""), "T": vw.T, "nseq": vw.nseq,
                   "lens": [int(x) for x in lens], "Hq": vw.Hq, "Hkv": vw.Hkv, "D": vw.D, "causal": vw.causal,
                   "window": vw.window, "metric_flops": flops, "pairs": npairs},
        "roofline": {"kernel": kname, "bound": "mfma", "achieved": round(ktf, 2), "peak": PEAK_MFMA_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(ktf / PEAK_MFMA_TFLOPS, 4), "traffic": None,
                     "algorithmic_flops_per_launch": kflops},
        "kernels_us_median": {n_: round(statistics.median(x), 2) for n_, x in per.items()},
    }
    if not args.forward and vw.window == 0 and (vw.Hq // vw.Hkv) % 2 == 0:
        # The split dK/dV: the landing pass reads two f32 slices each of dK and dV and writes dk, dv
        # over the tokens of the sequences.
        ntok = int(sum(min(int(n), mx) for n in lens))
        land_bytes = ntok * vw.Hkv * vw.D * (2 * 2 * 4 + 2 * 2)
        lus = statistics.fmean(per["landing"])
        result["landing"] = {"us": round(lus, 2), "GB/s": round(land_bytes / (lus * 1e-6) / 1e9, 1),
                             "frac_of_hbm_peak": round(land_bytes / (lus * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)}
    print(json.dumps(result), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--events-every", type=int, default=4,
                    help="timed steps that carry the per-kernel events: every N-th (1 = all); the\n"
                         "events' stream work is then a 1/N share of the measured step time")
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=synth.HEADLINE,
                    choices=sorted(synth.WORKLOADS) + sorted(synth.VARLEN_WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--cold-iters", type=int, default=10)
    ap.add_argument("--kv-shared", action="store_true",
                    help="top-k workloads: the shared-latent form (V is the first Dv columns of K; one dKV output)")
    ap.add_argument("--forward", action="store_true",
                    help="dense workloads: time the forward kernel (O and lse from q, k, v) instead")
    ap.add_argument("--fwd-bwd", action="store_true",
                    help="dense workloads: time forward + backward per step (O and lse from the forward kernel)")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="after timing, run one fp16->f32 device copy reading this many MiB (a known-size "
                         "kernel against which profiler byte counters are scaled)")
    ap.add_argument("--gemm-clock", type=int, default=0,
                    help="instead of a workload: time an n x n x n fp16 library GEMM on zero, constant and "
                         "random operands (the matrix cores' throughput as a function of the data)")
    args = ap.parse_args()
    if args.gemm_clock:
        gemm_clock(args.gemm_clock)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the backward runs on one GPU and this library has no "
              "multi-GPU path (it would shard by (batch, head) or by query rows); run it with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import attention_backward_amd as ab

    if args.workload in synth.VARLEN_WORKLOADS:
        bench_varlen(args, synth.VARLEN_WORKLOADS[args.workload], ab)
        return
    w = synth.WORKLOADS[args.workload]
    shared = bool(args.kv_shared)
    if shared and not w.topk:
        print("--kv-shared applies to the top-k workloads only", file=sys.stderr)
        sys.exit(2)
    if args.forward or args.fwd_bwd:
        if w.topk:
            print("--forward and --fwd-bwd cover the dense workloads only", file=sys.stderr)
            sys.exit(2)
        bench_forward(args, w, ab, with_bwd=args.fwd_bwd)
        return
    dev = torch.device("cuda:0")
    inp = synth.make_inputs(w)
    if shared:  # V is the first Dv columns of K
        inp["v"] = inp["k"][..., : w.Dv].contiguous()
    q, k, v, do = (inp[n].to(dev) for n in ("q", "k", "v", "dout"))
    idx = inp["idx"].to(dev) if w.topk else None
    o, lse = gpu_forward_inputs(q, k, v, w, idx)
    dq, dk = torch.empty_like(q), torch.empty_like(k)
    dv = None if shared else torch.empty_like(v)
    a = ab.make_args(q, k, None if shared else v, o, do, lse, dq, dk, dv, scale=w.scale, causal=w.causal,
                     window=w.window, topk_idx=idx, kv_shared=shared)
    need = ab.attn_bwd_workspace_size(a)
    ws = torch.empty(need, dtype=torch.uint8, device=dev)
    a.workspace, a.workspace_bytes = ws.data_ptr(), need
    stream = torch.cuda.current_stream()

    state_before = gpu_state()
    for _ in range(args.warmup):
        ab.attn_bwd_ex(a)
    torch.cuda.synchronize()

    # Timed region: exactly K back-to-back steps; every --events-every-th one passes 4 events that
    # the library records on its launch stream at its phase boundaries (dispatch timestamps).
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in timed_steps(args)]
    import ctypes

    for row in ev:
        for e in row:
            e.record(stream)  # materialise the underlying hipEvent before taking its handle
    torch.cuda.synchronize()
    ev_arrays = [(ctypes.c_void_p * 4)(*[e.cuda_event for e in row]) for row in ev]
    assert all(h for arr in ev_arrays for h in arr), "HIP event handles must be non-null"
    t0 = time.perf_counter()
    j = 0
    for s in range(args.steps):
        if carries_events(args, s):
            a.events = ctypes.cast(ev_arrays[j], ctypes.c_void_p)
            j += 1
        else:
            a.events = None
        ab.attn_bwd_ex(a)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    state_after = gpu_state()
    a.events = None
    # The library records its events between its phases: dense = dQ kernel (with the preprocess
    # in its prologue) | dK/dV kernel | (nothing); top-k = preprocess, zero-fill, key counts and
    # dQ kernel | dK/dV kernel | landing.
    names = ("dq", "dkdv") if not w.topk else ("pre_and_dq", "sparse_dkdv", "landing")
    per = {n_: [] for n_ in names + ("call",)}
    for row in ev:
        for j, n_ in enumerate(names):
            per[n_].append(row[j].elapsed_time(row[j + 1]) * 1e3)
        per["call"].append(row[0].elapsed_time(row[3]) * 1e3)
    ms_per_step = wall * 1e3 / args.steps

    # Cold-cache per-call timing (the pages flush L2 before every iteration): a 1 GiB write
    # before each call evicts the 256 MB Infinity Cache and the per-XCD L2s.
    flush = torch.empty(1 << 28, dtype=torch.float32, device=dev)
    cold = []
    for _ in range(args.cold_iters):
        flush.fill_(1.0)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        ab.attn_bwd_ex(a)
        e1.record(stream)
        torch.cuda.synchronize()
        cold.append(e0.elapsed_time(e1) * 1e3)
    del flush
    calib_copy(args, dev)

    npairs = pairs(w)
    flops = 2.5 * npairs * (2 * w.Dqk + 2 * w.Dv)
    value = flops / (ms_per_step * 1e-3) / 1e12
    esz = 2
    med = {kname: statistics.median(vals) for kname, vals in per.items()}
    mean = {kname: statistics.fmean(vals) for kname, vals in per.items()}
    if not w.topk:
        main_name = "dense_dkdv"
        main_flops = npairs * (4 * w.Dqk + 4 * w.Dv)   # S, dP, dV, dK products
        dq_flops = npairs * (4 * w.Dqk + 2 * w.Dv)     # S, dP recomputed, dQ
        main_tf = main_flops / (mean["dkdv"] * 1e-6) / 1e12
        kernels = {
            "dq": {"us": round(mean["dq"], 2), "TFLOP/s": round(dq_flops / (mean["dq"] * 1e-6) / 1e12, 1),
                   "note": "includes the preprocess (delta, lse copy) in its prologue"},
            "dkdv": {"us": round(mean["dkdv"], 2), "TFLOP/s": round(main_tf, 1)},
        }
    else:
        # Dominant kernel: the key-owned dK/dV pass.  Algorithmic work = its four products over
        # the listed (query, key, head) triples (it computes them over every visible pair).
        main_name = "sparse_dkdv"
        main_flops = npairs * (4 * w.Dqk + 4 * w.Dv)
        main_tf = main_flops / (mean["sparse_dkdv"] * 1e-6) / 1e12
        acc_bytes = w.B * w.Skv * w.Hkv * (w.Dqk + w.Dv) * 4
        land_bytes = acc_bytes + w.B * w.Skv * w.Hkv * (w.Dqk if shared else w.Dqk + w.Dv) * esz
        kernels = {
            "pre_and_dq": {"us": round(mean["pre_and_dq"], 2),
                           "note": "delta, zero-fill, key counts and the gathered dQ kernel"},
            "sparse_dkdv": {"us": round(mean["sparse_dkdv"], 2), "TFLOP/s": round(main_tf, 1)},
            "landing": {"us": round(mean["landing"], 2),
                        "GB/s": round(land_bytes / (mean["landing"] * 1e-6) / 1e9, 1)},
        }
    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "pct_of_mfma_peak": round(100 * value / PEAK_MFMA_TFLOPS, 2),
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic: N(0,1) q,k,v,dO from a seeded PCG64 generator" +
                ("; top-k lists of distinct causal keys drawn uniformly" if w.topk else "") +
                ("; V = the first Dv columns of K (shared-latent form)" if shared else "") +
                "; O and lse from an fp32 forward",
        "config": {"workload": w.name, "B": w.B, "Sq": w.Sq, "Skv": w.Skv, "Hq": w.Hq, "Hkv": w.Hkv,
                   "Dqk": w.Dqk, "Dv": w.Dv, "causal": w.causal, "window": w.window, "topk": w.topk,
                   "kv_shared": shared, "metric_flops": flops, "pairs": npairs},
        "roofline": {"kernel": main_name, "bound": "mfma", "achieved": round(main_tf, 2),
                     "peak": PEAK_MFMA_TFLOPS, "unit": "TFLOP/s", "frac": round(main_tf / PEAK_MFMA_TFLOPS, 4),
                     "traffic": None if shared else profiled_traffic(main_name, w.name),
                     "traffic_unit": "bytes per launch",
                     "algorithmic_flops_per_launch": main_flops},
        "kernels_us_median": {kname: round(v_, 2) for kname, v_ in med.items()},
        "kernels": kernels,
        "kernel_events": {"every_nth_timed_step": max(1, args.events_every), "samples": len(ev)},
        "cold_call_us": None if not cold else {
            "median": round(statistics.median(cold), 2), "mean": round(statistics.fmean(cold), 2),
            "std": round(statistics.pstdev(cold), 2), "min": round(min(cold), 2),
            "p10": round(float(np.percentile(cold, 10)), 2), "p90": round(float(np.percentile(cold, 90)), 2),
            "max": round(max(cold), 2), "n": len(cold),
            "tflops_at_median": round(flops / (statistics.median(cold) * 1e-6) / 1e12, 1)},
        "gpu_state": {"before": state_before, "after_timed_steps": state_after},
    }
    if not args.no_cpu_baseline:
        inp_cpu = {n: inp[n] for n in ("q", "k", "v", "dout", "idx")}
        inp_cpu["o"], inp_cpu["lse"] = o.cpu(), lse.cpu()
        result["cpu_baseline"] = cpu_baseline(w, inp_cpu, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
