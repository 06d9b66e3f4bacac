#!/usr/bin/env python3
"""Benchmark of the FP8 weight path on one MI355X (gfx950).

One step = one pass of the block-FP8 W8A16 GEMV at M = 1 over the 48-layer
per-rank projection set (12 x [6656x2560] + 36 x [8192x2560] + 48 x
[2560x3072], 96 calls, 1.337 GB of fp8 codes), the decode workload of
"feat(qwen4_exp): load-time per-tensor FP8 dense projections" (Why).  The 96
distinct weights exceed the 256 MB Infinity Cache, so every pass streams the
codes from HBM.  Weights are synthetic N(0, 0.02) bf16, quantized on the GPU
by fp8w_quantize_block before timing; activations are N(0, 1) bf16.

A step is one grouped launch (fp8w_gemv_grouped) computing the 96 GEMVs,
timed with HIP events on the launching stream; the same pass as 96 single
GEMV launches, captured in a HIP graph (as the pages' decode path is) and
launched one by one on the stream, is reported next to it.  Prints ONE
JSON line; the other workloads (M = 8 / 16, the quantizers, lm_head, the
dense layer, MXFP8) are reported under "rows".

    python bench.py [--steps K] [--warmup W] [--rows proj,quant,lm_head,dense,mx,single]
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM = 8.0e12          # MI355X HBM3E, bytes/s
PEAK_BF16 = 2.5e15         # MI355X dense bf16 MFMA, flop/s

# HBM bytes per launch of the grouped M=1 streaming GEMV on the projection
# set, from rocprofv3 FETCH_SIZE / WRITE_SIZE runs scaled by a 2 GiB device
# copy (read factor 1.99993, write factor 1.0): 1339.30 MB read + 1.00 MB
# written.  Valid only for the sources they were taken with (sha256 of the
# kernel, launch-plan and helper sources); any change to those reports
# traffic as null until the counters are retaken.
COUNTED_TRAFFIC = {
    "sources_sha256": "da643c86f7ff702dad9247d891e2c9480ebec2cce44877578dd155c9968fdd93",
    "bytes_per_launch": 1340.30e6,
}
TRAFFIC_SOURCES = ('gemv.hip', 'device.hpp', 'internal.hpp', 'api.cpp')


def counted_traffic():
    import hashlib
    h = hashlib.sha256()
    for f in TRAFFIC_SOURCES:
        with open(os.path.join(ROOT, "fp8_block_scaled_02_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    if h.hexdigest() != COUNTED_TRAFFIC["sources_sha256"]:
        return None
    return COUNTED_TRAFFIC["bytes_per_launch"]


TILE, GROUP = 128, 32
ALL_ROWS = ("proj", "quant", "lm_head", "dense", "mx", "single", "dequant", "gemm", "w8a8", "row", "route")


def parse():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    # MI355X runs the first ~2 ms of a burst of HBM-bound launches after an idle
    # spell at full speed, then 10-20 % slower for ~10 ms while its power
    # management settles (kernel traces of back-to-back launches); 200 warmup
    # steps (~40 ms) put the timed steps in the steady state of a decode loop.
    p.add_argument("--steps", type=int, default=300)
    p.add_argument("--warmup", type=int, default=200)
    p.add_argument("--rows", default=",".join(ALL_ROWS))
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    p.add_argument("--ms", default=None,
                   help="M values of the GEMV rows (default: projection set 1,8,16; the other "
                        "workloads their own)")
    p.add_argument("--route", default="auto", choices=("auto", "valu", "mfma"),
                   help="route of the projection-set rows (auto: the library's choice per M)")
    p.add_argument("--route-shapes", default=None,
                   help="weights of the route row, as NxK,NxK (default: every workload shape)")
    p.add_argument("--route-formats", default="block,mx", help="scale formats of the route row")
    p.add_argument("--calibrate-copy-mib", type=int, default=0,
                   help="also run one device copy of this many MiB (counter calibration)")
    a = p.parse_args()
    if a.route == "valu" and any(int(v) > 8 for v in (a.ms or "1,8,16").split(",") if v):
        p.error("--route valu serves m <= 8 only")
    return a


def row_ms(args, default):
    """M values of a GEMV row: --ms when given, else the workload's own."""
    return tuple(int(v) for v in args.ms.split(",") if v) if args.ms else tuple(default)


# ------------------------------------------------------------ byte counts --

def gemv_bytes_block(m, n, k):
    return n * k + 4 * (-(-n // TILE)) * (-(-k // TILE)) + 2 * m * k + 2 * m * n


def w8a8_bytes_block(m, n, k):
    """fp8 codes + block scales + fp8 activation codes and scale + bf16 y."""
    return n * k + 4 * (-(-n // TILE)) * (-(-k // TILE)) + m * k + 4 + 2 * m * n


def gemv_bytes_mx(m, n, k):
    return n * k + n * (-(-k // GROUP)) + 2 * m * k + 2 * m * n


def quant_bytes_block(n, k):
    return 3 * n * k + 4 * (-(-n // TILE)) * (-(-k // TILE))


def quant_bytes_mx(n, k):
    return 3 * n * k + n * (-(-k // GROUP))


# ----------------------------------------------------------------- timing --

class Timer:
    """Event timing on torch's current stream.  A spin kernel is queued first
    so the host can enqueue a whole sequence before the GPU reaches it: the
    intervals then measure back-to-back GPU execution, not host latency."""

    def __init__(self, torch):
        self.torch = torch
        self.cycles_per_ms = self._calibrate()

    def _calibrate(self):
        t = self.torch
        a, b = t.cuda.Event(enable_timing=True), t.cuda.Event(enable_timing=True)
        t.cuda._sleep(1000)
        a.record()
        t.cuda._sleep(20_000_000)
        b.record()
        t.cuda.synchronize()
        return 20_000_000 / max(a.elapsed_time(b), 1e-3)

    def hold(self, ms):
        self.torch.cuda._sleep(int(self.cycles_per_ms * ms))

    def run(self, fn, reps, warmup, hold_ms=0.0):
        """(per-rep ms, total ms).  The total brackets `reps` back-to-back
        calls of fn with one event pair and nothing between them; a second
        run puts an event pair around each call for the distribution.

        hold_ms > 0 queues a spin kernel first, for sequences whose host-side
        enqueue is slower than their GPU time (un-graphed launches); graph
        replays and single grouped launches are cheap to enqueue."""
        t = self.torch
        ev = lambda: t.cuda.Event(enable_timing=True)
        for _ in range(warmup):
            fn()
        t0, t1 = ev(), ev()
        t.cuda.synchronize()
        if hold_ms > 0:
            self.hold(hold_ms)
        t0.record()
        for _ in range(reps):
            fn()
        t1.record()
        t.cuda.synchronize()
        total = t0.elapsed_time(t1)
        starts = [ev() for _ in range(reps)]
        ends = [ev() for _ in range(reps)]
        if hold_ms > 0:
            self.hold(hold_ms)
        for i in range(reps):
            starts[i].record()
            fn()
            ends[i].record()
        t.cuda.synchronize()
        return [s.elapsed_time(e) for s, e in zip(starts, ends)], total


def graph_of(torch, fn):
    """Capture fn (a sequence of library calls) in a HIP graph."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def pct(v, q):
    v = sorted(v)
    return v[min(len(v) - 1, max(0, int(round(q * (len(v) - 1)))))]


def route_names(fp8w, m, calls, fmt="block"):
    """The kernel families AUTO takes for these single calls ("valu", "mfma")."""
    names = {fp8w.ROUTE_VALU: "valu", fp8w.ROUTE_MFMA: "mfma"}
    got = sorted({names[fp8w.fp8w_gemv_auto_route(m, c.shape[0], c.shape[1], fmt)] for (_, c, _, _) in calls})
    return "+".join(got)


def summarize(per_ms, calls, nbytes):
    med = statistics.median(per_ms)
    return {
        "us_per_call_p50": round(1e3 * med / calls, 3),
        "us_per_call_p10": round(1e3 * pct(per_ms, 0.1) / calls, 3),
        "us_per_call_p90": round(1e3 * pct(per_ms, 0.9) / calls, 3),
        "GBps": round(nbytes / (med * 1e-3) / 1e9, 1),
        "pct_of_peak": round(100 * nbytes / (med * 1e-3) / PEAK_HBM, 1),
    }


# --------------------------------------------------------------- launching --

class Lean:
    """Direct ctypes launches with pre-marshalled arguments (no Python checks
    per call), for timing sequences of calls on the current stream."""

    def __init__(self, fp8w, torch):
        self.lib = fp8w.lib()
        self.torch = torch

    def stream(self):
        return self.torch.cuda.current_stream().cuda_stream

    def gemv_block(self, calls, route=0):
        fn = self.lib.fp8w_gemv_block_route
        lib_args = [(x.data_ptr(), x.shape[0], c.data_ptr(), s.data_ptr(), c.shape[0], c.shape[1],
                     y.data_ptr(), route) for (x, c, s, y) in calls]

        def launch():
            st = self.stream()
            for a in lib_args:
                rc = fn(*a, st)
                if rc:
                    raise RuntimeError(f"fp8w_gemv_block_route failed: {rc}")
        return launch

    def gemv_mx(self, calls, route=0):
        fn = self.lib.fp8w_gemv_mx_route
        lib_args = [(x.data_ptr(), x.shape[0], c.data_ptr(), e.data_ptr(), c.shape[0], c.shape[1],
                     y.data_ptr(), route) for (x, c, e, y) in calls]

        def launch():
            st = self.stream()
            for a in lib_args:
                rc = fn(*a, st)
                if rc:
                    raise RuntimeError(f"fp8w_gemv_mx_route failed: {rc}")
        return launch

    def grouped(self, plan):
        fn = self.lib.fp8w_gemv_grouped
        ref = ctypes.byref(plan.plan)

        def launch():
            rc = fn(ref, self.stream())
            if rc:
                raise RuntimeError(f"fp8w_gemv_grouped failed: {rc}")
        return launch

    def quant_grouped(self, plan):
        fn = self.lib.fp8w_quantize_grouped
        p = ctypes.byref(plan.plan)

        def launch():
            rc = fn(p, self.stream())
            if rc:
                raise RuntimeError(f"fp8w_quantize_grouped failed: {rc}")
        return launch

    def quant(self, jobs, mx=False):
        fn = self.lib.fp8w_quantize_mx if mx else self.lib.fp8w_quantize_block
        lib_args = [(w.data_ptr(), w.shape[0], w.shape[1], c.data_ptr(), s.data_ptr())
                    for (w, c, s) in jobs]

        def launch():
            st = self.stream()
            for a in lib_args:
                rc = fn(*a, st)
                if rc:
                    raise RuntimeError(f"quantize failed: {rc}")
        return launch


# ---------------------------------------------------------------- workloads --

def upload_bf16(torch, bits):
    import numpy as np
    return torch.from_numpy(bits.view(np.int16)).to("cuda").view(torch.bfloat16)


def projection_set(torch, fp8w, W, log):
    """Generate, upload and quantize the 96 projection weights (load time)."""
    from concurrent.futures import ThreadPoolExecutor
    wl = W.WORKLOADS[2]
    t = time.time()
    with ThreadPoolExecutor(2) as ex:
        bits = list(ex.map(lambda w: w.bits(2), wl.weights))
    bf = [upload_bf16(torch, b) for b in bits]
    del bits
    codes, scales = [], []
    for w in bf:
        c, s = fp8w.fp8w_quantize_block(w)
        codes.append(c)
        scales.append(s)
    torch.cuda.synchronize()
    log(f"projection set ready in {time.time() - t:.1f}s")
    return wl, bf, codes, scales


def activations(torch, W, workload, ms, ks):
    return {(m, k): upload_bf16(torch, W.activation(workload, m, k)) for m in ms for k in ks}


def bench_proj(torch, fp8w, lean, timer, W, args, state, log):
    """The projection pass at M = 1, 8, 16: one grouped launch per pass, and
    96 single-GEMV launches per pass (both captured in a HIP graph)."""
    wl, bf, codes, scales = state
    ms = row_ms(args, (1, 8, 16))
    xs = activations(torch, W, 2, ms, (2560, 3072))
    rows, head = {}, None
    route = {"auto": fp8w.ROUTE_AUTO, "valu": fp8w.ROUTE_VALU, "mfma": fp8w.ROUTE_MFMA}[args.route]
    for m in ms:
        ys = [torch.empty((m, c.shape[0]), dtype=torch.bfloat16, device="cuda") for c in codes]
        calls = [(xs[(m, c.shape[1])], c, s, y) for c, s, y in zip(codes, scales, ys)]
        nbytes = sum(gemv_bytes_block(m, c.shape[0], c.shape[1]) for c in codes)
        plan = fp8w.fp8w_grouped_plan_init([x for x, _, _, _ in calls], codes, scales, ys, route=route)
        # one kernel per pass: launched directly (a one-kernel graph replay
        # adds 8-20 us of launch overhead per replay on ROCm)
        per, total = timer.run(lean.grouped(plan), args.steps, args.warmup)
        row = {"grouped": dict(summarize(per, len(calls), nbytes), launches_per_pass=1,
                               ms_per_pass=round(statistics.median(per), 4),
                               kernel="streaming" if plan.plan.tiles_per_block > 0 else "one tile per workgroup")}
        g = graph_of(torch, lean.gemv_block(calls, route))
        per_c, _ = timer.run(g.replay, args.steps, args.warmup)
        row["per_call"] = dict(summarize(per_c, len(calls), nbytes), launches_per_pass=len(calls),
                               ms_per_pass=round(statistics.median(per_c), 4))
        del g
        # the same 96 calls launched one by one on the stream (no graph): a spin
        # kernel queued first lets the host enqueue ahead of the GPU
        stream_steps = max(5, min(args.steps, 50))
        per_s, _ = timer.run(lean.gemv_block(calls, route), stream_steps, min(args.warmup, 20), hold_ms=20.0)
        row["per_call_stream"] = dict(summarize(per_s, len(calls), nbytes), launches_per_pass=len(calls),
                                      ms_per_pass=round(statistics.median(per_s), 4), graph=False)
        per_call_route = route_names(fp8w, m, calls) if route == fp8w.ROUTE_AUTO else args.route
        row.update({"bytes_per_pass": nbytes, "route": "valu" if plan.route == fp8w.ROUTE_VALU else "mfma",
                    "per_call_route": per_call_route})
        if m == 1 and route == fp8w.ROUTE_AUTO:
            head = {"per": per, "total_ms": total, "bytes": nbytes, "calls": len(calls), "row": row}
        rows[f"m{m}"] = row
        log(f"proj m={m}: {row}")
    return rows, head


def quant_passes(torch, fp8w, lean, timer, jobs, fmt, nbytes):
    """A quantizer pass over `jobs` (w, codes, scales): one graph-captured
    call per weight, and one grouped launch for all of them."""
    g = graph_of(torch, lean.quant(jobs, mx=fmt == "mx"))
    per, _ = timer.run(g.replay, 6, 3)
    row = {"per_call": dict(summarize(per, len(jobs), nbytes), ms_per_pass=round(statistics.median(per), 4))}
    del g
    plan = fp8w.fp8w_quant_plan_init([w for w, _, _ in jobs], fmt, codes=[c for _, c, _ in jobs],
                                     scales=[s for _, _, s in jobs])
    per_g, _ = timer.run(lean.quant_grouped(plan), 6, 3)
    row["grouped"] = dict(summarize(per_g, len(jobs), nbytes), ms_per_pass=round(statistics.median(per_g), 4),
                          workgroups=plan.blocks)
    row.update({"weights": len(jobs), "bytes_per_pass": nbytes})
    return row


def bench_quant(torch, fp8w, lean, timer, W, args, state, log):
    wl, bf, codes, scales = state
    jobs = list(zip(bf, codes, scales))
    nbytes = sum(quant_bytes_block(w.shape[0], w.shape[1]) for w in bf)
    row = quant_passes(torch, fp8w, lean, timer, jobs, "block", nbytes)
    row["workload"] = "projection set, 96 weights"
    log(f"quantize_block projection set: {row}")
    return {"quantize_block_projection_set": row}


def bench_lm_head(torch, fp8w, lean, timer, W, args, log):
    wl = W.WORKLOADS[3]
    w = wl.weights[0]
    bf = upload_bf16(torch, w.bits(3))
    n, k = w.n, w.k
    c0, s0 = fp8w.fp8w_quantize_block(bf)
    qper, _ = timer.run(lean.quant([(bf, c0, s0)]), 10, 2, hold_ms=5.0)
    out = {"quantize_block": dict(summarize(qper, 1, quant_bytes_block(n, k)), shape=[n, k])}
    del bf
    copies = [(c0, s0)] + [(c0.clone(), s0.clone()) for _ in range(3)]
    lib = fp8w.lib()
    for m in row_ms(args, wl.ms):
        x = upload_bf16(torch, W.activation(3, m, k))
        calls = [(x, c, s, torch.empty((m, n), dtype=torch.bfloat16, device="cuda")) for c, s in copies]
        g = graph_of(torch, lean.gemv_block(calls))
        per, _ = timer.run(g.replay, args.steps, args.warmup)
        out[f"gemv_m{m}"] = summarize(per, len(calls), len(calls) * gemv_bytes_block(m, n, k))
        del g
        # W8A8 on the same weights: activation quantized once, GEMV per call
        xc, xs = fp8w.fp8w_quantize_act(x)
        w8 = [(xc.data_ptr(), xs.data_ptr(), m, c.data_ptr(), s.data_ptr(), n, k, y.data_ptr())
              for (_, c, s, y) in calls]

        def run_w8():
            st = torch.cuda.current_stream().cuda_stream
            for a in w8:
                rc = lib.fp8w_gemv_block_w8a8(*a, st)
                if rc:
                    raise RuntimeError(f"fp8w_gemv_block_w8a8 failed: {rc}")
        g = graph_of(torch, run_w8)
        per, _ = timer.run(g.replay, args.steps, args.warmup)
        out[f"w8a8_gemv_m{m}"] = summarize(per, len(calls), len(calls) * w8a8_bytes_block(m, n, k))
        del g
    log(f"lm_head: {out}")
    return {"lm_head_151936x2048": out}


def bench_dense(torch, fp8w, lean, timer, W, args, log):
    wl = W.WORKLOADS[4]
    layer = []
    for w in wl.weights:
        bf = upload_bf16(torch, w.bits(4))
        layer.append(fp8w.fp8w_quantize_block(bf))
        del bf
    copies = [layer] + [[(c.clone(), s.clone()) for c, s in layer] for _ in range(5)]
    out = {}
    for m in row_ms(args, wl.ms):
        xs = {k: upload_bf16(torch, W.activation(4, m, k)) for k in (4096, 12288)}
        calls = [(xs[c.shape[1]], c, s, torch.empty((m, c.shape[0]), dtype=torch.bfloat16, device="cuda"))
                 for cp in copies for c, s in cp]
        nbytes = sum(gemv_bytes_block(m, c.shape[0], c.shape[1]) for (_, c, _, _) in calls)
        g = graph_of(torch, lean.gemv_block(calls))
        per, _ = timer.run(g.replay, args.steps, args.warmup)
        row = {"per_call": summarize(per, len(calls), nbytes), "route": route_names(fp8w, m, calls)}
        del g
        plan = fp8w.fp8w_grouped_plan_init([c[0] for c in calls], [c[1] for c in calls],
                                           [c[2] for c in calls], [c[3] for c in calls])
        per_g, _ = timer.run(lean.grouped(plan), args.steps, args.warmup)
        row["grouped"] = summarize(per_g, len(calls), nbytes)
        out[f"m{m}"] = row
        del plan
    log(f"dense layer: {out}")
    return {"dense_layer_h4096_i12288": out}


def bench_mx(torch, fp8w, lean, timer, W, args, log):
    wl = W.WORKLOADS[5]
    out = {}
    for w, copies_n in zip(wl.weights, (48, 128)):
        bf = upload_bf16(torch, w.bits(5))
        c0, e0 = fp8w.fp8w_quantize_mx(bf)
        key = f"{w.n}x{w.k}"
        # ~1 GB of bf16 copies: every pass streams from HBM
        qn = max(2, (1 << 30) // (2 * w.n * w.k))
        qjobs = [(bf if i == 0 else bf.clone(), torch.empty_like(c0), torch.empty_like(e0)) for i in range(qn)]
        out[f"quantize_mx_{key}"] = quant_passes(torch, fp8w, lean, timer, qjobs, "mx",
                                                 qn * quant_bytes_mx(w.n, w.k))
        del bf, qjobs
        copies = [(c0, e0)] + [(c0.clone(), e0.clone()) for _ in range(copies_n - 1)]
        for m in row_ms(args, wl.ms):
            x = upload_bf16(torch, W.activation(5, m, w.k))
            calls = [(x, c, e, torch.empty((m, w.n), dtype=torch.bfloat16, device="cuda")) for c, e in copies]
            nb = len(calls) * gemv_bytes_mx(m, w.n, w.k)
            g = graph_of(torch, lean.gemv_mx(calls))
            per, _ = timer.run(g.replay, max(10, args.steps // 2), args.warmup)
            row = {"per_call": summarize(per, len(calls), nb)}
            del g
            plan = fp8w.fp8w_grouped_plan_init([c[0] for c in calls], [c[1] for c in calls],
                                               [c[2] for c in calls], [c[3] for c in calls], fmt="mx")
            per_g, _ = timer.run(lean.grouped(plan), max(10, args.steps // 2), args.warmup)
            row["grouped"] = summarize(per_g, len(calls), nb)
            out[f"gemv_mx_{key}_m{m}"] = row
            del plan
        del copies
    log(f"mx: {out}")
    return {"mxfp8": out}


def dequant_bytes(n, k, mx):
    return 3 * n * k + (n * (-(-k // GROUP)) if mx else 4 * (-(-n // TILE)) * (-(-k // TILE)))


def bench_dequant(torch, fp8w, lean, timer, W, args, log):
    """Dequantize to bf16: the dense layer's four weights x 6 copies (block),
    and 16 copies of the MX [8192x2560] weight; one graph-captured pass of
    every call, HBM-bound (1 B in, 2 B out per weight)."""
    lib = fp8w.lib()
    out = {}
    layer = []
    for w in W.WORKLOADS[4].weights:
        c, s = fp8w.fp8w_quantize_block(upload_bf16(torch, w.bits(4)))
        layer.append((c, s))
    jobs = [(c if i == 0 else c.clone(), s if i == 0 else s.clone()) for i in range(6) for c, s in layer]
    outs = [torch.empty(c.shape, dtype=torch.bfloat16, device="cuda") for c, _ in jobs]
    args_c = [(c.data_ptr(), s.data_ptr(), c.shape[0], c.shape[1], o.data_ptr()) for (c, s), o in zip(jobs, outs)]
    nbytes = sum(dequant_bytes(c.shape[0], c.shape[1], False) for c, _ in jobs)

    def run_block():
        st = lean.stream()
        for a in args_c:
            if lib.fp8w_dequantize_block(*a, st):
                raise RuntimeError("fp8w_dequantize_block failed")
    g = graph_of(torch, run_block)
    per, _ = timer.run(g.replay, max(10, args.steps // 4), min(args.warmup, 20))
    out["dequantize_block_dense_layer_x6"] = dict(summarize(per, len(jobs), nbytes), calls_per_pass=len(jobs))
    del g, jobs, outs, layer
    mw = W.WORKLOADS[5].weights[0]
    c0, e0 = fp8w.fp8w_quantize_mx(upload_bf16(torch, mw.bits(5)))
    mj = [(c0, e0)] + [(c0.clone(), e0.clone()) for _ in range(15)]
    mo = [torch.empty(c0.shape, dtype=torch.bfloat16, device="cuda") for _ in mj]
    margs = [(c.data_ptr(), e.data_ptr(), mw.n, mw.k, o.data_ptr()) for (c, e), o in zip(mj, mo)]

    def run_mx():
        st = lean.stream()
        for a in margs:
            if lib.fp8w_dequantize_mx(*a, st):
                raise RuntimeError("fp8w_dequantize_mx failed")
    g = graph_of(torch, run_mx)
    per, _ = timer.run(g.replay, max(10, args.steps // 4), min(args.warmup, 20))
    out[f"dequantize_mx_{mw.n}x{mw.k}_x16"] = dict(summarize(per, len(mj), 16 * dequant_bytes(mw.n, mw.k, True)),
                                                    calls_per_pass=len(mj))
    log(f"dequant: {out}")
    return {"dequantize": out}


def bench_gemm(torch, fp8w, lean, timer, W, args, log):
    """The large-M route (dequantize + rocBLAS bf16 GEMM) on the dense layer's
    four weights at prefill M; TFLOP/s against the bf16 MFMA peak.  Beside it,
    for context, torch.matmul (hipBLASLt) on the already-dequantized bf16
    weight: the GEMM alone."""
    lib = fp8w.lib()
    layer = []
    for w in W.WORKLOADS[4].weights:
        c, s = fp8w.fp8w_quantize_block(upload_bf16(torch, w.bits(4)))
        layer.append((w, c, s))
    ws = torch.empty(max(int(lib.fp8w_gemm_workspace_bytes(c.shape[0], c.shape[1])) for _, c, _ in layer),
                     dtype=torch.uint8, device="cuda")
    out = {}
    for m in (128, 512, 2048):
        xs = {k: upload_bf16(torch, W.activation(4, m, k)) for k in (4096, 12288)}
        calls = [(xs[w.k], c, s, torch.empty((m, w.n), dtype=torch.bfloat16, device="cuda")) for w, c, s in layer]
        flops = sum(2.0 * m * w.n * w.k for w, _, _ in layer)
        cargs = [(x.data_ptr(), m, c.data_ptr(), s.data_ptr(), c.shape[0], c.shape[1], y.data_ptr(),
                  ws.data_ptr(), ws.numel()) for x, c, s, y in calls]

        def run():
            st = lean.stream()
            for a in cargs:
                if lib.fp8w_gemm_block(*a, st):
                    raise RuntimeError("fp8w_gemm_block failed")
        run()
        torch.cuda.synchronize()
        per, _ = timer.run(run, 20, 3, hold_ms=5.0)
        med = statistics.median(per)
        row = {"ms_per_layer": round(med, 4), "TFLOPs": round(flops / (med * 1e-3) / 1e12, 1),
               "pct_of_bf16_peak": round(100 * flops / (med * 1e-3) / PEAK_BF16, 1)}
        deq = [fp8w.fp8w_dequantize_block(c, s) for _, c, s in layer]
        mm = [(x, d) for (x, _, _, _), d in zip(calls, deq)]

        def run_mm():
            for x, d in mm:
                torch.matmul(x, d.t())
        run_mm()
        torch.cuda.synchronize()
        per_mm, _ = timer.run(run_mm, 20, 3, hold_ms=5.0)
        med_mm = statistics.median(per_mm)
        row["bf16_gemm_alone"] = {"ms_per_layer": round(med_mm, 4),
                                  "TFLOPs": round(flops / (med_mm * 1e-3) / 1e12, 1)}
        out[f"m{m}"] = row
        del deq, mm, calls
    log(f"gemm route: {out}")
    return {"gemm_route_dense_layer": out}


def bench_w8a8(torch, fp8w, lean, timer, W, args, state, log):
    """The W8A8 route on the projection set at M = 1, 8, 16: 96 single
    fp8w_gemv_block_w8a8 calls per pass (graph-captured), the activations
    quantized outside the timed region as the pages' raw W8A8 rows are; the
    per-tensor activation quantization timed on its own."""
    wl, bf, codes, scales = state
    lib = fp8w.lib()
    out = {}
    ws = torch.empty(int(lib.fp8w_quantize_act_workspace_bytes()), dtype=torch.uint8, device="cuda")
    for m in (1, 8, 16):
        xq = {}
        for k in (2560, 3072):
            x = upload_bf16(torch, W.activation(2, m, k))
            xq[k] = fp8w.fp8w_quantize_act(x, workspace=ws)
        ys = [torch.empty((m, c.shape[0]), dtype=torch.bfloat16, device="cuda") for c in codes]
        cargs = [(xq[c.shape[1]][0].data_ptr(), xq[c.shape[1]][1].data_ptr(), m, c.data_ptr(), s.data_ptr(),
                  c.shape[0], c.shape[1], y.data_ptr()) for c, s, y in zip(codes, scales, ys)]
        nbytes = sum(gemv_bytes_block(m, c.shape[0], c.shape[1]) - m * c.shape[1] for c in codes)  # fp8 x

        def run():
            st = lean.stream()
            for a in cargs:
                if lib.fp8w_gemv_block_w8a8(*a, st):
                    raise RuntimeError("fp8w_gemv_block_w8a8 failed")
        g = graph_of(torch, run)
        per, _ = timer.run(g.replay, max(10, args.steps // 4), min(args.warmup, 20))
        out[f"m{m}"] = dict(summarize(per, len(cargs), nbytes), ms_per_pass=round(statistics.median(per), 4),
                            launches_per_pass=len(cargs))
        del g
    for m, k in ((1, 2560), (16, 3072), (32, 12288)):
        x = upload_bf16(torch, W.activation(2, m, k))
        c = torch.empty((m, k), dtype=torch.uint8, device="cuda")
        sc = torch.empty(1, dtype=torch.float32, device="cuda")
        a = (x.data_ptr(), m, k, c.data_ptr(), sc.data_ptr(), ws.data_ptr(), ws.numel())

        def q():
            if lib.fp8w_quantize_act(*a, lean.stream()):
                raise RuntimeError("fp8w_quantize_act failed")
        g = graph_of(torch, lambda: [q() for _ in range(32)])
        per, _ = timer.run(g.replay, 20, 3)
        out[f"quantize_act_{m}x{k}_us"] = round(1e3 * statistics.median(per) / 32, 3)
    out["pages_per_pass_ms_context"] = {"raw torch._scaled_mm per-tensor, RTX 6000 Ada": [1.94, 1.93, 1.92],
                                        "per-tensor W8A8 wrapper": [3.62, 3.59, 3.58]}
    log(f"w8a8: {out}")
    return {"w8a8_projection_set": out}


def bench_row_format(torch, fp8w, lean, timer, W, args, state, log):
    """The projection set quantized with one fp32 scale per row (the pages'
    per-row W8A16 route), GEMV at M = 1, 8, 16: one grouped launch per pass,
    and 96 single fp8w_gemv calls (graph-captured)."""
    wl, bf, _, _ = state
    lib = fp8w.lib()
    qs = [fp8w.fp8w_quantize(w, "row") for w in bf]
    codes = [c for c, _ in qs]
    scales = [s for _, s in qs]
    out = {}
    for m in (1, 8, 16):
        xs = {k: upload_bf16(torch, W.activation(2, m, k)) for k in (2560, 3072)}
        ys = [torch.empty((m, c.shape[0]), dtype=torch.bfloat16, device="cuda") for c in codes]
        nbytes = sum(c.shape[0] * c.shape[1] + 4 * c.shape[0] + 2 * m * c.shape[1] + 2 * m * c.shape[0]
                     for c in codes)
        plan = fp8w.fp8w_grouped_plan_init([xs[c.shape[1]] for c in codes], codes, scales, ys, fmt="row")
        per, _ = timer.run(lean.grouped(plan), max(10, args.steps // 2), args.warmup)
        row = {"grouped": dict(summarize(per, len(codes), nbytes), ms_per_pass=round(statistics.median(per), 4))}
        cargs = [(xs[c.shape[1]].data_ptr(), m, c.data_ptr(), s.data_ptr(), fp8w.FORMAT_ROW, c.shape[0],
                  c.shape[1], y.data_ptr(), 0) for c, s, y in zip(codes, scales, ys)]

        def run():
            st = lean.stream()
            for a in cargs:
                if lib.fp8w_gemv(*a, st):
                    raise RuntimeError("fp8w_gemv failed")
        g = graph_of(torch, run)
        per_c, _ = timer.run(g.replay, max(10, args.steps // 4), min(args.warmup, 20))
        row["per_call"] = dict(summarize(per_c, len(codes), nbytes), ms_per_pass=round(statistics.median(per_c), 4))
        del g, plan
        out[f"m{m}"] = row
    out["pages_per_pass_ms_context"] = {"FreeToken per-row W8A16, RTX 6000 Ada": [3.70, 3.07, 3.06]}
    log(f"row format: {out}")
    return {"row_scale_projection_set": out}


def bench_single(torch, fp8w, lean, timer, W, args, log):
    w = W.WORKLOADS[1].weights[0]
    bf = upload_bf16(torch, w.bits(1))
    c0, s0 = fp8w.fp8w_quantize_block(bf)
    x = upload_bf16(torch, W.activation(1, 1, w.k))
    nb = gemv_bytes_block(1, w.n, w.k)
    hot = [(x, c0, s0, torch.empty((1, w.n), dtype=torch.bfloat16, device="cuda"))] * 64
    g = graph_of(torch, lean.gemv_block(hot))
    per, _ = timer.run(g.replay, args.steps, args.warmup)
    out = {"hot_cache_resident": summarize(per, len(hot), len(hot) * nb)}
    pool = [(x, c0.clone(), s0.clone(), torch.empty((1, w.n), dtype=torch.bfloat16, device="cuda"))
            for _ in range(1024)]
    g2 = graph_of(torch, lean.gemv_block(pool))
    per2, _ = timer.run(g2.replay, 10, 2)
    out["pool_1024_copies"] = summarize(per2, len(pool), len(pool) * nb)
    log(f"single [1024x1024]: {out}")
    return {"single_1024x1024": out}


# Every weight shape of the workloads: the projection set, the dense layer
# and the lm_head.
ROUTE_SHAPES = ((6656, 2560), (8192, 2560), (2560, 3072), (4096, 4096), (6144, 4096), (24576, 4096),
                (4096, 12288), (151936, 2048))


def bench_route(torch, fp8w, lean, timer, W, args, log):
    """The single-call VALU / MFMA crossover behind the AUTO rule: for every
    weight shape of the workloads, block and MX scales, a graph-captured pass
    of single calls over ~0.5 GB of weight copies at M = 2..8 on each route
    forced, next to the route AUTO takes.  Codes and scales are random
    (finite codes; the time does not depend on the values)."""
    gen = torch.Generator(device="cuda")
    gen.manual_seed(7)
    names = {fp8w.ROUTE_VALU: "valu", fp8w.ROUTE_MFMA: "mfma"}
    out = {}
    shapes = ROUTE_SHAPES
    if args.route_shapes:
        shapes = tuple(tuple(int(v) for v in sh.split("x")) for sh in args.route_shapes.split(",") if sh)
    for fmt in (f for f in args.route_formats.split(",") if f):
        if fmt not in ("block", "mx"):
            raise SystemExit(f"--route-formats: unknown format {fmt}")
        for n, k in shapes:
            copies = []
            for _ in range(max(2, (1 << 29) // (n * k))):
                c = torch.randint(0, 0x7E, (n, k), dtype=torch.uint8, device="cuda", generator=gen)
                if fmt == "block":
                    s = torch.rand(((n + TILE - 1) // TILE, (k + TILE - 1) // TILE), device="cuda",
                                   generator=gen) * 1e-3 + 1e-4
                else:
                    s = torch.randint(110, 125, (n, (k + GROUP - 1) // GROUP), dtype=torch.uint8, device="cuda",
                                      generator=gen)
                copies.append((c, s))
            for m in row_ms(args, (2, 3, 4, 5, 6, 7, 8)):
                x = (torch.randn((m, k), device="cuda", generator=gen)).to(torch.bfloat16)
                calls = [(x, c, s, torch.empty((m, n), dtype=torch.bfloat16, device="cuda")) for c, s in copies]
                nb = len(calls) * (gemv_bytes_block(m, n, k) if fmt == "block" else gemv_bytes_mx(m, n, k))
                row = {"auto": names[fp8w.fp8w_gemv_auto_route(m, n, k, fmt)], "calls_per_pass": len(calls)}
                for rname, r in (("valu", fp8w.ROUTE_VALU), ("mfma", fp8w.ROUTE_MFMA)):
                    if r == fp8w.ROUTE_VALU and m > 8:
                        continue
                    fn = lean.gemv_block(calls, r) if fmt == "block" else lean.gemv_mx(calls, r)
                    g = graph_of(torch, fn)
                    per, _ = timer.run(g.replay, max(10, args.steps // 4), min(args.warmup, 20))
                    row[rname] = summarize(per, len(calls), nb)
                    del g
                if "valu" in row:
                    t = {rn: row[rn]["us_per_call_p50"] for rn in ("valu", "mfma")}
                    row["auto_vs_best_pct"] = round(100 * (t[row["auto"]] / min(t.values()) - 1), 1)
                out[f"{fmt}_{n}x{k}_m{m}"] = row
            del copies
            torch.cuda.empty_cache()
    log(f"route crossover: {out}")
    return {"route_crossover_single_calls": out}


# ------------------------------------------------------ HBM read ceiling --

def read_ceiling(torch, fp8w, timer, log, gib=2, reps=100, warmup=150):
    """GB/s of fp8w_read_ceiling over a `gib` GiB buffer: a kernel that only
    reads HBM, with the GEMV's load pattern, in this session.  Warmed up for
    ~45 ms like the GEMV (past the power-management transient: ten warm-up
    reads leave the timed ones in its slow phase, 5 % low)."""
    buf = torch.empty(gib << 30, dtype=torch.uint8, device="cuda")
    buf.fill_(1)
    out = torch.empty(2048, dtype=torch.int32, device="cuda")
    fn = fp8w.lib().fp8w_read_ceiling
    a = (buf.data_ptr(), buf.numel(), out.data_ptr(), out.numel())
    def launch():
        rc = fn(*a, torch.cuda.current_stream().cuda_stream)
        if rc:
            raise RuntimeError(f"fp8w_read_ceiling failed: {rc}")
    per, _ = timer.run(launch, reps, warmup)
    med = statistics.median(per)
    res = {"GBps": round(buf.numel() / (med * 1e-3) / 1e9, 1), "bytes": buf.numel(),
           "ms_p50": round(med, 4), "kernel": "k_read_xor (16-byte non-temporal loads, XOR fold)"}
    log(f"read ceiling: {res}")
    del buf, out
    torch.cuda.empty_cache()
    return res


# ------------------------------------------------------------ CPU baseline --

def cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            return next((ln.split(":", 1)[1].strip() for ln in fh if ln.startswith("model name")), "")
    except OSError:
        return ""


def cpu_baseline(W, log, min_seconds=10.0, max_passes=40):
    """The CPU oracle (unchanged, plain C driven through ctypes) on the host
    cores of this run, as GB/s of the same algorithmic bytes as the GPU rows:

    * value: fp64 GEMV passes at M = 1 over the whole projection set on all
      host threads (its own block quantization of the 96 weights first),
      repeated until about `min_seconds`;
    * per_op: on one [8192x2560] projection weight, block quantization and
      the fp64 GEMV at M = 1, 8, 16, and MX quantization of the MXFP8
      workload's [8192x2560] weight, each on 1 thread and on all threads."""
    import platform
    import oracle
    wl = W.WORKLOADS[2]
    threads = oracle.max_threads()
    x = {k: W.activation(2, 1, k) for k in (2560, 3072)}
    t_q = 0.0
    quantized = []
    for w in wl.weights:
        bits = w.bits(2)
        t = time.perf_counter()
        quantized.append((w.k, oracle.quantize_block(bits)))
        t_q += time.perf_counter() - t
    pass_bytes = sum(gemv_bytes_block(1, w.n, w.k) for w in wl.weights)
    passes, t_g = 0, 0.0
    while passes < max_passes and (passes == 0 or t_g < min_seconds):
        t = time.perf_counter()
        for k, (c, s) in quantized:
            oracle.gemv_block_f64(x[k], c, s)
        t_g += time.perf_counter() - t
        passes += 1
    del quantized
    qbytes = sum(quant_bytes_block(w.n, w.k) for w in wl.weights)

    def timed(fn, nbytes):
        t = time.perf_counter()
        r = fn()
        dt = time.perf_counter() - t
        return r, round(nbytes / dt / 1e9, 4)

    w = wl.weights[12]
    n, k = w.n, w.k
    bits = w.bits(2)
    wmx = W.WORKLOADS[5].weights[0]
    bits_mx = wmx.bits(5)
    per_op = {}
    try:
        for th in (1, threads):
            oracle.set_threads(th)
            (c, s), per_op.setdefault("quantize_block", {})[f"t{th}"] = timed(
                lambda: oracle.quantize_block(bits), quant_bytes_block(n, k))
            _, per_op.setdefault("quantize_mx", {})[f"t{th}"] = timed(
                lambda: oracle.quantize_mx(bits_mx), quant_bytes_mx(wmx.n, wmx.k))
            for m in (1, 8, 16):
                xm = W.activation(2, m, k)
                _, per_op.setdefault(f"gemv_block_m{m}", {})[f"t{th}"] = timed(
                    lambda: oracle.gemv_block_f64(xm, c, s), gemv_bytes_block(m, n, k))
    finally:
        oracle.set_threads(threads)
    res = {"value": round(passes * pass_bytes / t_g / 1e9, 3), "unit": "GB/s", "cores": threads,
           "kind": "oracle",
           "sample": f"{passes} fp64 GEMV passes at M=1 over the 48-layer projection set "
                     f"({len(wl.weights)} weights, {pass_bytes} algorithmic bytes per pass) on the "
                     f"oracle's own codes, {threads} threads",
           "seconds": round(t_g, 3),
           "nproc": os.cpu_count(), "cpu_model": cpu_model() or platform.processor(),
           "quantize_block_projection_set_GBps": round(qbytes / t_q / 1e9, 3),
           "quantize_block_projection_set_seconds": round(t_q, 3),
           "per_op_GBps": per_op,
           "per_op_weights": {"quantize_block, gemv": f"projection [{n}x{k}]",
                              "quantize_mx": f"MXFP8 workload [{wmx.n}x{wmx.k}]",
                              "t1 / tN": f"1 thread / {threads} threads"}}
    log(f"cpu baseline: {res}")
    return res


# -------------------------------------------------------------------- main --

def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the FP8 GEMV path has no multi-GPU leg "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    import torch

    import fp8_block_scaled_02_amd as fp8w
    from fp8_block_scaled_02_amd import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a ROCm GPU", file=sys.stderr)
        sys.exit(1)

    def log(msg):
        print(f"[bench] {msg}", file=sys.stderr, flush=True)

    rows_wanted = [r for r in args.rows.split(",") if r]
    fp8w.lib()
    torch.cuda.set_device(0)
    timer = Timer(torch)
    lean = Lean(fp8w, torch)
    rows = {}
    headline = None
    if args.calibrate_copy_mib:
        n = args.calibrate_copy_mib << 20
        a = torch.empty(n, dtype=torch.uint8, device="cuda")
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        log(f"calibration copy of {args.calibrate_copy_mib} MiB done")
    if any(r in rows_wanted for r in ("proj", "quant", "w8a8", "row")):
        state = projection_set(torch, fp8w, W, log)
        if "quant" in rows_wanted:
            rows.update(bench_quant(torch, fp8w, lean, timer, W, args, state, log))
        if "w8a8" in rows_wanted:
            rows.update(bench_w8a8(torch, fp8w, lean, timer, W, args, state, log))
        if "row" in rows_wanted:
            rows.update(bench_row_format(torch, fp8w, lean, timer, W, args, state, log))
        if "proj" in rows_wanted:
            proj, headline = bench_proj(torch, fp8w, lean, timer, W, args, state, log)
            rows["projection_set"] = proj
        del state
        torch.cuda.empty_cache()
    for name, fn in (("lm_head", bench_lm_head), ("dense", bench_dense), ("mx", bench_mx),
                     ("single", bench_single), ("dequant", bench_dequant), ("gemm", bench_gemm),
                     ("route", bench_route)):
        if name in rows_wanted:
            rows.update(fn(torch, fp8w, lean, timer, W, args, log))
            torch.cuda.empty_cache()
    ceiling = None if headline is None else read_ceiling(torch, fp8w, timer, log)
    cpu = None if args.no_cpu or headline is None else cpu_baseline(W, log)

    if headline is None:
        print(json.dumps({"rows": rows}))
        return
    ms_per_step = headline["total_ms"] / args.steps
    value = headline["bytes"] / (ms_per_step * 1e-3) / 1e9
    per_call = headline["row"]["per_call"]
    out = {
        "metric": "us/call + achieved HBM GB/s (% of peak), block-FP8 W8A16 GEMV, M=1..32",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "us_per_call": round(1e3 * ms_per_step / headline["calls"], 3),
        "pct_of_peak": round(100 * value * 1e9 / PEAK_HBM, 1),
        "per_call_launches": {"us_per_call": per_call["us_per_call_p50"], "GBps": per_call["GBps"],
                              "pct_of_peak": per_call["pct_of_peak"],
                              "note": "96 single-GEMV launches per pass, graph-captured"},
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": round(value / ceiling["GBps"], 4),
        "vs_baseline_basis": "the pass's GB/s over fp8w_read_ceiling's in this session (a pure 2 GiB "
                             "HBM read with the GEMV's 16-byte non-temporal loads)",
        "pages_context": {"block-FP8 Triton, 48-layer pass at M=1, RTX 6000 Ada (other hardware)": "3.78 ms",
                          "this pass": f"{ms_per_step:.4f} ms"},
        "dtype": "bf16",
        "weights": "fp8_e4m3fn, fp32 128x128 block scales",
        "data": "synthetic",
        "config": {"workload": "projection_set_48_layers", "m": 1, "calls_per_step": headline["calls"],
                   "shapes": "12x[6656x2560] + 36x[8192x2560] + 48x[2560x3072]",
                   "bytes_per_step": headline["bytes"],
                   "execution": "the 96 independent GEMVs of a pass in one grouped launch "
                                "(fp8w_gemv_grouped) per step, HIP events on the launch stream"},
        "roofline": {"bound": "hbm", "achieved": round(value, 1), "peak": PEAK_HBM / 1e9, "unit": "GB/s",
                     "frac": round(value * 1e9 / PEAK_HBM, 4), "traffic": counted_traffic(),
                     "traffic_unit": "bytes per launch",
                     "kernel": "k_gemv_valu_stream<R=4, C=3, block> (grouped, m=1)",
                     "avg_launch_us": round(ms_per_step * 1e3, 3),
                     "bytes_per_launch": headline["bytes"],
                     "read_ceiling_GBps": ceiling["GBps"],
                     "frac_of_read_ceiling": round(value / ceiling["GBps"], 4)},
        "cpu_baseline": cpu,
        "rows": rows,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
