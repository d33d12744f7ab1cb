#!/usr/bin/env python3
"""Throughput of the low-bit linear layer on one MI355X.

Metric: ternary GEMV HBM GB/s (% of peak) at batch 1, and batched GEMM int8
TOPS (% of MFMA peak).

One step = one pass of the hot path over one batch of seeded synthetic input:
per-token int8 activation quantisation of every matrix's input, then the
low-bit product of every weight matrix of the workload, with packed weights,
scales and inputs already resident in HBM.  Packing (the offline export step)
is done before timing.  The step is captured once in a HIP graph and replayed.

Default workload (the GEMV line, `value`): the 4B-class ternary decode pass -
36 layer-equivalents x {4 x [2560, 2560], 2 x [9728, 2560], 1 x [2560, 9728]},
group-128 scales, 1 token per call (1.03 GB of packed codes + scales).
The batched-GEMM figure is measured in the same run on the int4 prefill pass
(20 layers x {[3840,1280], [1280,1280], 2 x [3584,1280], [1280,3584]},
4096 tokens) and reported under "gemm".

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--tokens 1]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import re
import sys
import time
from concurrent.futures import ThreadPoolExecutor

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
I8_PEAK_TOPS = 5000.0          # MI355X dense int8 MFMA, TOPS
F16_PEAK_TFLOPS = 2500.0       # MI355X dense fp16 / bf16 MFMA, TFLOP/s
METRIC = "ternary GEMV HBM GB/s (% peak) at batch 1; batched GEMM int8 TOPS (% MFMA peak)"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ------------------------------------------------------------------ set-up

class Pass:
    """Every matrix of one workload pass, packed and resident on the GPU, with
    per-call activations stacked by k so one act-quant launch serves all
    inputs of equal width."""

    def __init__(self, wl, tokens, entry, layers=None, threads=16, weights_from=None):
        import torch
        import bit_weight_linear_bitlinear_amd as lb
        import workloads

        self.wl, self.t, self.entry = wl, tokens, entry
        self.lb = lb
        n_layers = wl.layers if layers is None else layers
        self.mats = [(layer, mi, m) for layer in range(n_layers) for mi, m in enumerate(wl.matrices)
                     if layer < m.count]
        fmt, scale = lb.FORMATS[wl.fmt], lb.SCALES[wl.scale]
        flags = lb.FLAG_TANH3 if wl.tanh_premap else 0
        if weights_from is not None:                     # same packed weights, other token count
            assert weights_from.mats == self.mats
            self.desc, self.packed, self.scales = weights_from.desc, weights_from.packed, weights_from.scales
            xs = [workloads.workload_activations(wl, layer, mi, tokens, m.k) for layer, mi, m in self.mats]
            self._activations(xs, tokens, entry)
            return

        def prep(item):
            layer, mi, m = item
            d = lb.lowbit_describe(fmt, scale, m.n, m.k, wl.group, flags)
            w = workloads.latent_weights(wl.index, layer, mi, m.n, m.k)
            packed = np.empty(d.packed_bytes, np.uint8)
            scales = np.empty(d.n_scales, np.float32)
            lb.lowbit_pack(d, w, packed, scales)
            x = workloads.workload_activations(wl, layer, mi, tokens, m.k)
            return d, packed, scales, x

        t0 = time.time()
        self.desc, self.packed, self.scales = [], [], []
        xs = []
        with ThreadPoolExecutor(threads) as ex:
            for d, packed, scales, x in ex.map(prep, self.mats):
                self.desc.append(d)
                self.packed.append(torch.from_numpy(packed).cuda())
                self.scales.append(torch.from_numpy(scales).cuda())
                xs.append(x)
        log(f"[bench] {wl.name}: {len(self.mats)} matrices generated and packed in {time.time() - t0:.1f}s")
        self._activations(xs, tokens, entry)

    def _activations(self, xs, tokens, entry):
        import torch
        lb = self.lb
        # activations stacked per k; q / sx / y views per matrix
        self.kgroups = {}
        for i, (_, _, m) in enumerate(self.mats):
            self.kgroups.setdefault(m.k, []).append(i)
        self.x, self.q, self.sx = {}, {}, {}
        self.views = [None] * len(self.mats)
        self.pos = {}                                    # matrix -> (k, position in its k-stack)
        for k, idx in self.kgroups.items():
            for j, i in enumerate(idx):
                self.pos[i] = (k, j)
        for k, idx in self.kgroups.items():
            rows = len(idx) * tokens
            self.x[k] = torch.from_numpy(np.concatenate([xs[i] for i in idx], axis=0)).cuda()
            self.q[k] = torch.empty((rows, k), dtype=torch.int8, device="cuda")
            self.sx[k] = torch.empty((rows,), dtype=torch.float32, device="cuda")
            for j, i in enumerate(idx):
                self.views[i] = (self.q[k][j * tokens:(j + 1) * tokens], self.sx[k][j * tokens:(j + 1) * tokens])
        self.y = [torch.empty((tokens, m.n), dtype=torch.float32, device="cuda") for _, _, m in self.mats]
        self.xv = [None] * len(self.mats)
        for k, idx in self.kgroups.items():
            for j, i in enumerate(idx):
                self.xv[i] = self.x[k][j * tokens:(j + 1) * tokens]
        self.status = torch.zeros(1, dtype=torch.int32, device="cuda")
        self.xs = xs
        self.fn = lb.lowbit_linear if entry == "gemv" else lb.lowbit_linear_batched

        # algorithmic accounting
        self.linear_bytes = [d.packed_bytes + 4 * d.n_scales + tokens * d.k + 4 * tokens + 4 * tokens * d.n
                             for d in self.desc]
        self.linear_ops = [2 * tokens * d.n * d.k for d in self.desc]
        # what one pass must move at least: fp32 x read, codes and scales of x
        # written, packed weights and scales read, fp32 y written (the separate
        # schedules also read the codes back: that re-read is their overhead)
        self.pass_bytes = [d.packed_bytes + 4 * d.n_scales + 5 * tokens * d.k + 4 * tokens + 4 * tokens * d.n
                           for d in self.desc]

    def act_quant(self):
        for k in self.kgroups:
            self.lb.lowbit_act_quant(self.x[k], self.q[k], self.sx[k])

    def linears(self):
        for i, d in enumerate(self.desc):
            q, sx = self.views[i]
            self.fn(d, self.packed[i], self.scales[i], q, sx, self.y[i])

    def _grouped(self, idx):
        return self.lb.GroupedCall([self.desc[i] for i in idx], [self.packed[i] for i in idx],
                                   [self.scales[i] for i in idx], [self.views[i][0] for i in idx],
                                   [self.views[i][1] for i in idx], [self.y[i] for i in idx],
                                   batched=self.entry == "gemm")

    def _grouped_fused(self, idx):
        return self.lb.GroupedFusedCall([self.desc[i] for i in idx], [self.packed[i] for i in idx],
                                        [self.scales[i] for i in idx], [self.xv[i] for i in idx],
                                        [self.views[i][0] for i in idx], [self.views[i][1] for i in idx],
                                        [self.y[i] for i in idx], self.status)

    def _quant_rows(self, idx):
        """act-quant of the inputs of matrices idx (adjacent in one k-stack)
        as one call"""
        k, j0 = self.pos[idx[0]]
        assert all(self.pos[i] == (k, j0 + n) for n, i in enumerate(idx))
        r0, r1 = j0 * self.t, (j0 + len(idx)) * self.t
        x, q, sx = self.x[k][r0:r1], self.q[k][r0:r1], self.sx[k][r0:r1]
        return lambda: self.lb.lowbit_act_quant(x, q, sx)

    def build_schedules(self):
        """grouped: every matrix of equal k in one call, on inputs quantised
        beforehand by the act-quant kernel (one launch per k); grouped_fused:
        the same calls from fp32 inputs, the quantiser run in the product
        kernel's prologue.  The layer schedules issue the calls a decoder
        layer's data dependencies allow - q/k/v together, o, gate/up together,
        down: layer quantises every input up front (one launch per k),
        layer_dep quantises each call's inputs right before it (what a model
        whose next input is the previous output must do), layer_fused does that
        inside the product kernel.  A prefill pass has the grouped schedule
        only (lowbit_linear_batched_grouped, at most 64 products per launch)."""
        self.grouped_calls = [self._grouped(idx) for idx in self.kgroups.values()]
        if self.entry == "gemm":
            return
        self.fused_calls = [self._grouped_fused(idx) for idx in self.kgroups.values()]
        names = [m.name for _, _, m in self.mats]
        self.layer_calls, self.layer_fused_calls, self.layer_dep_calls = [], [], []
        by_layer = {}
        for i, (layer, _, _) in enumerate(self.mats):
            by_layer.setdefault(layer, []).append(i)
        for layer, idx in sorted(by_layer.items()):
            sets = [[i for i in idx if names[i] in ("attn0", "attn1", "attn2")],
                    [i for i in idx if names[i] == "attn3"],
                    [i for i in idx if names[i] in ("gate", "up")],
                    [i for i in idx if names[i] == "down"]]
            for s_ in sets:
                if not s_:
                    continue
                self.layer_calls.append(self._grouped(s_))
                self.layer_fused_calls.append(self._grouped_fused(s_))
                self.layer_dep_calls += [self._quant_rows(s_), self.layer_calls[-1]]

    def launches(self, calls):
        if self.entry == "gemm":
            return sum((c.count + 63) // 64 for c in calls)
        return sum((c.count + 255) // 256 * ((c.t + 15) // 16) for c in calls)

    def step(self, schedule="per_matrix"):
        if schedule in ("grouped_fused", "layer_fused", "layer_dep"):
            calls = {"grouped_fused": self.fused_calls, "layer_fused": self.layer_fused_calls,
                     "layer_dep": self.layer_dep_calls}[schedule]
            for c in calls:
                c()
            return
        self.act_quant()
        if schedule == "grouped":
            for c in self.grouped_calls:
                c()
        elif schedule == "layer":
            for c in self.layer_calls:
                c()
        else:
            self.linears()

    @property
    def step_bytes(self):
        return sum(self.pass_bytes)


def capture(fn):
    """Capture fn's launches into a HIP graph; returns a replay callable or None."""
    import torch
    try:
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
        return g.replay
    except Exception as e:   # eager launches are still correct, just slower
        log(f"[bench] graph capture unavailable ({e}); timing eager launches")
        return None


def time_steps(run, steps, warmup, per_step=None):
    """Seconds for `steps` runs between two HIP events on the current stream
    (and the wall time); per_step, a list, receives each run's own duration
    (an event recorded between consecutive runs)."""
    import torch
    for _ in range(warmup):
        run()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1 if per_step is not None else 2)]
    wall0 = time.perf_counter()
    ev[0].record()
    for i in range(steps):
        run()
        if per_step is not None:
            ev[i + 1].record()
    if per_step is None:
        ev[1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    if per_step is not None:
        per_step.extend(ev[i].elapsed_time(ev[i + 1]) / 1e3 for i in range(steps))
    return ev[0].elapsed_time(ev[-1]) / 1e3, wall


def step_stats(per_step):
    v = np.asarray(per_step) * 1e3
    return {"median_ms": round(float(np.median(v)), 4), "min_ms": round(float(v.min()), 4),
            "max_ms": round(float(v.max()), 4), "steps": len(v)}


def calibration(nbytes=2 << 30, reps=5, mfma_iters=40000):
    """The device's own ceilings (the library's calibration kernels): a 16-byte
    non-temporal read stream over nbytes (8x the 256 MB last-level cache), and
    the int8 matrix-core loop (two wavefronts per SIMD, back-to-back
    v_mfma_i32_32x32x32_i8).  Medians of `reps` event-timed launches."""
    import torch
    lb = __import__("bit_weight_linear_bitlinear_amd")
    buf = torch.empty(nbytes // 4, dtype=torch.int32, device="cuda").fill_(7)
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = {}
    for name, fn in (("read", lambda: lb.lowbit_calib_read(buf, sink)),
                     ("mfma", lambda: lb.lowbit_calib_mfma_i8(mfma_iters, sink))):
        fn()
        torch.cuda.synchronize()
        t = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            t.append(e0.elapsed_time(e1) / 1e3)
        out[name] = float(np.median(t))
    ops = lb.lowbit_calib_mfma_i8(mfma_iters, sink)
    torch.cuda.synchronize()
    del buf
    read_gbs = nbytes / out["read"] / 1e9
    tops = ops / out["mfma"] / 1e12
    return {"read_stream_GBps": round(read_gbs, 1), "read_bytes": nbytes,
            "read_frac_of_spec": round(read_gbs / HBM_PEAK_GBS, 4),
            "mfma_i8_TOPS": round(tops, 1), "mfma_i8_frac_of_spec": round(tops / I8_PEAK_TOPS, 4),
            "what": "lowbit_calib_read (16-byte non-temporal read stream, 8x the last-level cache) and "
                    "lowbit_calib_mfma_i8 (back-to-back 32x32x32 int8 MFMAs, two wavefronts per SIMD), "
                    f"medians of {reps} launches"}


def per_launch_grouped(p: Pass, calls, reps: int, fused: bool):
    """Average duration of one gemv launch of a grouped schedule: the gemv
    launches alone (for the unfused calls, inputs quantised beforehand)
    captured in a HIP graph and replayed `reps` times between two HIP events on
    the replaying stream; a call of c matrices issues ceil(c / 40) launches.
    Returns (seconds, algorithmic bytes) per launch."""
    import torch
    if not fused:
        p.act_quant()
    torch.cuda.synchronize()

    def gemvs():
        for c in calls:
            c()
    run = capture(gemvs) or gemvs
    run()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        run()
    e1.record()
    torch.cuda.synchronize()
    total = e0.elapsed_time(e1) / 1e3
    n_launch = p.launches(calls) * reps
    per_pass = sum(p.pass_bytes) if fused else sum(p.linear_bytes)
    return total / n_launch, per_pass / p.launches(calls)


def committed_traffic():
    """HBM bytes per grouped gemv launch from the committed rocprofv3 counter
    summary (FETCH_SIZE and WRITE_SIZE scaled by a copy of known size), or None
    when the GEMV sources have changed since those counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "gemv_ternary_4b_t1_traffic.md")
    try:
        text = open(path).read()
    except OSError:
        return None
    vals = dict(re.findall(r"^(traffic_bytes_per_launch|kernel_source_sha256): (\S+)$", text, re.M))
    h = hashlib.sha256()
    for f in ("gemv_kernel.hpp", "gemv.hip", "gemv.hpp", "device_common.hpp"):
        with open(os.path.join(ROOT, "bit_weight_linear_bitlinear_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    if vals.get("kernel_source_sha256") != h.hexdigest() or "traffic_bytes_per_launch" not in vals:
        return None
    return float(vals["traffic_bytes_per_launch"])


def gemm_pass(p: Pass, steps: int, no_graph: bool = False):
    """A prefill pass both ways: every product as its own launch, and equal-k
    products as grouped launches; seconds per step of each.  Then the
    average grouped launch (inputs quantised beforehand), timed like
    per_launch_grouped: (seconds, bytes, ops) per launch."""
    import torch
    p.build_schedules()
    res = {}
    p.grouped_step_times = []
    for sched in ("per_matrix", "grouped"):
        fn = (lambda sc=sched: p.step(sc))
        run = None if no_graph else capture(fn)
        el, _ = time_steps(run or fn, steps, 1, per_step=p.grouped_step_times if sched == "grouped" else None)
        res[sched] = el / steps
    p.act_quant()
    torch.cuda.synchronize()

    def prods():
        for c in p.grouped_calls:
            c()
    run = capture(prods) or prods
    run()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 3
    e0.record()
    for _ in range(reps):
        run()
    e1.record()
    torch.cuda.synchronize()
    n = p.launches(p.grouped_calls)
    dur = e0.elapsed_time(e1) / 1e3 / (reps * n)
    return res, (dur, sum(p.linear_bytes) / n, sum(p.linear_ops) / n)


def per_launch(p: Pass, reps: int):
    """Average duration of the product kernel: every product of the pass
    (inputs quantised beforehand) captured in a HIP graph and replayed `reps`
    times between two HIP events on the replaying stream."""
    import torch
    p.act_quant()
    torch.cuda.synchronize()

    def products():
        for i, d in enumerate(p.desc):
            q, sx = p.views[i]
            p.fn(d, p.packed[i], p.scales[i], q, sx, p.y[i])
    run = capture(products) or products
    run()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        run()
    e1.record()
    torch.cuda.synchronize()
    total = e0.elapsed_time(e1) / 1e3
    n = len(p.desc)
    return total / (n * reps), sum(p.linear_bytes) / n, sum(p.linear_ops) / n


def gemm_shapes_vs_library(p: Pass, reps: int = 10):
    """Each distinct product shape of a prefill pass as its own launch (one
    matrix, inputs quantised beforehand, 'reps' launches captured in a HIP
    graph), next to the ROCm library's plain int8 GEMM (torch._int_mm, int8 x
    int8 -> int32: unpacked int8 weights, no scales, no fp32 output; launched
    eagerly, back to back) on the same t, n, k.  Context for the matrix-core
    fraction, not a parity check."""
    import torch
    p.act_quant()
    torch.cuda.synchronize()
    seen, rows = set(), []
    g = torch.Generator(device="cuda").manual_seed(11)
    for i, (_, _, m) in enumerate(p.mats):
        if (m.n, m.k) in seen:
            continue
        seen.add((m.n, m.k))
        d, (q, sx) = p.desc[i], p.views[i]
        ops = 2 * p.t * m.n * m.k
        body = (lambda i=i, d=d, q=q, sx=sx: [p.fn(d, p.packed[i], p.scales[i], q, sx, p.y[i]) for _ in range(reps)])
        el, _ = time_steps(capture(body) or body, 3, 1)
        ours = el / (3 * reps)
        a = torch.randint(-127, 128, (p.t, m.k), dtype=torch.int8, device="cuda", generator=g)
        b = torch.randint(-7, 8, (m.n, m.k), dtype=torch.int8, device="cuda", generator=g)
        lib_us = None
        try:
            lbody = (lambda: [torch._int_mm(a, b.t()) for _ in range(reps)])
            el, _ = time_steps(lbody, 3, 1)      # eager: the library call is not captured
            lib_us = el / (3 * reps)
        except Exception as e:   # the library path may be missing on some builds
            log(f"[bench] torch._int_mm unavailable: {e}")
        rows.append({"n": m.n, "k": m.k, "t": p.t, "us": round(ours * 1e6, 2),
                     "TOPS": round(ops / ours / 1e12, 1), "pct_mfma_peak": round(100 * ops / ours / 1e12 / I8_PEAK_TOPS, 2),
                     "library_int8_us": None if lib_us is None else round(lib_us * 1e6, 2),
                     "library_int8_pct_mfma_peak": None if lib_us is None else
                     round(100 * ops / lib_us / 1e12 / I8_PEAK_TOPS, 2)})
        del a, b
    log(f"[bench] gemm shapes vs library int8: {rows}")
    return rows


def gemm_profile(args):
    """The int4 prefill pass alone as the bench runs it (one act-quant launch
    per k, equal-k products as grouped launches), then each distinct GEMM
    shape timed on its own (HIP events on the launching stream)."""
    import torch
    import workloads
    wl4 = workloads.BY_NAME["int4_t4nt"]
    p4 = Pass(wl4, wl4.tokens[0], "gemm", layers=args.layers)
    p4.build_schedules()
    fn = lambda: p4.step("grouped")
    run = (None if args.no_graph else capture(fn)) or fn
    el, _ = time_steps(run, args.steps, args.warmup)
    st = el / args.steps
    log(f"[bench] gemm pass: {sum(p4.linear_ops) / st / 1e12:.1f} TOPS/step, {st * 1e3:.3f} ms/step, "
        f"{p4.launches(p4.grouped_calls)} grouped launches")
    p4.act_quant()
    torch.cuda.synchronize()
    seen = {}
    for i, (layer, mi, m) in enumerate(p4.mats):
        seen.setdefault((m.n, m.k), i)
    for (n, k), i in seen.items():
        q, sx = p4.views[i]
        d = p4.desc[i]
        for _ in range(2):
            p4.fn(d, p4.packed[i], p4.scales[i], q, sx, p4.y[i])
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = 10
        e0.record()
        for _ in range(reps):
            p4.fn(d, p4.packed[i], p4.scales[i], q, sx, p4.y[i])
        e1.record()
        torch.cuda.synchronize()
        dt = e0.elapsed_time(e1) / reps / 1e3
        ops = 2.0 * p4.t * n * k
        log(f"[bench] gemm N={n} K={k} T={p4.t}: {dt * 1e6:.1f} us, {ops / dt / 1e12:.1f} TOPS "
            f"({100 * ops / dt / 1e12 / I8_PEAK_TOPS:.1f}% of peak)")


def copy_calibration(nbytes=1 << 30, reps=5):
    """A plain copy of known size (torch's copy kernel): its rate is the
    practical streaming ceiling of this GPU, and its FETCH_SIZE / WRITE_SIZE
    counters scale the GEMV's counters into bytes."""
    import torch
    a = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    b.copy_(a)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    t = e0.elapsed_time(e1) / 1e3 / reps
    del a, b
    return {"bytes_read": nbytes, "bytes_written": nbytes, "GBps_read_plus_write": round(2 * nbytes / t / 1e9, 1),
            "us": round(t * 1e6, 1)}


# ------------------------------------------------------------- correctness

def sampled_check(p: Pass, picks, rows_per=48, seed=0):
    """Full-size parity on sampled outputs: the oracle recomputes sampled weight
    rows (group/row scales are row-local) for every token of picked matrices."""
    import torch
    import oracle
    import workloads
    wl = p.wl
    rng = np.random.default_rng(seed)
    worst = 0.0
    for i in picks:
        layer, mi, m = p.mats[i]
        d = p.desc[i]
        q, sx = p.views[i]
        y = torch.empty((p.t, m.n), dtype=torch.float32, device="cuda")
        acc = torch.empty((p.t, m.n, d.n_groups), dtype=torch.int32, device="cuda")
        p.fn(d, p.packed[i], p.scales[i], q, sx, y, acc)
        torch.cuda.synchronize()
        rows = np.sort(rng.choice(m.n, size=min(rows_per, m.n), replace=False))
        w = workloads.latent_weights(wl.index, layer, mi, m.n, m.k)[rows]
        if wl.scale == "tensor":
            raise RuntimeError("sampled rows need row-local scales")
        pk, sc, _, _ = oracle.quantize_and_pack(w, wl.fmt, wl.scale, wl.group, wl.tanh_premap)
        q_ref, sx_ref, _ = oracle.act_quant(p.xs[i])
        assert (q.cpu().numpy() == q_ref).all(), "activation codes differ"
        y32, y64, acc_ref = oracle.linear(pk, sc, wl.fmt, wl.scale, wl.group, len(rows), m.k, q_ref, sx_ref)
        a = acc.cpu().numpy()[:, rows]
        assert (a == acc_ref).all(), f"matrix {i}: accumulators differ"
        yy = y.cpu().numpy()[:, rows].astype(np.float64)
        err = np.abs(yy - y32)
        assert (err <= 1e-6 + 1e-5 * np.abs(y32)).all(), f"matrix {i}: y out of tolerance"
        if p.entry == "gemv":
            # the fused entry on the same fp32 input: codes, scales and y equal
            # to the separate path's bit for bit
            qf, sxf, yf = torch.empty_like(q), torch.empty_like(sx), torch.empty_like(y)
            p.lb.lowbit_linear_fused(d, p.packed[i], p.scales[i], p.xv[i], qf, sxf, yf)
            torch.cuda.synchronize()
            assert (qf.cpu().numpy() == q_ref).all(), f"matrix {i}: fused activation codes differ"
            assert torch.equal(sxf, sx) and torch.equal(yf, y), f"matrix {i}: fused path differs"
        worst = max(worst, float((err / (1e-6 + 1e-5 * np.abs(y32))).max()))
    return {"matrices": len(picks), "rows_each": rows_per, "acc_bit_exact": True,
            "fused_equals_separate": True if p.entry == "gemv" else None,
            "y_worst_frac_of_tol": round(worst, 4)}


# --------------------------------------------------------------- CPU oracle

def _oracle_items(wl, layers, tokens, token_rows=None):
    """The oracle's inputs for the first `layers` layer-equivalents of a
    workload: (matrix, packed, scales, x) with x the workload's activations at
    `tokens` rows per call, cut to the first `token_rows` (None: all); weights
    packed by the oracle, untimed."""
    import oracle
    import workloads
    items = [(layer, mi, m) for layer in range(min(layers, wl.layers)) for mi, m in enumerate(wl.matrices)
             if layer < m.count]

    def prep(item):
        layer, mi, m = item
        w = workloads.latent_weights(wl.index, layer, mi, m.n, m.k)
        pk, sc, _, _ = oracle.quantize_and_pack(w, wl.fmt, wl.scale, wl.group, wl.tanh_premap)
        x = workloads.workload_activations(wl, layer, mi, tokens, m.k)
        if token_rows is not None:
            x = np.ascontiguousarray(x[:token_rows])
        return m, pk, sc, x

    with ThreadPoolExecutor(8) as ex:
        return list(ex.map(prep, items))


def _oracle_rate(wl, items, budget_s):
    """act-quant + unpack + integer product + fp32 epilogue over every item,
    repeated until budget_s of timed work (at least once): bytes and ops
    counted as the GPU step counts them (fp32 x read, codes and s_x written,
    packed codes and scales read, fp32 y written; 2 t n k operations)."""
    import oracle
    spent, nbytes, nops, passes = 0.0, 0, 0, 0
    while passes == 0 or spent < budget_s:
        for m, pk, sc, x in items:
            t = x.shape[0]
            t0 = time.perf_counter()
            q, sx, _ = oracle.act_quant(x)
            oracle.linear(pk, sc, wl.fmt, wl.scale, wl.group, m.n, m.k, q, sx)
            spent += time.perf_counter() - t0
            nbytes += pk.size + 4 * sc.size + 5 * t * m.k + 4 * t + 4 * t * m.n
            nops += 2 * t * m.n * m.k
        passes += 1
    return {"GBps": round(nbytes / spent / 1e9, 4), "GOPS": round(nops / spent / 1e9, 3),
            "wall_s": round(spent, 2), "threads": oracle.num_threads(), "passes": passes}


def cpu_baseline(wl, tokens, budget_s=3.0, sample_layers=2):
    """The oracle as it stands, on the host's cores, beside the GPU figures:
    the headline (the 4B-class decode pass at `tokens` tokens) over a bounded
    sample of its layer-equivalents, then every workload (the 4B-class pass at
    1, 4 and 16 tokens), each over a stated sample, and the single-thread
    comparables.  A reported baseline, not a target."""
    items = _oracle_items(wl, sample_layers, tokens)
    r = _oracle_rate(wl, items, budget_s)
    out = {"value": r["GBps"], "unit": "GB/s", "cores": r["threads"], "kind": "oracle",
           "sample": f"{len(items)} matrices ({min(sample_layers, wl.layers)} of {wl.layers} layer-equivalents) "
                     f"x {r['passes']} passes, T={tokens}: act-quant + unpack + int64 product + fp32 epilogue, "
                     f"{r['wall_s']:.1f}s timed",
           "gops": r["GOPS"]}
    out["per_config"] = per_config_baselines()
    out["single_thread"] = single_thread_baselines()
    return out


def per_config_baselines(budget_s=1.0):
    """The oracle on each workload, all host threads: GB/s and GOPS counted
    as the GPU step counts them, the timed wall time and the sample."""
    import workloads
    res = {}
    plan = [("single_ternary", 1, None, None, "the whole [768, 192] projection, 256 tokens"),
            ("decode_stack", 6, None, None, "all 31 matrices, 1 token each"),
            ("binary_gqa", 1, None, 1024, "layer 0 (7 products), 1024 of the 8192 tokens"),
            ("ternary_4b", 1, 1, None, "layer-equivalent 0 (7 matrices) of 36, 1 token"),
            ("ternary_4b", 1, 4, None, "layer-equivalent 0 (7 matrices) of 36, 4 tokens"),
            ("ternary_4b", 1, 16, None, "layer-equivalent 0 (7 matrices) of 36, 16 tokens"),
            ("int4_t4nt", 1, None, 256, "layer 0 (5 products) of 20, 256 of the 4096 tokens")]
    for name, layers, tokens, rows, what in plan:
        wl = workloads.BY_NAME[name]
        t = tokens if tokens is not None else wl.tokens[0]
        items = _oracle_items(wl, layers, t, rows)
        r = _oracle_rate(wl, items, budget_s)
        r["sample"] = what
        res[name if tokens is None else f"{name}_t{tokens}"] = r
    log(f"[bench] cpu oracle per config: {res}")
    return res


def single_thread_baselines(min_s=1.0):
    """The oracle on one host thread, the comparable of a single-thread CPU
    engine: the single ternary projection (768 x 192, 256 tokens), one pass
    of the 256-d decode stack at t = 1 (31 products, each input quantised),
    and decode steps of the 256-d model (binary64 float steps, exact
    products); each repeated for at least min_s seconds."""
    import oracle
    import workloads
    from oracle import model as om
    n_before = oracle.num_threads()
    oracle.set_threads(1)
    try:
        def timed(fn):
            n, t0 = 0, time.perf_counter()
            while True:
                fn()
                n += 1
                dt = time.perf_counter() - t0
                if dt >= min_s:
                    return dt / n
        res = {}
        wl0 = workloads.BY_NAME["single_ternary"]
        m0 = wl0.matrices[0]
        pk0, sc0, _, _ = oracle.quantize_and_pack(workloads.latent_weights(wl0.index, 0, 0, m0.n, m0.k), "ternary",
                                                  "tensor")
        x0 = workloads.workload_activations(wl0, 0, 0, wl0.tokens[0], m0.k)

        def call0():
            q, sx, _ = oracle.act_quant(x0)
            oracle.linear(pk0, sc0, "ternary", "tensor", 0, m0.n, m0.k, q, sx)
        res["single_ternary_ms_per_call"] = round(timed(call0) * 1e3, 3)
        wl1 = workloads.BY_NAME["decode_stack"]
        mats = []
        for layer in range(wl1.layers):
            for mi, m in enumerate(wl1.matrices):
                if layer < m.count:
                    pk, sc, _, _ = oracle.quantize_and_pack(workloads.latent_weights(wl1.index, layer, mi, m.n, m.k),
                                                            "ternary", "tensor")
                    mats.append((m, pk, sc, workloads.workload_activations(wl1, layer, mi, 1, m.k)))

        def pass1():
            for m, pk, sc, x in mats:
                q, sx, _ = oracle.act_quant(x)
                oracle.linear(pk, sc, "ternary", "tensor", 0, m.n, m.k, q, sx)
        res["decode_stack_ms_per_pass"] = round(timed(pass1) * 1e3, 3)
        cfg = workloads.DECODE_MODEL
        d, L, H, ff, V, C = (cfg[k] for k in ("d", "layers", "heads", "d_ff", "vocab", "context"))
        order = {0: 0, 1: 1, 2: 3, 3: 2, 4: 4}
        shapes = [(3 * d, d), (d, d), (ff, d), (ff, d), (d, ff)]
        packed, scales = [], []
        for layer in range(L):
            for slot in range(5):
                n, k = shapes[slot]
                pk, sc, _, _ = oracle.quantize_and_pack(
                    workloads.latent_weights(wl1.index, layer, order[slot], n, k), "ternary", "tensor")
                packed.append(pk)
                scales.append(sc)
        pk, sc, _, _ = oracle.quantize_and_pack(workloads.latent_weights(wl1.index, 0, 5, V, d), "ternary", "tensor")
        packed.append(pk)
        scales.append(sc)
        model = om.Model(d, L, H, ff, V, C, workloads.decode_model_embedding(V, d),
                         workloads.decode_model_norms(L, d), packed, scales)
        kc, vc = np.zeros((L, C, d)), np.zeros((L, C, d))
        state = {"tok": int(workloads.decode_model_tokens(1, V, seed=3)[0]), "pos": 0}

        def step():
            if state["pos"] >= C:
                state["pos"] = 0
            _, state["tok"], _ = om.decode_step(model, state["tok"], state["pos"], kc, vc)
            state["pos"] += 1
        res["decode_model_tokens_per_s"] = round(1.0 / timed(step), 1)
        res["threads"] = 1
        return res
    finally:
        oracle.set_threads(n_before)


# ------------------------------------------------------------------- main

def build_decode_model(lb):
    """The 256-d ternary decoder (quick-start shape of the add/sub-only engine,
    the decode stack's projections) from the seeded latent weights, packed by
    the library: (DecodeModel, config)."""
    import torch
    import workloads
    cfg = workloads.DECODE_MODEL
    d, L, H, ff, V, C = (cfg[k] for k in ("d", "layers", "heads", "d_ff", "vocab", "context"))
    shapes = [(3 * d, d), (d, d), (ff, d), (ff, d), (d, ff), (V, d)]
    descs = [lb.lowbit_describe(lb.TERNARY2, lb.SCALE_TENSOR, n, k) for n, k in shapes]
    mi = {0: 0, 1: 1, 2: 3, 3: 2, 4: 4, 5: 5}                 # decode_stack matrix of each slot
    wl = workloads.BY_NAME["decode_stack"]
    packed, scales = [], []
    for layer in range(L + 1):
        for slot in (range(5) if layer < L else [5]):
            n, k = shapes[slot]
            w = workloads.latent_weights(wl.index, layer if slot < 5 else 0, mi[slot], n, k)
            pk = np.empty(descs[slot].packed_bytes, np.uint8)
            sc = np.empty(descs[slot].n_scales, np.float32)
            lb.lowbit_pack(descs[slot], w, pk, sc)
            packed.append(torch.from_numpy(pk).cuda())
            scales.append(torch.from_numpy(sc).cuda())
    embed = torch.from_numpy(workloads.decode_model_embedding(V, d)).cuda()
    norms = torch.from_numpy(workloads.decode_model_norms(L, d)).cuda()
    return lb.DecodeModel(d, L, H, ff, V, C, descs, embed, norms, packed, scales), cfg


def layers_profile(args):
    """The dependency-respecting decode schedules alone, for profiler runs:
    the 4B-class ternary pass at one token layer by layer through the fused
    entry (layer_fused) and as act-quant + product per call (layer_dep),
    graph replays, then the 256-d decoder's greedy steps (decode_model_view)."""
    import workloads
    wl = workloads.BY_NAME["ternary_4b"]
    p = Pass(wl, 1, "gemv", layers=args.layers)
    p.build_schedules()
    for sched, calls in (("layer_fused", p.layer_fused_calls), ("layer_dep", p.layer_calls)):
        fn = (lambda sc=sched: p.step(sc))
        run = capture(fn) or fn
        el, _ = time_steps(run, args.steps, args.warmup)
        st = el / args.steps
        log(f"[bench] gemv {sched}: {p.step_bytes / st / 1e9:.1f} GB/s, {st * 1e3:.3f} ms/step, "
            f"{p.launches(calls)} launches")
    dm = decode_model_view()
    log(f"[bench] decode model: {dm.get('graph')} (graph), {dm.get('eager')} (eager)")


def decode_model_view():
    """Greedy generation with the 256-d ternary decoder at batch 1: one step
    captured in a HIP graph and replayed across the whole 128-token context
    (each replay reads the token and position the previous one left on the
    device), timed with events; the eager step beside it."""
    import torch
    import workloads
    lb = __import__("bit_weight_linear_bitlinear_amd")
    gm, cfg = build_decode_model(lb)
    V, C = cfg["vocab"], cfg["context"]
    start = int(workloads.decode_model_tokens(1, V, seed=3)[0])
    st = torch.tensor([start, 0, 0, 0], dtype=torch.int32, device="cuda")
    logits = torch.empty(V, device="cuda")
    toks = torch.zeros(C, dtype=torch.int32, device="cuda")

    def reset():
        st.copy_(torch.tensor([start, 0, 0, 0], dtype=torch.int32))
        gm.k_cache.zero_()
        gm.v_cache.zero_()

    step = lambda: gm.step(st, logits, tokens=toks)
    run = capture(step)
    steps = C - 1
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    res = {}
    for name, fn in (("graph", run), ("eager", step)):
        if fn is None:
            continue
        for rep in range(2):                                 # the second pass is timed
            reset()
            torch.cuda.synchronize()
            e0.record()
            for _ in range(steps):
                fn()
            e1.record()
            torch.cuda.synchronize()
        dt = e0.elapsed_time(e1) / 1e3
        res[name] = {"tokens_per_s": round(steps / dt, 1), "us_per_token": round(dt / steps * 1e6, 2)}
    s = st.cpu().tolist()
    L = cfg["layers"]
    out = {"what": "greedy decode, batch 1, of the 256-d 6-layer ternary decoder (4 heads, 4096 vocabulary, "
                   "128-token context; RMSNorm, rotary attention over an fp32 KV cache, SwiGLU, ternary head), "
                   f"{steps} tokens per timed run from position 0; 3 + 5 * {L} launches per token (residual adds, "
                   f"norms and SwiGLU inside the products' quantiser prologues)",
           "launches_per_token": 3 + 5 * L, "final_state": s, **res,
           "context_not_target": "the engine's README quotes ~170-185 tokens/s for this configuration on one "
                                 "Apple M-series CPU thread without a KV cache"}
    log(f"[bench] decode model: {res}")
    return out


def h4_launches(lb, shapes, reps, graph=True):
    """Average duration of one lowbit_act_quant_h4 launch per [t, k] (and of
    the int8 quantiser on the same input beside it): `reps` launches back to
    back, captured in a HIP graph (so that host-side call overhead does not
    stand in for short kernels) and replayed three times between events on
    the replaying stream: {(t, k): (h4_s, int8_s)}."""
    import torch
    out = {}
    g = torch.Generator(device="cuda").manual_seed(7)
    for t, k in shapes:
        x = torch.randn((t, k), device="cuda", generator=g)
        q = torch.empty((t, k), dtype=torch.int8, device="cuda")
        sx = torch.empty(t, device="cuda")
        res = []
        for fn in (lb.lowbit_act_quant_h4, lb.lowbit_act_quant):
            body = (lambda fn=fn: [fn(x, q, sx) for _ in range(reps)])
            run = (capture(body) if graph else None) or body
            el, _ = time_steps(run, 3, 1)
            res.append(el / (3 * reps))
        out[(t, k)] = tuple(res)
        del x, q, sx
    return out


def h_bitlinear_view():
    """H-BitLinear ("Native Binary and Ternary Transformers", 0x07C): the
    rotated 4-bit quantiser on its own (per launch, against the HBM roofline:
    4 bytes read and 1 written per element, 4 per row), and the int4 4-bit
    QAT model's attention-output and FFN-down products at 4096 tokens with
    that quantiser in place of the int8 one (the rotation's overhead on a
    layer)."""
    import torch
    import workloads
    lb = __import__("bit_weight_linear_bitlinear_amd")
    shapes = [(4096, 1280), (4096, 3584), (1, 2560), (1, 9728), (16, 9728)]
    times = h4_launches(lb, shapes, reps=50)
    per = {}
    for (t, k), (th, t8) in times.items():
        nb = 5 * t * k + 4 * t
        per[f"t{t}_k{k}"] = {"us": round(th * 1e6, 2), "GBps": round(nb / th / 1e9, 1),
                             "frac_hbm_peak": round(nb / th / 1e9 / HBM_PEAK_GBS, 4),
                             "int8_quantiser_us": round(t8 * 1e6, 2), "block": int(k & -k if (k & -k) <= 2048 else 2048)}
    # the o and down products of layer 0 of the int4 prefill workload
    wl = workloads.BY_NAME["int4_t4nt"]
    T = wl.tokens[0]
    layer = {}
    for mi in (1, 4):
        m = wl.matrices[mi]
        d = lb.lowbit_describe(lb.FORMATS[wl.fmt], lb.SCALES[wl.scale], m.n, m.k, wl.group,
                               lb.FLAG_TANH3 if wl.tanh_premap else 0)
        pk = np.empty(d.packed_bytes, np.uint8)
        sc = np.empty(d.n_scales, np.float32)
        lb.lowbit_pack(d, workloads.latent_weights(wl.index, 0, mi, m.n, m.k), pk, sc)
        pk, sc = torch.from_numpy(pk).cuda(), torch.from_numpy(sc).cuda()
        x = torch.from_numpy(workloads.workload_activations(wl, 0, mi, T, m.k)).cuda()
        q = torch.empty((T, m.k), dtype=torch.int8, device="cuda")
        sx = torch.empty(T, device="cuda")
        y = torch.empty((T, m.n), device="cuda")
        res = {}
        for name, quant in (("bitlinear_int8", lb.lowbit_act_quant), ("h_bitlinear_int4", lb.lowbit_act_quant_h4)):
            def fn(quant=quant):
                quant(x, q, sx)
                lb.lowbit_linear_batched(d, pk, sc, q, sx, y)
            run = capture(fn) or fn
            el, _ = time_steps(run, 20, 3)
            res[name] = round(el / 20 * 1e6, 2)
        res["overhead_pct"] = round(100 * (res["h_bitlinear_int4"] / res["bitlinear_int8"] - 1), 2)
        layer[f"{m.name}_[{m.n},{m.k}]"] = res
    out = {"what": "H-BitLinear's rotated INT4 activation quantiser (block Walsh-Hadamard over B = largest "
                   "power of two dividing k, at most 2048; per-token absmax codes in [-7, 7]); per launch vs "
                   "the HBM roofline (5 B per element + 4 B per row), and the int4 model's o / down layers "
                   "at 4096 tokens (quantiser + GEMM, us per layer) with it in place of the int8 quantiser",
           "kernel": "act_quant_h4_kernel", "per_launch": per, "layers_t4096": layer}
    log(f"[bench] h-bitlinear: {per}; layers {layer}")
    return out


def bitnet_v1_view():
    """The original BitNet forward ("Native Binary and Ternary Transformers",
    0x02B-0x02E) on the binary d = 192 model's shapes at 8192 tokens: the
    sub-layer LayerNorm (8 bytes per element), the Q_b = 128 quantiser per
    token and per tensor beside the int8 one (5 bytes per element), each
    launch run 20 times in a captured HIP graph; and the FFN up projection
    [768, 192] with centered binary weights as LayerNorm + quantiser + GEMM
    against the int8 quantiser + GEMM."""
    import torch
    import workloads
    lb = __import__("bit_weight_linear_bitlinear_amd")
    wl = workloads.BY_NAME["binary_gqa"]
    T = wl.tokens[0]
    reps = 20
    out = {"what": " ".join(bitnet_v1_view.__doc__.split()), "tokens": T}
    g = torch.Generator(device="cuda").manual_seed(5)
    work = torch.zeros(2, dtype=torch.int32, device="cuda")

    def timed(fn):
        body = (lambda: [fn() for _ in range(reps)])
        el, _ = time_steps(capture(body) or body, 3, 1)
        return el / (3 * reps)
    for k in (192, 768):
        x = torch.randn((T, k), device="cuda", generator=g)
        xn = torch.empty_like(x)
        q = torch.empty((T, k), dtype=torch.int8, device="cuda")
        sx = torch.empty(T, device="cuda")
        res = {"layernorm": timed(lambda: lb.lowbit_layernorm(x, xn)),
               "v1_per_token": timed(lambda: lb.lowbit_act_quant_v1(x, q, sx)),
               "v1_per_tensor": timed(lambda: lb.lowbit_act_quant_v1(x, q, sx, per_tensor=True, work=work)),
               "int8_absmax": timed(lambda: lb.lowbit_act_quant(x, q, sx))}
        byt = {"layernorm": 8 * T * k}
        out[f"k{k}"] = {n: {"us": round(v * 1e6, 2),
                            "GBps": round(byt.get(n, 5 * T * k + 4 * T) / v / 1e9, 1)} for n, v in res.items()}
        del x, xn, q, sx
    m = wl.matrices[4]                                       # up [768, 192]
    w = workloads.latent_weights(wl.index, 0, 4, m.n, m.k)
    x = torch.from_numpy(workloads.workload_activations(wl, 0, 4, T, m.k)).cuda()
    xn = torch.empty_like(x)
    q = torch.empty((T, m.k), dtype=torch.int8, device="cuda")
    sx = torch.empty(T, device="cuda")
    y = torch.empty((T, m.n), device="cuda")
    layer = {}
    for name, flags in (("v1_centered", lb.FLAG_CENTERED), ("b1_sign", 0)):
        d = lb.lowbit_describe(lb.BINARY1, lb.SCALE_ROW, m.n, m.k, 0, flags)
        pk = np.empty(d.packed_bytes, np.uint8)
        sc = np.empty(d.n_scales, np.float32)
        lb.lowbit_pack(d, w, pk, sc)
        pk, sc = torch.from_numpy(pk).cuda(), torch.from_numpy(sc).cuda()
        if flags:
            def fwd(d=d, pk=pk, sc=sc):
                lb.lowbit_layernorm(x, xn)
                lb.lowbit_act_quant_v1(xn, q, sx)
                lb.lowbit_linear_batched(d, pk, sc, q, sx, y)
        else:
            def fwd(d=d, pk=pk, sc=sc):
                lb.lowbit_act_quant(x, q, sx)
                lb.lowbit_linear_batched(d, pk, sc, q, sx, y)
        layer[name] = round(timed(fwd) * 1e6, 2)
    out["up_projection_t8192_us"] = {"layernorm_v1_quant_gemm": layer["v1_centered"],
                                     "int8_quant_gemm": layer["b1_sign"]}
    log(f"[bench] bitnet v1: {out}")
    return out


def onebit_view():
    """OneBit's W1A16 projection ("Native Binary and Ternary Transformers",
    0x06A): h * (fp16(x * g) . S^T) with 1-bit signs, at the section's
    N = K = 4096 and the 4B-class shapes; t = 1 against the HBM roofline
    (n k / 8 bytes of signs + fp16 x, g, h + fp32 y per call), t = 4096
    against the dense fp16 matrix-core peak.  Launch runs captured in a HIP
    graph; the LayerNorm after it is the bitnet_v1 view's kernel."""
    import torch
    lb = __import__("bit_weight_linear_bitlinear_amd")
    g = torch.Generator(device="cuda").manual_seed(9)
    rows = []
    for n, k, t in ((4096, 4096, 1), (9728, 2560, 1), (2560, 9728, 1), (4096, 4096, 16), (4096, 4096, 4096)):
        d = lb.lowbit_describe(lb.BINARY1, lb.SCALE_ROW, n, k, 0, 0)
        packed = torch.randint(0, 256, (d.packed_bytes,), dtype=torch.uint8, device="cuda", generator=g)
        x = torch.randn((t, k), device="cuda", generator=g).half()
        gv = (1 + 0.1 * torch.randn(k, device="cuda", generator=g)).half()
        hv = (0.02 * torch.rand(n, device="cuda", generator=g)).half()
        y = torch.empty((t, n), device="cuda")
        reps = 20 if t < 4096 else 5
        body = (lambda d=d, packed=packed, x=x, gv=gv, hv=hv, y=y:
                [lb.lowbit_onebit_linear(d, packed, gv, hv, x, y) for _ in range(reps)])
        el, _ = time_steps(capture(body) or body, 3, 1)
        dt = el / (3 * reps)
        nbytes = d.packed_bytes + 2 * t * k + 2 * k + 2 * n + 4 * t * n
        flops = 2 * t * n * k
        rows.append({"n": n, "k": k, "t": t, "us": round(dt * 1e6, 2), "GBps": round(nbytes / dt / 1e9, 1),
                     "frac_hbm_peak": round(nbytes / dt / 1e9 / HBM_PEAK_GBS, 4),
                     "TFLOPS": round(flops / dt / 1e12, 1),
                     "frac_fp16_mfma_peak": round(flops / dt / 1e12 / F16_PEAK_TFLOPS, 4)})
        del packed, x, y
    out = {"what": " ".join(onebit_view.__doc__.split()), "kernel": "onebit_kernel", "shapes": rows}
    log(f"[bench] onebit: {rows}")
    return out


def onebit_profile():
    """OneBit's projection launches only (for profiler runs): the view's
    shapes, each call timed on its own."""
    rows = onebit_view()["shapes"]
    for r in rows:
        print(json.dumps({"onebit": [r["n"], r["k"], r["t"]], "us": r["us"], "TFLOPS": r["TFLOPS"],
                          "GBps": r["GBps"]}), flush=True)


def h4_profile():
    """The rotated quantiser's prefill launches only (for profiler runs)."""
    lb = __import__("bit_weight_linear_bitlinear_amd")
    times = h4_launches(lb, [(4096, 3584), (4096, 1280)], reps=20, graph=False)
    for (t, k), (th, _) in times.items():
        nb = 5 * t * k + 4 * t
        print(json.dumps({"h4_t": t, "k": k, "us": round(th * 1e6, 2), "GBps": round(nb / th / 1e9, 1),
                          "bytes_per_launch": nb}), flush=True)


def a48_launches(lb, shapes, reps, graph=True):
    """Average launch duration of BitNet a4.8's two quantisers per [t, k]:
    the sparse 8-bit one keeping half of each row, the dense int8 one on the
    same input beside it, and the 4-bit one; `reps` launches captured in a
    HIP graph and replayed three times between events on the replaying
    stream: {(t, k): {"sparse8": s, "int8": s, "a4": s}}."""
    import torch
    out = {}
    g = torch.Generator(device="cuda").manual_seed(11)
    for t, k in shapes:
        x = torch.randn((t, k), device="cuda", generator=g)
        q = torch.empty((t, k), dtype=torch.int8, device="cuda")
        sx = torch.empty(t, device="cuda")
        fns = {"sparse8": lambda: lb.lowbit_act_quant_sparse8(x, q, sx, k // 2),
               "int8": lambda: lb.lowbit_act_quant(x, q, sx),
               "a4": lambda: lb.lowbit_act_quant_a4(x, q, sx)}
        res = {}
        for name, fn in fns.items():
            body = (lambda fn=fn: [fn() for _ in range(reps)])
            run = (capture(body) if graph else None) or body
            el, _ = time_steps(run, 3, 1)
            res[name] = el / (3 * reps)
        out[(t, k)] = res
        del x, q, sx
    return out


def a48_view():
    """BitNet a4.8 ("Native Binary and Ternary Transformers", 0x07B) on the
    4B-class ternary model's widths: the sparse 8-bit codes of the states in
    front of the attention output (k = 2560) and FFN down (k = 9728)
    projections, half of each row kept, and the 4-bit input codes, at 4096
    tokens and at one; per launch against the HBM roofline (4 bytes read and
    1 written per element, 4 per row), the dense int8 quantiser beside them."""
    lb = __import__("bit_weight_linear_bitlinear_amd")
    out = {"what": " ".join(a48_view.__doc__.split())}
    for (t, k), res in a48_launches(lb, [(4096, 2560), (4096, 9728), (1, 2560), (1, 9728)], reps=50).items():
        nb = 5 * t * k + 4 * t
        out[f"t{t}_k{k}"] = {name: {"us": round(v * 1e6, 2), "GBps": round(nb / v / 1e9, 1),
                                    "frac_hbm_peak": round(nb / v / 1e9 / HBM_PEAK_GBS, 4)}
                             for name, v in res.items()}
    log(f"[bench] a4.8: {out}")
    return out


def a48_profile():
    """The a4.8 quantisers' prefill launches only (for profiler runs)."""
    lb = __import__("bit_weight_linear_bitlinear_amd")
    for (t, k), res in a48_launches(lb, [(4096, 9728), (4096, 2560)], reps=20, graph=False).items():
        nb = 5 * t * k + 4 * t
        print(json.dumps({"a48_t": t, "k": k, "bytes_per_launch": nb,
                          **{name: {"us": round(v * 1e6, 2), "GBps": round(nb / v / 1e9, 1)}
                             for name, v in res.items()}}), flush=True)


def extra_views(args):
    """The other timing views: (iii) the streaming ceiling on one large cold
    matrix, the cache-resident 256-d decode stack at t = 1, and the binary
    8192-token GEMM pass (output-bound)."""
    import torch
    import workloads
    lb = __import__("bit_weight_linear_bitlinear_amd")
    views = {}

    # (iii) one [524288, 2560] ternary group-128 matrix at t = 1, four copies
    # rotated (4 x 377 MB, six times the 256 MB last-level cache): random
    # valid two-bit fields (00, 01, 11) straight into the packed layout
    n, k = 524288, 2560
    d = lb.lowbit_describe(lb.FORMATS["ternary"], lb.SCALES["group"], n, k, 128, 0)
    rng = np.random.default_rng(123)
    mats = []
    for _ in range(4):
        low = rng.integers(0, 256, size=d.packed_bytes, dtype=np.uint8) & np.uint8(0x55)
        high = (low & rng.integers(0, 256, size=d.packed_bytes, dtype=np.uint8)) << np.uint8(1)
        packed = torch.from_numpy(low | high).cuda()
        scales = torch.from_numpy(rng.random(d.n_scales, dtype=np.float32) + np.float32(0.5)).cuda()
        mats.append((packed, scales))
    q = torch.from_numpy(rng.integers(-127, 128, size=(1, k), dtype=np.int8)).cuda()
    sx = torch.ones(1, device="cuda")
    y = torch.empty((1, n), device="cuda")
    reps = 20
    for i in range(4):
        lb.lowbit_linear(d, *mats[i % 4], q, sx, y)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(reps):
        lb.lowbit_linear(d, *mats[i % 4], q, sx, y)
    e1.record()
    torch.cuda.synchronize()
    dt = e0.elapsed_time(e1) / 1e3 / reps
    nbytes = d.packed_bytes + 4 * d.n_scales + k + 4 + 4 * n
    views["steady_cold_matrix"] = {
        "what": "view (iii): one ternary group-128 [524288, 2560] GEMV at t = 1, four copies rotated "
                "(6x the last-level cache); lowbit_linear launches timed back to back",
        "bytes_per_call": nbytes, "us_per_call": round(dt * 1e6, 2), "GBps": round(nbytes / dt / 1e9, 1),
        "pct_hbm_peak": round(100 * nbytes / dt / 1e9 / HBM_PEAK_GBS, 2)}
    log(f"[bench] steady cold matrix: {nbytes / dt / 1e9:.1f} GB/s, {dt * 1e6:.1f} us/call")
    del mats, packed, scales

    # the 256-d decode stack at t = 1: every matrix cache-resident
    wl1 = workloads.BY_NAME["decode_stack"]
    p1 = Pass(wl1, 1, "gemv")
    run = capture(lambda: p1.step("per_matrix")) or (lambda: p1.step("per_matrix"))
    el, _ = time_steps(run, 50, 5)
    st = el / 50
    dur, bpl, _ = per_launch(p1, reps=20)

    # the same 31 products as a model runs them, each input quantised right
    # before its product: the quantiser kernel + product per call, or the
    # fused entry (one launch per call)
    def dep_separate():
        for i, d in enumerate(p1.desc):
            q, sx = p1.views[i]
            lb.lowbit_act_quant(p1.xv[i], q, sx)
            lb.lowbit_linear(d, p1.packed[i], p1.scales[i], q, sx, p1.y[i])

    def dep_fused():
        for i, d in enumerate(p1.desc):
            q, sx = p1.views[i]
            lb.lowbit_linear_fused(d, p1.packed[i], p1.scales[i], p1.xv[i], q, sx, p1.y[i])
    dep = {}
    for name, fn in (("separate", dep_separate), ("fused", dep_fused)):
        el_d, _ = time_steps(capture(fn) or fn, 50, 5)
        dep[name] = round(el_d / 50 * 1e6, 2)
    views["decode_stack_t1"] = {
        "what": "the 256-d 6-layer ternary decode stack (31 GEMVs + 2 act-quant per step), t = 1; "
                "1.9 MB of weights, cache-resident: launch- and latency-bound, not an HBM figure",
        "us_per_step": round(st * 1e6, 2), "gemv_calls": len(p1.mats), "us_per_gemv_call": round(dur * 1e6, 2),
        "effective_GBps_not_hbm": round(p1.step_bytes / st / 1e9, 1),
        "dependent_us_per_step": {"what": "each input quantised right before its product (31 calls)", **dep}}
    log(f"[bench] decode stack t=1: {st * 1e6:.1f} us/step, {dur * 1e6:.2f} us per GEMV call; "
        f"dependent calls: {dep}")
    del p1

    views["decode_model_t1"] = decode_model_view()
    views["h_bitlinear"] = h_bitlinear_view()
    views["bitnet_v1"] = bitnet_v1_view()
    views["onebit"] = onebit_view()
    views["a48"] = a48_view()

    # the binary 8192-token GEMM pass
    wl2 = workloads.BY_NAME["binary_gqa"]
    p2 = Pass(wl2, wl2.tokens[0], "gemm")
    sched, (dur, bpl, opl) = gemm_pass(p2, 5)
    st = sched["grouped"]
    ops = sum(p2.linear_ops)
    views["binary_gqa_gemm"] = {
        "what": "the binary d=192 8-layer model's 56 products at 8192 tokens, act-quant included, equal-k "
                "products as grouped launches; bound by the fp32 output (HBM), not by the matrix cores",
        "ms_per_step": round(st * 1e3, 4), "TOPS_step": round(ops / st / 1e12, 2),
        "GBps_step": round(p2.step_bytes / st / 1e9, 1),
        "pct_hbm_peak_step": round(100 * p2.step_bytes / st / 1e9 / HBM_PEAK_GBS, 2),
        "ms_per_step_one_launch_per_product": round(sched["per_matrix"] * 1e3, 4),
        "grouped_launches": p2.launches(p2.grouped_calls),
        "GBps_per_grouped_launch": round(bpl / dur / 1e9, 1), "TOPS_per_grouped_launch": round(opl / dur / 1e12, 2)}
    log(f"[bench] binary gqa gemm: {ops / st / 1e12:.1f} TOPS/step, {p2.step_bytes / st / 1e9:.1f} GB/s/step")
    del p2

    # group-scale prefill: the 4B-class ternary layer (group-128 scales) at
    # 4096 tokens on the batched path, which runs group scales on the
    # 128 x 128 tile only
    wl3 = workloads.BY_NAME["ternary_4b"]
    p3 = Pass(wl3, 4096, "gemm", layers=1)
    sched, (dur, bpl, opl) = gemm_pass(p3, 3)
    st = sched["grouped"]
    ops = sum(p3.linear_ops)
    views["group_prefill"] = {
        "what": "the 4B-class ternary layer-equivalent (7 group-128 products: 4 x [2560, 2560], [9728, 2560] x 2, "
                "[2560, 9728]) at 4096 tokens on the batched path (group scales run the 128 x 128 tile), "
                "act-quant included, equal-k products as grouped launches",
        "ms_per_step": round(st * 1e3, 4), "TOPS_step": round(ops / st / 1e12, 2),
        "grouped_launches": p3.launches(p3.grouped_calls),
        "TOPS_per_grouped_launch": round(opl / dur / 1e12, 2),
        "pct_mfma_peak_per_grouped_launch": round(100 * opl / dur / 1e12 / I8_PEAK_TOPS, 2)}
    log(f"[bench] group prefill: {views['group_prefill']}")
    del p3
    return views


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--tokens", type=int, default=1)
    ap.add_argument("--layers", type=int, default=None, help="fewer layer-equivalents (debug only)")
    ap.add_argument("--skip-gemm", action="store_true")
    ap.add_argument("--skip-cpu", action="store_true")
    ap.add_argument("--skip-check", action="store_true")
    ap.add_argument("--skip-views", action="store_true", help="skip the steady-state, decode-stack and binary views")
    ap.add_argument("--no-graph", action="store_true")
    ap.add_argument("--quick", action="store_true", help="grouped schedule only")
    ap.add_argument("--profile-gemm", action="store_true",
                    help="batched GEMM pass only, with per-shape launch timings (for profiler runs)")
    ap.add_argument("--profile-h4", action="store_true",
                    help="the rotated 4-bit quantiser's prefill launches only (for profiler runs)")
    ap.add_argument("--profile-a48", action="store_true",
                    help="the a4.8 quantisers' prefill launches only (for profiler runs)")
    ap.add_argument("--profile-onebit", action="store_true",
                    help="OneBit's projection launches only (for profiler runs)")
    ap.add_argument("--profile-layers", action="store_true",
                    help="the layer-by-layer decode schedules and the 256-d decoder only (for profiler runs)")
    ap.add_argument("--profile-pass", action="store_true",
                    help="copy calibration + grouped GEMV pass only (for profiler runs)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (run with --gpus 1)",
              file=sys.stderr, flush=True)
        sys.exit(2)

    import torch
    import workloads
    torch.cuda.set_device(0)
    out = {"metric": METRIC}
    if args.profile_pass:
        args.quick = args.skip_gemm = args.skip_cpu = args.skip_check = args.skip_views = True
    calib = copy_calibration()
    log(f"[bench] copy calibration: {calib}")
    ceilings = (None if args.profile_pass or args.profile_gemm or args.profile_h4 or args.profile_a48 or
                args.profile_onebit or args.profile_layers else calibration())
    if ceilings:
        log(f"[bench] device ceilings: {ceilings}")

    if args.profile_gemm:
        gemm_profile(args)
        return
    if args.profile_onebit:
        onebit_profile()
        return
    if args.profile_h4:
        h4_profile()
        return
    if args.profile_a48:
        a48_profile()
        return
    if args.profile_layers:
        layers_profile(args)
        return

    # ---- GEMV line: ternary_4b decode pass
    wl = workloads.BY_NAME["ternary_4b"]
    p = Pass(wl, args.tokens, "gemv", layers=args.layers)
    p.build_schedules()
    schedules = {}
    # untimed: about half a second of the headline step first, so that the
    # first schedule timed does not meet the device still at idle clocks
    # (skipped in the short profiler runs, where it would only add dispatches)
    warm = capture(lambda: p.step("grouped")) or (lambda: p.step("grouped"))
    t_end = time.perf_counter() + (0.0 if args.profile_pass else 0.5)
    while time.perf_counter() < t_end:
        for _ in range(20):
            warm()
        torch.cuda.synchronize()
    order = (["grouped"] if args.quick else
             ["grouped", "grouped_fused", "layer", "layer_dep", "layer_fused", "per_matrix"])
    head_steps = []
    for sched in order:
        fn = (lambda sc=sched: p.step(sc))
        run = None if args.no_graph else capture(fn)
        elapsed, wall = time_steps(run or fn, args.steps, args.warmup,
                                   per_step=head_steps if sched == "grouped" else None)
        st = elapsed / args.steps
        n_l = {"grouped": p.launches(p.grouped_calls), "grouped_fused": p.launches(p.fused_calls),
               "layer": p.launches(p.layer_calls), "layer_dep": p.launches(p.layer_calls),
               "layer_fused": p.launches(p.layer_fused_calls), "per_matrix": len(p.mats)}[sched]
        n_aq = {"grouped_fused": 0, "layer_fused": 0, "layer_dep": len(p.layer_calls)}.get(sched, len(p.kgroups))
        schedules[sched] = {"GBps": round(p.step_bytes / st / 1e9, 2), "ms_per_step": round(st * 1e3, 4),
                            "gemv_launches": n_l, "act_quant_launches": n_aq,
                            "graph": run is not None, "wall_s": round(wall, 3)}
        log(f"[bench] gemv {sched}: {p.step_bytes / st / 1e9:.1f} GB/s, {st * 1e3:.3f} ms/step, {n_l} launches")
    head = schedules["grouped"]
    step_s = head["ms_per_step"] / 1e3
    value = p.step_bytes / step_s / 1e9
    dur, bytes_per_launch = per_launch_grouped(p, p.grouped_calls, reps=10, fused=False)
    achieved = bytes_per_launch / dur / 1e9
    if not args.quick:
        dur_f, bytes_f = per_launch_grouped(p, p.fused_calls, reps=10, fused=True)
        schedules["grouped_fused"]["per_launch"] = {"avg_launch_us": round(dur_f * 1e6, 3),
                                                    "GBps": round(bytes_f / dur_f / 1e9, 2)}
    check = None if args.skip_check else sampled_check(p, [0, 4, 6, len(p.mats) - 1])
    # the same pass at 4 and 16 tokens per call (the same packed weights)
    tok_lines = {}
    if not args.quick:
        for tt in (4, 16):
            if tt == args.tokens:
                continue
            pt = Pass(wl, tt, "gemv", layers=args.layers, weights_from=p)
            pt.build_schedules()
            fn = lambda: pt.step("grouped")
            run = (None if args.no_graph else capture(fn)) or fn
            per = []
            el, _ = time_steps(run, args.steps, args.warmup, per_step=per)
            st_t = el / args.steps
            d_t, b_t = per_launch_grouped(pt, pt.grouped_calls, reps=10, fused=False)
            ach_t = b_t / d_t / 1e9
            tok_lines[f"t{tt}"] = {
                "tokens": tt, "ms_per_step": round(st_t * 1e3, 4), "GBps_step": round(pt.step_bytes / st_t / 1e9, 2),
                "pct_hbm_peak_step": round(100 * pt.step_bytes / st_t / 1e9 / HBM_PEAK_GBS, 2),
                "step": step_stats(per), "launches": pt.launches(pt.grouped_calls),
                "per_launch": {"avg_us": round(d_t * 1e6, 3), "bytes": round(b_t), "GBps": round(ach_t, 2),
                               "frac_hbm_peak": round(ach_t / HBM_PEAK_GBS, 4),
                               "frac_of_measured_read": (round(ach_t / ceilings["read_stream_GBps"], 4)
                                                         if ceilings else None)}}
            log(f"[bench] gemv t={tt}: {tok_lines[f't{tt}']}")
            del pt

    out.update({
        "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(step_s * 1e3, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "int8", "data": "synthetic",
        "config": {"workload": f"ternary_4b decode pass: {len(p.mats)} ternary group-128 GEMVs "
                               f"(K=2560/9728, N=2560/9728), T={args.tokens}, from fp32 inputs: per-token "
                               f"act-quant of every input included (one launch per k); equal-k products "
                               f"issued as grouped launches",
                   "tokens": args.tokens, "matrices": len(p.mats), "bytes_per_step": p.step_bytes,
                   "pct_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2), "schedules": schedules},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": committed_traffic(),
                     "kernel": "gemv_kernel (grouped schedule)", "avg_launch_us": round(dur * 1e6, 3),
                     "bytes_per_launch": round(bytes_per_launch),
                     "measured_peak": ceilings["read_stream_GBps"] if ceilings else None,
                     "frac_of_measured": round(achieved / ceilings["read_stream_GBps"], 4) if ceilings else None},
        "step": step_stats(head_steps) if head_steps else None,
        "gemv_tokens": tok_lines,
    })
    out["device_ceilings"] = ceilings
    out["copy_calibration"] = calib
    if check:
        out["check"] = check
    log(f"[bench] gemv grouped per launch {dur * 1e6:.2f} us -> {achieved:.1f} GB/s")

    # ---- batched GEMM figure: int4_t4nt prefill pass
    if not args.skip_gemm:
        wl4 = workloads.BY_NAME["int4_t4nt"]
        p4 = Pass(wl4, wl4.tokens[0], "gemm")
        sched4, (dg, _, opg) = gemm_pass(p4, max(3, args.steps // 4), args.no_graph)
        st4 = min(sched4.values())
        ops4 = sum(p4.linear_ops)
        d1, _, ops_single = per_launch(p4, reps=3)             # each product as its own launch
        d4, ops_per_launch = dg, opg                           # the launches the pass runs (grouped)
        tops_launch = ops_per_launch / d4 / 1e12
        chk4 = None if args.skip_check else sampled_check(p4, [0, 1, 4], rows_per=32)
        shapes4 = gemm_shapes_vs_library(p4)
        # the second roofline of a prefill product: its HBM bytes (fp32 y
        # dominates) at peak bandwidth; the larger of the two floors bounds it
        bytes4 = sum(p4.linear_bytes)
        floor_mfma = ops4 / (I8_PEAK_TOPS * 1e12)
        floor_hbm = bytes4 / (HBM_PEAK_GBS * 1e9)
        n4 = p4.launches(p4.grouped_calls)
        out["gemm"] = {"workload": "int4_t4nt prefill pass: 100 int4 row-scale GEMMs, T=4096, act-quant included; "
                                   "equal-k products as grouped launches (at most 64 per launch, of near-equal size)",
                       "tops_step": round(ops4 / st4 / 1e12, 2), "ms_per_step": round(st4 * 1e3, 4),
                       "step": step_stats(p4.grouped_step_times),
                       "schedules_ms_per_step": {k: round(v * 1e3, 4) for k, v in sched4.items()},
                       "single_product_launch": {"avg_us": round(d1 * 1e6, 2),
                                                 "TOPS": round(ops_single / d1 / 1e12, 2)},
                       "tops_per_launch": round(tops_launch, 2),
                       "pct_mfma_peak": round(100 * tops_launch / I8_PEAK_TOPS, 2),
                       "avg_launch_us": round(d4 * 1e6, 2), "launches": n4,
                       "kernel": "gemm_mfma_kernel (grouped launches)",
                       "roofline": {"bound": "mfma", "achieved": round(tops_launch, 2), "peak": I8_PEAK_TOPS,
                                    "unit": "TOPS", "frac": round(tops_launch / I8_PEAK_TOPS, 4),
                                    "measured_peak": ceilings["mfma_i8_TOPS"] if ceilings else None,
                                    "frac_of_measured": (round(tops_launch / ceilings["mfma_i8_TOPS"], 4)
                                                         if ceilings else None),
                                    "mfma_floor_us_per_launch": round(floor_mfma / n4 * 1e6, 2),
                                    "hbm_floor_us_per_launch": round(floor_hbm / n4 * 1e6, 2),
                                    "frac_of_larger_floor": round(max(floor_mfma, floor_hbm) / n4 / d4, 4)},
                       "shapes_vs_library_int8": {
                           "what": "each distinct shape as its own launch (graph-captured runs), beside the ROCm "
                                   "library's plain int8 GEMM (torch._int_mm: unpacked int8 weights, int32 output, "
                                   "no scales) on the same t, n, k",
                           "shapes": shapes4},
                       "check": chk4}
        log(f"[bench] gemm pass: {ops4 / st4 / 1e12:.1f} TOPS/step; per launch {tops_launch:.1f} TOPS")
        del p4

    if not args.skip_views and not args.quick:
        out["views"] = extra_views(args)

    if not args.skip_cpu:
        out["cpu_baseline"] = cpu_baseline(wl, args.tokens)
        log(f"[bench] cpu oracle: {out['cpu_baseline']}")
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
