#!/usr/bin/env python3
"""Benchmark of the SSD scan on one MI355X.

The headline step is one ssd_chunk_scan over the grouped long-context
workload (batch 1, seqlen 65536, 64 heads of head_dim 64, state 128,
8 groups, chunk 256, bf16 io, fp32 state), the largest single-GPU scan
workload; inputs resident in HBM, several independently drawn input sets
cycled through so that the working set exceeds the 256 MB Infinity Cache.
Every other workload is timed the same way and reported beside it (tiny
fp32, the Mamba2-130m and 2.7B shapes, the decode workload's 256 x 1024
prefill), plus 128 decode steps at batch 256.

Kernel durations come from HIP events that the library records at each
kernel's own dispatch (ssd_chunk_scan_ex's kernel_events), over the timed
steps themselves.  Algorithmic bytes per launch follow the method: every
operand of the kernel's step moved once, in the type the kernel stores it.

Printed: one JSON line.

    python bench.py [--steps K] [--warmup W] [--gpus 1]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "SSD scan tokens/sec at 1 GPU; % of MFMA/HBM roofline; decode steps/sec"
HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published
SLOTS = ("chunk_state", "state_scan", "chunk_out")
HEADLINE = "grouped_long"
SCAN_WORKLOADS = ("tiny_fp32", "mamba2_130m", "mamba2_2p7b", "grouped_long", "decode_2p7b")
PROFILES = os.path.join(ROOT, "profiles")
_CSRC = "mamba_ssd_chunked_chunk_amd/csrc/"
# the sources of each profiled kernel (its counter summaries are retired
# when they change)
KERNEL_SOURCES = {
    "scan": tuple(_CSRC + f for f in ("ssd_scan16.hpp", "ssd_device.hpp", "ssd_plan.hpp")),
    "k_step": tuple(_CSRC + f for f in ("ssd_step.hpp", "ssd_device.hpp", "ssd_plan.hpp")),
    "neighbors": tuple(_CSRC + f for f in ("ssd_neighbors.hip", "ssd_mixer.hip",
                                           "ssd_device.hpp")),
}


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def source_digest(kernel: str = "scan") -> str:
    """Digest of a kernel's code (the bf16 scan kernels: "scan"): comments
    and blank lines do not count, so a comment edit does not retire the
    counter summaries."""
    import re
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[kernel if kernel in KERNEL_SOURCES else "scan"]:
        with open(os.path.join(ROOT, rel)) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        lines = [ln.rstrip() for ln in text.split("\n") if ln.strip()]
        h.update("\n".join(lines).encode())
    return h.hexdigest()[:16]


# ----------------------------------------------------------- byte counts ---
def bytes_scan_alg(b, l, h, p, n, g, Q, s, init=False, final=False):
    """Algorithmic bytes of the whole scan: inputs and outputs once plus one
    write and one read of the fp32 chunk-boundary-state tensor."""
    th = b * l * h
    per = 2 * p * s + 2 * n * s * g / h + s + 8.0 * n * p / Q
    return th * per + 4 * n * p * b * h * (int(init) + int(final))


def bytes_scan_min(b, l, h, p, n, g, Q, s, init=False, final=False):
    """The same without the boundary-state tensor: inputs and outputs once."""
    th = b * l * h
    return th * (2 * p * s + 2 * n * s * g / h + s) + 4 * n * p * b * h * (int(init) + int(final))


def bytes_kernel(name, b, l, h, p, n, g, Q, s, init=False, final=False, nst=None):
    """Algorithmic bytes of one launch: every operand of the kernel's step
    moved once, in the type the kernel keeps it.  bf16 io: chunk states and
    boundary states are fp16 (with one fp32 scale or maximum per (batch,
    chunk, head)); fp32 io: fp32.  B and C count once per group.  nst: the
    chunks per sequence whose states the call stores (the library's
    ssd_chunk_scan_state_chunks; default ceil(l / Q))."""
    nc = -(-l // Q) if nst is None else nst
    th = b * l * h
    x = th * p * s                      # x (or y)
    BC = b * l * g * n * s              # B or C
    dt = th * s
    es = 2 if s == 2 else 4             # stored state element
    ns = nc if final else nc - 1        # chunk states needed
    sn = b * ns * h * n * p * es + b * ns * h * 8
    sb = b * (nc if init else nc - 1) * h * (n * p * es + 4)   # boundary states stored
    io_state = b * h * n * p * 4
    if name == "chunk_state":
        # x, B and dt read; the chunk states, their maxima and log decays written
        rows = 0 if s == 2 else 3 * b * h * nc * (-(-Q // 32) * 32) * 4
        return x + BC + dt + sn + rows
    if name == "state_scan":
        return sn + sb + io_state * (int(init) + int(final))
    if name == "chunk_out":
        # x, B, C, dt and the boundary states read, y written
        rows = 0 if s == 2 else 3 * b * h * nc * (-(-Q // 32) * 32) * 4
        return 2 * x + 2 * BC + dt + sb + rows
    raise KeyError(name)


def bytes_step(b, h, p, n, g, s):
    return b * h * (8 * n * p + 2 * p * s + s) + 2 * b * g * n * s + 12 * h


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None when there is none or the kernel sources changed since."""
    path = os.path.join(PROFILES, "%s_%s_traffic.txt" % (kernel, workload))
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    try:
        if kv.get("source_digest") != source_digest(kernel):
            return None
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


# ----------------------------------------------------------------- inputs --
def device_inputs(torch, w, dev, seed):
    """One input set of workload w drawn on the device with the workloads'
    distributions (A = -exp(U[0, ln 16]), dt_bias = softplus^-1 of a
    log-uniform step in [1e-3, 0.1], x, dt, B, C ~ N(0, 1) rounded to the io
    dtype, D = 1, initial state N(0, init_std^2) where the workload has one)."""
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed)
    b, l, h, p, n, g = w.batch, w.seqlen, w.heads, w.head_dim, w.state_dim, w.groups
    io = torch.float32 if w.io == "f32" else torch.bfloat16
    A = -torch.exp(torch.rand(h, generator=gen, device=dev) * math.log(16.0))
    dt0 = torch.exp(math.log(1e-3) + torch.rand(h, generator=gen, device=dev)
                    * (math.log(0.1) - math.log(1e-3)))
    bias = dt0 + torch.log(-torch.expm1(-dt0))

    def nrm(*shape):
        return torch.randn(*shape, generator=gen, device=dev).to(io)
    d = dict(A=A, bias=bias, D=torch.ones(h, device=dev), x=nrm(b, l, h, p), dt=nrm(b, l, h),
             B=nrm(b, l, g, n), C=nrm(b, l, g, n))
    d["init"] = (w.init_std * torch.randn(b, h, n, p, generator=gen, device=dev)
                 if w.init_std > 0 else None)
    d["y"] = torch.empty_like(d["x"])
    return d


class Events:
    """8 HIP events (start, end of each kernel slot) per timed call, created
    through torch (recorded once so that they exist)."""

    def __init__(self, torch, calls):
        self.torch = torch
        self.ev = [[torch.cuda.Event(enable_timing=True) for _ in range(8)] for _ in range(calls)]
        for row in self.ev:
            for e in row:
                e.record()
        torch.cuda.synchronize()
        self.handles = [[e.cuda_event for e in row] for row in self.ev]

    def slot_ms(self, k, calls):
        """Average duration of slot k over the first `calls` calls (ms)."""
        tot = 0.0
        for i in range(calls):
            tot += self.ev[i][2 * k].elapsed_time(self.ev[i][2 * k + 1])
        return tot / calls


def time_scan(torch, ssd, w, dev, steps, warmup, max_sets=4, prewarm_s=0.0):
    """`prewarm_s` seconds of untimed calls, then W warmup + K timed
    ssd_chunk_scan calls over cycled input sets; then the same K calls again
    with kernel events.  Returns the step time and the average duration of
    every kernel."""
    b, l, h, p, n, g, Q = w.batch, w.seqlen, w.heads, w.head_dim, w.state_dim, w.groups, w.chunk
    s = 4 if w.io == "f32" else 2
    per_set = b * l * h * p * s * 2 + 2 * b * l * g * n * s
    nsets = max(1, min(max_sets, int(math.ceil(600e6 / per_set))))
    sets = [device_inputs(torch, w, dev, w.seed + 1000 * k) for k in range(nsets)]
    final = w.return_final
    fin = torch.empty((b, h, n, p), dtype=torch.float32, device=dev) if final else None
    ws = torch.empty(ssd.workspace_bytes(b, l, h, p, n, g, Q), dtype=torch.uint8, device=dev)

    def run(i, ev=None):
        S = sets[i % nsets]
        ssd.chunk_scan(S["x"], S["dt"], S["A"], S["B"], S["C"], S["D"], chunk_size=Q,
                       dt_bias=S["bias"], initial_state=S["init"], return_final_state=final,
                       final_out=fin, out=S["y"], workspace=ws, kernel_events=ev)
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < prewarm_s:
        for i in range(8):
            run(i)
        torch.cuda.synchronize()
    for i in range(warmup):
        run(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        run(i)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    evs = Events(torch, steps)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for i in range(steps):
        run(i, evs.handles[i])
    torch.cuda.synchronize()
    ms_ev = (time.perf_counter() - t1) * 1e3 / steps
    init = w.init_std > 0
    nst = ssd.state_chunks(b, l, h, p, n, g, Q, io=w.io)
    kern = {}
    # one stored chunk (bf16): the chunk output runs alone, from the initial
    # state to the final one
    one = w.io == "bf16" and nst == 1
    for k, name in enumerate(SLOTS):
        if one and name != "chunk_out":
            kern[name] = {"avg_us": 0.0, "alg_bytes": 0, "launched": False}
            continue
        us = 1e3 * evs.slot_ms(k, steps)
        alg = bytes_kernel(name, b, l, h, p, n, g, Q, s, init=init, final=final, nst=nst)
        if one:
            # x, B, C, dt read, y written, the fp32 initial state read and the
            # final state written
            alg = (2 * b * l * h * p * s + 2 * b * l * g * n * s + b * l * h * s
                   + b * h * n * p * 4 * (int(init) + int(final)))
        kern[name] = {"avg_us": round(us, 2), "alg_bytes": alg,
                      "GBs": round(alg / (us * 1e-6) / 1e9, 1),
                      "frac": round(alg / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
    balg = bytes_scan_alg(b, l, h, p, n, g, Q, s, init=init, final=final)
    bmin = bytes_scan_min(b, l, h, p, n, g, Q, s, init=init, final=final)
    res = {"workload": w.name, "batch": b, "seqlen": l, "heads": h, "head_dim": p,
           "state_dim": n, "groups": g, "chunk": Q, "stored_state_chunks": nst,
           "io": w.io, "init_state": init,
           "final_state": final, "input_sets": nsets,
           "ms_per_step": round(ms, 4), "ms_per_step_with_events": round(ms_ev, 4),
           "tokens_per_s": round(b * l / (ms * 1e-3), 1),
           "alg_bytes": balg, "min_bytes": bmin,
           "t_roof_us": round(balg / (HBM_PEAK_GBS * 1e9) * 1e6, 2),
           "frac_alg": round(balg / (HBM_PEAK_GBS * 1e9) / (ms * 1e-3), 4),
           "frac_min": round(bmin / (HBM_PEAK_GBS * 1e9) / (ms * 1e-3), 4),
           "kernels": kern}
    log("%s: %.4f ms/step (%.4f with events), %.4g tokens/s, frac_alg %.3f; %s" % (
        w.name, ms, ms_ev, res["tokens_per_s"], res["frac_alg"],
        json.dumps({k: v["avg_us"] for k, v in kern.items()})))
    del sets, ws
    torch.cuda.empty_cache()
    return res


# ---------------------------------------------------- profile summaries ---
CALIB_BYTES = 256 << 20
# kernel name patterns of the bf16 scan (the io type of every scan workload
# but the tiny fp32 one)
PROFILED = {"k_state16": "k_state16", "k_scan16": "k_scan16", "k_out16": "k_out16",
            "k_step": "k_step"}


def _csv_rows(path):
    import csv
    with open(path) as f:
        return list(csv.DictReader(f))


def _find(d, suffix):
    for root, _, files in os.walk(d):
        for fn in files:
            if fn.endswith(suffix):
                return os.path.join(root, fn)
    raise FileNotFoundError("no *%s under %s" % (suffix, d))


def _short(name):
    for k in PROFILED:
        if k in name:
            return k
    if "neg_kernel" in name:
        return "calib"
    return None


def syn_workload(name):
    sys.path.insert(0, ROOT)
    import ssd_synth as syn
    return syn.WORKLOADS[name]


def _kernel_label(name):
    """k_name<template ints> from a mangled or demangled kernel name."""
    import re
    m = re.search(r"(k_[a-z0-9_]+)", name)
    if not m:
        return name[:40]
    k = m.group(1)
    rest = name[m.end():]
    if name.startswith("_Z"):
        t = re.match(r"I((?:L[a-z]+\d+E|DF16b|[a-z])+)E", rest)
        if t:
            args = re.findall(r"L[a-z]+(\d+)E|(DF16b)|([fd])", t.group(1))
            vals = [a or ("bf16" if b else ("f32" if c == "f" else c)) for a, b, c in args]
            return "%s<%s>" % (k, ",".join(vals))
        return k
    t = re.match(r"<([^>]*)>", rest)
    return "%s<%s>" % (k, t.group(1).replace(" ", "")) if t else k


def summarize(a):
    """profiles/ summaries from rocprofv3 csv output (see --summarize)."""
    kind, wl = a[0], a[1]
    if kind == "trace":
        rows = _csv_rows(_find(a[2], "kernel_trace.csv"))
        cmd = " ".join(a[3:])
        per = {}
        for r in rows:
            k = _short(r.get("Kernel_Name", ""))
            if k in PROFILED:
                per.setdefault(k, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
        path = os.path.join(PROFILES, "scan_kernels_%s_kernel_trace.txt" % wl)
        with open(path, "w") as f:
            f.write("# rocprofv3 kernel trace of the bf16 chunked scan on the %s workload\n" % wl)
            f.write("# command (from /tmp with TMPDIR=/tmp, repository at $R):\n#   %s\n" % cmd)
            f.write("# every dispatch of the kernels: the probe's warmup, plain and "
                    "event-timed launches (decode: then the steps after the prefill, "
                    "as many again)\n\n")
            f.write("%-12s %6s %10s %10s %10s %10s\n" % ("kernel", "calls", "avg_us", "med_us",
                                                        "min_us", "max_us"))
            for k in PROFILED:
                v = sorted(per.get(k, []))
                if v:
                    f.write("%-12s %6d %10.2f %10.2f %10.2f %10.2f\n" % (
                        k, len(v), sum(v) / len(v), v[len(v) // 2], v[0], v[-1]))
            f.write("\nsource_digest: %s\n" % source_digest())
            if per.get("k_step"):
                f.write("k_step_source_digest: %s\n" % source_digest("k_step"))
        print("wrote", path)
        return
    if kind == "traffic":
        cmd = " ".join(a[4:])
        vals = {}
        for ctr, d in (("FETCH_SIZE", a[2]), ("WRITE_SIZE", a[3])):
            for r in _csv_rows(_find(d, "counter_collection.csv")):
                if r.get("Counter_Name") != ctr:
                    continue
                k = _short(r.get("Kernel_Name", ""))
                if k:
                    vals.setdefault((ctr, k), []).append(float(r["Counter_Value"]))
        # the calibration kernel: its largest dispatches (CALIB_BYTES each way)
        scale = {}
        for ctr in ("FETCH_SIZE", "WRITE_SIZE"):
            c = sorted(vals.get((ctr, "calib"), []))
            big = [v for v in c if v >= 0.5 * c[-1]] if c else []
            scale[ctr] = (CALIB_BYTES / 1024.0) / (sum(big) / len(big)) if big else None
        for k in PROFILED:
            fe, wr = vals.get(("FETCH_SIZE", k)), vals.get(("WRITE_SIZE", k))
            if not fe or not wr or scale["FETCH_SIZE"] is None or scale["WRITE_SIZE"] is None:
                continue
            fk, wk = sum(fe) / len(fe), sum(wr) / len(wr)
            hbm = fk * 1024 * scale["FETCH_SIZE"] + wk * 1024 * scale["WRITE_SIZE"]
            path = os.path.join(PROFILES, "%s_%s_traffic.txt" % (k, wl))
            with open(path, "w") as f:
                f.write("# HBM traffic of %s on the %s workload, from two rocprofv3 counter "
                        "runs\n" % (k, wl))
                f.write("# commands (from /tmp with TMPDIR=/tmp, repository at $R):\n")
                f.write("#   %s\n" % cmd.replace("COUNTER", "FETCH_SIZE"))
                f.write("#   %s\n" % cmd.replace("COUNTER", "WRITE_SIZE"))
                f.write("# per-dispatch means over the kernel's dispatches (KiB), each scaled "
                        "by what the\n# same counter reads for an elementwise kernel that "
                        "reads and writes %d MiB\n# (torch.neg) in the same run\n"
                        % (CALIB_BYTES >> 20))
                f.write("fetch_kib_raw_calibration: %.1f\n" % (CALIB_BYTES / 1024.0 /
                                                           scale["FETCH_SIZE"]))
                f.write("write_kib_raw_calibration: %.1f\n" % (CALIB_BYTES / 1024.0 /
                                                           scale["WRITE_SIZE"]))
                f.write("dispatches: %d\n" % len(fe))
                f.write("fetch_kib_per_dispatch: %.1f\n" % fk)
                f.write("write_kib_per_dispatch: %.1f\n" % wk)
                f.write("fetch_scale: %.4f\n" % scale["FETCH_SIZE"])
                f.write("write_scale: %.4f\n" % scale["WRITE_SIZE"])
                f.write("hbm_bytes_per_launch: %d\n" % int(hbm))
                f.write("source_digest: %s\n" % source_digest(k))
            print("wrote", path)
        return
    if kind == "sq":
        # SQ counters of the scan kernels: per-dispatch means of every
        # counter in the comma-separated counter-run directories; the
        # commands that made them separated by ' ;; '
        dirs = a[2].split(",")
        cmds = " ".join(a[3:]).split(" ;; ")
        vals = {}
        for d in dirs:
            for r in _csv_rows(_find(d, "counter_collection.csv")):
                k = _short(r.get("Kernel_Name", ""))
                if k in ("k_state16", "k_scan16", "k_out16"):
                    vals.setdefault(k, {}).setdefault(r["Counter_Name"], []).append(
                        float(r["Counter_Value"]))
        path = os.path.join(PROFILES, "scan_kernels_%s_sq_counters.txt" % wl)
        w = syn_workload(wl)
        with open(path, "w") as f:
            f.write("# SQ counters of the bf16 scan kernels on the %s workload (batch %d, seqlen "
                    "%d,\n# %d heads, head_dim %d, state_dim %d, %d groups, chunk %d), "
                    "per-dispatch means over the\n# probe's dispatches; %d counter runs (from "
                    "/tmp with TMPDIR=/tmp, repository at $R):\n"
                    % (wl, w.batch, w.seqlen, w.heads, w.head_dim, w.state_dim, w.groups,
                       w.chunk, len(cmds)))
            for c in cmds:
                f.write("#   %s\n" % c.strip())
            f.write("\n")
            for k in ("k_state16", "k_scan16", "k_out16"):
                if k not in vals:
                    continue
                f.write("%s\n" % k)
                for ctr in sorted(vals[k]):
                    v = vals[k][ctr]
                    f.write("  %-30s %18.1f\n" % (ctr, sum(v) / len(v)))
                f.write("\n")
            f.write("source_digest: %s\n" % source_digest())
        print("wrote", path)
        return
    if kind == "bench":
        # every scan kernel of a bench.py run of one workload (its pre-warm,
        # warm-up, timed and event-timed calls)
        rows = _csv_rows(_find(a[2], "kernel_trace.csv"))
        cmd = " ".join(a[3:])
        per = {}
        for r in rows:
            k = _short(r.get("Kernel_Name", ""))
            if k in ("k_state16", "k_scan16", "k_out16"):
                per.setdefault(k, []).append(
                    (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
        path = os.path.join(PROFILES, "bench_%s_kernel_trace.txt" % wl)
        with open(path, "w") as f:
            f.write("# rocprofv3 kernel trace of the bench's own measurement of the %s "
                    "workload\n" % wl)
            f.write("# command (from /tmp with TMPDIR=/tmp, repository at $R):\n#   %s\n" % cmd)
            f.write("# every dispatch of the scan kernels in the run: pre-warm, warm-up, "
                    "timed and event-timed calls\n\n")
            f.write("%-12s %6s %10s %10s %10s %10s\n" % ("kernel", "calls", "avg_us", "med_us",
                                                        "min_us", "max_us"))
            for k in ("k_state16", "k_scan16", "k_out16"):
                v = sorted(per.get(k, []))
                if v:
                    f.write("%-12s %6d %10.2f %10.2f %10.2f %10.2f\n" % (
                        k, len(v), sum(v) / len(v), v[len(v) // 2], v[0], v[-1]))
            f.write("\nsource_digest: %s\n" % source_digest())
        print("wrote", path)
        return
    if kind == "bwd":
        # the gradient calls of a run (each from its first kernel,
        # k_transpose_tiles, to its last, k_bwd_sum): every kernel's
        # dispatches inside them, grouped by kernel and template arguments
        rows = _csv_rows(_find(a[2], "kernel_trace.csv"))
        cmd = " ".join(a[3:])
        ev = sorted(((int(r["Start_Timestamp"]), int(r["End_Timestamp"]),
                      r.get("Kernel_Name", "")) for r in rows))
        calls, cur = [], None
        for t0, t1, nm in ev:
            if "k_transpose_tiles" in nm:
                cur = []
            if cur is not None:
                cur.append((t0, t1, nm))
                if "k_bwd_sum" in nm:
                    calls.append(cur)
                    cur = None
        per, spans, ktot = {}, [], []
        for c in calls:
            spans.append((c[-1][1] - c[0][0]) / 1e3)
            ktot.append(sum(t1 - t0 for t0, t1, _ in c) / 1e3)
            for t0, t1, nm in c:
                per.setdefault(_kernel_label(nm), []).append((t1 - t0) / 1e3)
        path = os.path.join(PROFILES, "gradient_pass_%s_kernel_trace.txt" % wl)
        with open(path, "w") as f:
            f.write("# rocprofv3 kernel trace of bench.py's gradient-pass measurement, %s "
                    "workload (bf16 io,\n# final-state cotangent)\n" % wl)
            f.write("# command (from /tmp with TMPDIR=/tmp, repository at $R):\n#   %s\n" % cmd)
            f.write("# every gradient call in the run (%d), from its first kernel "
                    "(k_transpose_tiles) to its last (k_bwd_sum)\n\n" % len(calls))
            f.write("%-58s %6s %10s %10s\n" % ("kernel", "calls", "avg_us", "total_us"))
            for k, v in sorted(per.items(), key=lambda kv: -sum(kv[1])):
                f.write("%-58s %6d %10.2f %10.1f\n" % (k, len(v), sum(v) / len(v), sum(v)))
            if calls:
                f.write("\nkernel time per call: %.1f us; first dispatch to last end per call: "
                        "median %.1f us\n" % (sum(ktot) / len(ktot),
                                              sorted(spans)[len(spans) // 2]))
            f.write("source_digest: %s\n" % source_digest())
        print("wrote", path)
        return
    if kind == "mixer":
        # every kernel of a --mixer-probe run: the conv, the scan's three
        # kernels and the norm, as one ssd_mixer_forward call launches them
        rows = _csv_rows(_find(a[2], "kernel_trace.csv"))
        cmd = " ".join(a[3:])
        names = ("k_conv1d_silu", "k_state16", "k_scan16", "k_out16", "k_gated_norm")
        per = {}
        for r in rows:
            nm = r.get("Kernel_Name", "")
            k = next((x for x in names if x in nm), None)
            if k:
                per.setdefault(k, []).append(
                    (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
        path = os.path.join(PROFILES, "mixer_%s_kernel_trace.txt" % wl)
        with open(path, "w") as f:
            f.write("# rocprofv3 kernel trace of ssd_mixer_forward (conv1d + SiLU, chunk scan, "
                    "gated norm) at the %s mixer shape\n" % wl)
            f.write("# command (from /tmp with TMPDIR=/tmp, repository at $R):\n#   %s\n" % cmd)
            f.write("# every dispatch of the probe's calls (warm-up and timed)\n\n")
            f.write("%-14s %6s %10s %10s %10s %10s\n" % ("kernel", "calls", "avg_us", "med_us",
                                                        "min_us", "max_us"))
            tot = 0.0
            for k in names:
                v = sorted(per.get(k, []))
                if v:
                    tot += sum(v) / len(v)
                    f.write("%-14s %6d %10.2f %10.2f %10.2f %10.2f\n" % (
                        k, len(v), sum(v) / len(v), v[len(v) // 2], v[0], v[-1]))
            f.write("\nsum of kernel averages: %.2f us\n" % tot)
            f.write("neighbors_source_digest: %s\n" % source_digest("neighbors"))
            f.write("source_digest: %s\n" % source_digest())
        print("wrote", path)
        return
    raise SystemExit("unknown summary kind %r" % kind)


# ------------------------------------------------------------------ main ---
def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--decode-steps", type=int, default=128)
    ap.add_argument("--workloads", default=",".join(SCAN_WORKLOADS),
                    help="scan workloads timed (the headline is always included)")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-states", action="store_true",
                    help="skip the packed-sequence and state-output measurements")
    ap.add_argument("--no-neighbors", action="store_true",
                    help="skip the conv1d and gated-norm measurements")
    ap.add_argument("--no-backward", action="store_true",
                    help="skip the gradient-pass measurement")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--prewarm-s", type=float, default=0.3,
                    help="seconds of untimed scan calls on each workload before its W warmup "
                         "steps: a sudden sustained load drives the GPU's power management "
                         "through a transient of ~40 steps (grouped_long per-step times 0.62, "
                         "then up to 0.83, settling at 0.60 ms)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--traffic-probe", default="",
                    help="workload: run a few scans of it and a 256 MiB copy (the counters' "
                         "calibration), for profiler runs, and exit")
    ap.add_argument("--mixer-probe", action="store_true",
                    help="run the 130m-shape mixer (ssd_mixer_forward) 2 x --probe-steps "
                         "times after its warm-up, for profiler runs, and exit")
    ap.add_argument("--probe-steps", type=int, default=3,
                    help="timed scans of the probe (each run twice: plain and with events)")
    ap.add_argument("--summarize", nargs="+", metavar="ARG", default=None,
                    help="write profiles/ summaries from rocprofv3 csv output and exit: "
                         "'trace WORKLOAD TRACE_DIR COMMAND...' or "
                         "'traffic WORKLOAD FETCH_DIR WRITE_DIR COMMAND...'")
    args = ap.parse_args()
    global PREWARM_S
    PREWARM_S = args.prewarm_s

    if args.summarize:
        summarize(args.summarize)
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the scan is built and measured on a single "
              "MI355X (no multi-GPU path); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch

    import mamba_ssd_chunked_chunk_amd as ssd
    import ssd_synth as syn

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")

    if args.mixer_probe:
        r = bench_mixer(argparse.Namespace(steps=2 * args.probe_steps), torch, ssd, syn, dev,
                        only_one_call=True)
        print(json.dumps({"mixer_probe": r}))
        return

    if args.traffic_probe:
        # a fixed number of dispatches for the profilers: no time-based pre-warm
        PREWARM_S = 0.0
        w = syn.WORKLOADS[args.traffic_probe]
        if w.name == "decode_2p7b":
            w = w.replace(name="decode_2p7b_prefill")
        r = time_scan(torch, ssd, w, dev, steps=args.probe_steps, warmup=2)
        if w.name == "decode_2p7b_prefill":
            # the decode step after the prefill (the k_step counters)
            bench_decode(argparse.Namespace(decode_steps=args.probe_steps), torch, ssd, syn, dev)
        # calibration: a plain elementwise kernel that reads CALIB_BYTES and
        # writes CALIB_BYTES (torch.neg; a same-type copy_ would go to the
        # copy engine, which the counters do not see)
        src = torch.ones(CALIB_BYTES // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        print(json.dumps({"traffic_probe": w.name,
                          "kernels_us": {k: v["avg_us"] for k, v in r["kernels"].items()}}))
        return

    names = [nm for nm in args.workloads.split(",") if nm]
    if HEADLINE not in names:
        names.append(HEADLINE)
    results = {}
    for nm in names:
        w = syn.WORKLOADS[nm]
        if nm == "decode_2p7b":
            w = w.replace(name="decode_2p7b_prefill")
        results[w.name] = time_scan(torch, ssd, w, dev, args.steps, args.warmup,
                                    prewarm_s=args.prewarm_s)
    head = results[HEADLINE]
    wh = syn.WORKLOADS[HEADLINE]
    dom = max(SLOTS, key=lambda k: head["kernels"][k]["avg_us"])
    dk = head["kernels"][dom]
    achieved = dk["alg_bytes"] / (dk["avg_us"] * 1e-6) / 1e9
    kname = {"chunk_state": "k_state16", "state_scan": "k_scan16", "chunk_out": "k_out16"}[dom]
    roofline = {"kernel": kname, "bound": "hbm", "achieved": round(achieved, 1),
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": measured_traffic(kname, HEADLINE),
                "alg_bytes_per_launch": dk["alg_bytes"], "avg_launch_us": dk["avg_us"],
                "launches_timed": args.steps}
    scan_roof = {"bound": "hbm", "alg_bytes": head["alg_bytes"], "min_bytes": head["min_bytes"],
                 "t_roof_us": head["t_roof_us"], "t_step_us": round(head["ms_per_step"] * 1e3, 2),
                 "frac_alg": head["frac_alg"], "frac_min": head["frac_min"],
                 "kernels": head["kernels"]}

    extra = {}
    if not args.no_states:
        extra["states"] = bench_states(args, torch, ssd, syn, dev)
    if not args.no_neighbors:
        extra["neighbors"] = bench_neighbors(args, torch, ssd, syn, dev)
    if not args.no_backward:
        extra["backward"] = bench_backward(args, torch, ssd, syn, dev)
    decode = None if args.no_decode else bench_decode(args, torch, ssd, syn, dev)
    cpu = None if args.no_cpu else cpu_baseline(args, syn, wh)

    out = {
        "metric": METRIC, "value": head["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "prewarm_s": args.prewarm_s,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) x/B/C/dt, A=-exp(U[0,ln16]), "
                "dt_bias=softplus^-1(loguniform[1e-3,0.1]), D=1, zero initial state)",
        "config": {"workload": HEADLINE, "batch": wh.batch, "seqlen": wh.seqlen,
                   "heads": wh.heads, "head_dim": wh.head_dim, "state_dim": wh.state_dim,
                   "groups": wh.groups, "chunk": wh.chunk, "io": "bf16", "state": "fp32",
                   "input_sets": head["input_sets"]},
        "roofline": roofline,
        "scan_roofline": scan_roof,
        "workloads": results,
        "decode": decode,
        "cpu_baseline": cpu,
    }
    out.update(extra)
    print(json.dumps(out))


# --------------------------------------------------------------- extras ----
# seconds of untimed calls before each measurement's warmup (--prewarm-s)
PREWARM_S = 0.0


def _prewarm(torch, fn):
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < PREWARM_S:
        for i in range(8):
            fn(i)
        torch.cuda.synchronize()


def _time_calls(torch, fn, calls, warm=3):
    """Average ms of fn(i) over `calls` calls, each bracketed by events on
    the current stream (one kernel per call), after PREWARM_S seconds and
    `warm` calls of untimed calls."""
    _prewarm(torch, fn)
    for i in range(warm):
        fn(i)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(calls)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(calls):
        evs[i][0].record()
        fn(i)
        evs[i][1].record()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3 / calls
    return wall, sum(a.elapsed_time(b) for a, b in evs) / calls


def bench_states(args, torch, ssd, syn, dev):
    """The scan at the Mamba2-130m shape with packed documents (a per-token
    document index), with the state after every chunk written, and the state
    after every token (chunk 1) for one batch row."""
    w = syn.WORKLOADS["mamba2_130m"]
    b, l, h, p, n, g, Q = w.batch, w.seqlen, w.heads, w.head_dim, w.state_dim, w.groups, w.chunk
    S = device_inputs(torch, w, dev, w.seed + 77)
    ws = torch.empty(ssd.workspace_bytes(b, l, h, p, n, g, Q), dtype=torch.uint8, device=dev)
    seq = torch.from_numpy(syn.doc_index(w.seed + 77, b, l)).to(dev)
    nc = -(-l // Q)
    st_out = torch.empty((b, nc, h, n, p), dtype=torch.float32, device=dev)
    steps = max(args.steps // 2, 10)

    evs = Events(torch, steps)

    def plain(i, ev=None):
        ssd.chunk_scan(S["x"], S["dt"], S["A"], S["B"], S["C"], S["D"], chunk_size=Q,
                       dt_bias=S["bias"], out=S["y"], workspace=ws, kernel_events=ev)

    def packed(i, ev=None):
        ssd.chunk_scan(S["x"], S["dt"], S["A"], S["B"], S["C"], S["D"], chunk_size=Q,
                       dt_bias=S["bias"], out=S["y"], workspace=ws, seq_idx=seq,
                       kernel_events=ev)

    def states(i, ev=None):
        ssd.chunk_scan(S["x"], S["dt"], S["A"], S["B"], S["C"], S["D"], chunk_size=Q,
                       dt_bias=S["bias"], out=S["y"], workspace=ws, return_chunk_states=True,
                       chunk_states_out=st_out, kernel_events=ev)
    res = {}
    # the plain scan on the same single input set, for a like-for-like ratio
    for name, fn in (("plain_same_inputs", plain), ("packed", packed),
                     ("chunk_states", states)):
        wall, _ = _time_calls(torch, fn, steps)
        for i in range(steps):
            fn(i, evs.handles[i])
        torch.cuda.synchronize()
        kern = {k: round(1e3 * evs.slot_ms(j, steps), 2) for j, k in enumerate(SLOTS)}
        res[name] = {"value": round(b * l / (wall * 1e-3), 1), "unit": "tokens/s",
                     "ms_per_step": round(wall, 4), "kernels_us": kern}
        log("%s: %.4f ms/step %s" % (name, wall, json.dumps(kern)))
    res["packed"]["documents_per_step"] = int(seq[:, -1].sum()) + b
    res["packed"]["over_plain"] = round(res["packed"]["ms_per_step"] /
                                        res["plain_same_inputs"]["ms_per_step"], 4)
    x1, dt1, B1, C1 = S["x"][:1], S["dt"][:1], S["B"][:1], S["C"][:1]
    y1 = torch.empty((1, l, h, p), dtype=torch.bfloat16, device=dev)
    tok = torch.empty((1, l, h, n, p), dtype=torch.float32, device=dev)
    ws1 = torch.empty(ssd.workspace_bytes(1, l, h, p, n, g, 1), dtype=torch.uint8, device=dev)

    def per_token(i):
        ssd.chunk_scan(x1, dt1, S["A"], B1, C1, S["D"], chunk_size=1, dt_bias=S["bias"],
                       out=y1, workspace=ws1, return_chunk_states=True, chunk_states_out=tok)
    wall, _ = _time_calls(torch, per_token, max(steps // 10, 5))
    wbytes = l * h * n * p * 4
    res["per_token"] = {"value": round(l / (wall * 1e-3), 1), "unit": "tokens/s",
                        "ms_per_call": round(wall, 4), "state_bytes_written": wbytes,
                        "state_write_GBs": round(wbytes / (wall * 1e-3) / 1e9, 1)}
    log("per-token states: %.3f ms per row" % wall)
    res["config"] = {"workload": "mamba2_130m", "doc_lengths": "log-uniform in [32, 2048]"}
    return res


def bench_neighbors(args, torch, ssd, syn, dev):
    """The steps around the scan at the 130m mixer's shape (8 x 2048 tokens,
    24 heads of 64, state 128, 1 group, bf16): the width-4 causal conv1d +
    SiLU + split of the 1792 projection channels, and the silu(z) gate with
    one RMS norm over the 1536 channels."""
    b, l, h, p, n, g, K = 8, 2048, 24, 64, 128, 1, 4
    ch = h * p + 2 * g * n
    gen = torch.Generator(device=dev)
    gen.manual_seed(900)
    xbc = torch.randn(b, l, ch, generator=gen, device=dev).bfloat16()
    wt = (torch.rand(ch, K, generator=gen, device=dev) * 2 - 1) / math.sqrt(K)
    bias = (torch.rand(ch, generator=gen, device=dev) * 2 - 1) / math.sqrt(K)
    y = torch.randn(b * l, h * p, generator=gen, device=dev).bfloat16()
    z = torch.randn(b * l, h * p, generator=gen, device=dev).bfloat16()
    nw = 1 + 0.1 * torch.randn(h * p, generator=gen, device=dev)
    outs = (torch.empty((b, l, h, p), dtype=torch.bfloat16, device=dev),
            torch.empty((b, l, g, n), dtype=torch.bfloat16, device=dev),
            torch.empty((b, l, g, n), dtype=torch.bfloat16, device=dev))
    nout = torch.empty_like(y)
    steps = max(args.steps // 2, 10)
    res = {}
    for name, fn, alg in (
            ("conv1d_silu", lambda i: ssd.conv1d_silu(xbc, wt, h, p, n, g, bias=bias, out=outs),
             2 * b * l * ch * 2 + ch * (K + 1) * 4),
            ("gated_norm", lambda i: ssd.gated_norm(y, z, nw, eps=1e-5, out=nout),
             3 * b * l * h * p * 2 + h * p * 4)):
        _, ms = _time_calls(torch, fn, steps)
        gbs = alg / (ms * 1e-3) / 1e9
        log("%s: %.2f us, %.0f GB/s" % (name, ms * 1e3, gbs))
        res[name] = {"avg_launch_us": round(ms * 1e3, 2), "alg_bytes_per_launch": alg,
                     "roofline": {"bound": "hbm", "achieved": round(gbs, 1),
                                  "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                  "frac": round(gbs / HBM_PEAK_GBS, 4)}}
    res["mixer"] = bench_mixer(args, torch, ssd, syn, dev)
    res["config"] = {"workload": "mamba2_130m mixer", "conv_width": K, "norm_groups": 1}
    return res


def bench_mixer(args, torch, ssd, syn, dev, sets=4, only_one_call=False):
    """The whole mixer between the projections at the 130m shape (8 x 2048
    tokens, bf16, conv width 4 over 1792 channels, one RMS norm over 1536):
    one ssd_mixer_forward call against the three entry points called in a
    row on the same inputs, both cycling through `sets` independently drawn
    input sets (xbc, dt, z: 110 MB a set) so that inputs are not served
    from the 256 MB Infinity Cache."""
    w = syn.WORKLOADS["mamba2_130m"]
    b, l, h, p, n, g, Q, K = w.batch, w.seqlen, w.heads, w.head_dim, w.state_dim, w.groups, \
        w.chunk, 4
    ch = h * p + 2 * g * n
    gen = torch.Generator(device=dev)
    gen.manual_seed(901)
    S = []
    for _ in range(sets):
        S.append(dict(xbc=torch.randn(b, l, ch, generator=gen, device=dev).bfloat16(),
                      z=torch.randn(b, l, h * p, generator=gen, device=dev).bfloat16(),
                      dt=torch.randn(b, l, h, generator=gen, device=dev).bfloat16()))
    wt = (torch.rand(ch, K, generator=gen, device=dev) * 2 - 1) / math.sqrt(K)
    cb = (torch.rand(ch, generator=gen, device=dev) * 2 - 1) / math.sqrt(K)
    A = -torch.exp(torch.rand(h, generator=gen, device=dev) * math.log(16))
    dtb = torch.log(torch.expm1(torch.exp(
        torch.rand(h, generator=gen, device=dev) * (math.log(0.1) - math.log(1e-3)) +
        math.log(1e-3))))
    D = torch.ones(h, device=dev)
    nw = 1 + 0.1 * torch.randn(h * p, generator=gen, device=dev)
    out = torch.empty((b, l, h, p), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(ssd.mixer_workspace_bytes(b, l, h, p, n, g, Q), dtype=torch.uint8,
                     device=dev)
    xs = (torch.empty((b, l, h, p), dtype=torch.bfloat16, device=dev),
          torch.empty((b, l, g, n), dtype=torch.bfloat16, device=dev),
          torch.empty((b, l, g, n), dtype=torch.bfloat16, device=dev))
    y = torch.empty((b, l, h, p), dtype=torch.bfloat16, device=dev)
    sws = torch.empty(ssd.workspace_bytes(b, l, h, p, n, g, Q), dtype=torch.uint8, device=dev)

    def one(i):
        s = S[i % sets]
        ssd.mixer_forward(s["xbc"], s["dt"], A, wt, h, p, n, g, z=s["z"], conv_bias=cb, D=D,
                          dt_bias=dtb, norm_weight=nw, chunk_size=Q, out=out, workspace=ws)

    def chain(i):
        s = S[i % sets]
        x, B, C = ssd.conv1d_silu(s["xbc"], wt, h, p, n, g, bias=cb, out=xs)
        ssd.chunk_scan(x, s["dt"], A, B, C, D, chunk_size=Q, dt_bias=dtb, out=y, workspace=sws)
        ssd.gated_norm(y.reshape(b * l, h * p), s["z"].reshape(b * l, h * p), nw,
                       out=out.reshape(b * l, h * p))
    steps = max(args.steps // 2, 10)
    res = {}
    for name, fn in (("one_call", one),) + (() if only_one_call else
                                             (("separate_calls", chain),)):
        wall, ev = _time_calls(torch, fn, steps)
        res[name] = {"ms_per_call": round(ev, 4), "wall_ms_per_call": round(wall, 4),
                     "value": round(b * l / (ev * 1e-3), 1), "unit": "tokens/s"}
        log("mixer %s: %.4f ms" % (name, ev))
    # bytes a mixer must move: xbc, dt and z read, out written (bf16), the
    # conv taps and the per-head and norm parameters (the scan's state
    # round trip and the x/B/C and y intermediates are the design's, not
    # the method's)
    alg = (b * l * (ch + h + 2 * h * p)) * 2 + ch * (K + 1) * 4 + 3 * h * 4 + h * p * 4
    ms = res["one_call"]["ms_per_call"]
    res["alg_bytes"] = alg
    res["frac_of_hbm_roof"] = round(alg / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)
    if not only_one_call:
        res["one_call_over_separate"] = round(ms / res["separate_calls"]["ms_per_call"], 4)
    res["input_sets"] = sets
    return res


def bench_backward(args, torch, ssd, syn, dev):
    """The gradient pass (ssd_chunk_scan_bwd) at the Mamba2-130m shape with a
    final-state cotangent, against the bytes any gradient pass must move."""
    w = syn.WORKLOADS["mamba2_130m"]
    b, l, h, p, n, g, Q = w.batch, w.seqlen, w.heads, w.head_dim, w.state_dim, w.groups, w.chunk
    S = device_inputs(torch, w, dev, w.seed + 99)
    gen = torch.Generator(device=dev)
    gen.manual_seed(w.seed + 98)
    dy = torch.randn((b, l, h, p), generator=gen, device=dev).bfloat16()
    dfin = torch.randn((b, h, n, p), generator=gen, device=dev)
    wsb = int(ssd._lib.load().ssd_chunk_scan_bwd_workspace_bytes(b, l, h, p, n, g, Q,
                                                                 1 if w.io == "bf16" else 0))
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev)

    def run(i):
        ssd.chunk_scan_bwd(S["x"], S["dt"], S["A"], S["B"], S["C"], dy, D=S["D"], chunk_size=Q,
                           dt_bias=S["bias"], d_final=dfin, workspace=ws)
    wall, _ = _time_calls(torch, run, max(args.steps // 10, 5))
    s = 2
    min_bytes = (2 * (2 * b * l * h * p * s + 2 * b * l * g * n * s + b * l * h * s)
                 + 2 * b * h * n * p * 4)
    gbs = min_bytes / (wall * 1e-3) / 1e9
    log("backward: %.3f ms per call" % wall)
    return {"metric": "gradient pass tokens/s", "value": round(b * l / (wall * 1e-3), 1),
            "unit": "tokens/s", "ms_per_call": round(wall, 4), "workspace_bytes": wsb,
            "min_bytes": min_bytes,
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4)},
            "config": {"workload": "mamba2_130m", "io": "bf16", "d_final": True,
                       "deterministic": True}}


def bench_decode(args, torch, ssd, syn, dev):
    """Decode steps/s: batch 256, 80 heads, head_dim 64, state 128, bf16 io,
    fp32 state initialised by a 1024-token chunk-scan prefill."""
    w = syn.WORKLOADS["decode_2p7b"]
    b, l, h, p, n, g = w.batch, w.seqlen, w.heads, w.head_dim, w.state_dim, w.groups
    S = device_inputs(torch, w, dev, w.seed)
    _, st = ssd.chunk_scan(S["x"], S["dt"], S["A"], S["B"], S["C"], S["D"], chunk_size=w.chunk,
                           dt_bias=S["bias"], return_final_state=True)
    A, D, bias = S["A"], S["D"], S["bias"]
    del S
    gen = torch.Generator(device=dev)
    gen.manual_seed(w.seed + 5)
    K = args.decode_steps

    def rnd(*shape):
        return torch.randn(*shape, generator=gen, device=dev).bfloat16()
    xs, dts, Bs, Cs = rnd(K, b, h, p), rnd(K, b, h), rnd(K, b, g, n), rnd(K, b, g, n)
    y = torch.empty((b, h, p), dtype=torch.bfloat16, device=dev)
    _prewarm(torch, lambda k: ssd.step(st, xs[k % K], dts[k % K], A, Bs[k % K], Cs[k % K], D,
                                       dt_bias=bias, out=y))
    for k in range(3):
        ssd.step(st, xs[k], dts[k], A, Bs[k], Cs[k], D, dt_bias=bias, out=y)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(K):
        ssd.step(st, xs[k], dts[k], A, Bs[k], Cs[k], D, dt_bias=bias, out=y)
    torch.cuda.synchronize()
    rate = K / (time.perf_counter() - t0)
    _, ms = _time_calls(torch, lambda k: ssd.step(st, xs[k % K], dts[k % K], A, Bs[k % K],
                                                  Cs[k % K], D, dt_bias=bias, out=y), K, warm=0)
    alg = bytes_step(b, h, p, n, g, 2)
    achieved = alg / (ms * 1e-3) / 1e9
    log("decode: %.1f steps/s, kernel %.2f us, %.0f GB/s" % (rate, ms * 1e3, achieved))
    return {"metric": "decode steps/s", "value": round(rate, 1), "unit": "steps/s",
            "tokens_per_s": round(rate * b, 1), "steps": K,
            "config": {"workload": "decode_2p7b", "batch": b, "heads": h, "head_dim": p,
                       "state_dim": n, "groups": g, "io": "bf16", "state": "fp32",
                       "prefill_tokens": l},
            "roofline": {"kernel": "k_step", "bound": "hbm", "achieved": round(achieved, 1),
                         "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(achieved / HBM_PEAK_GBS, 4),
                         "traffic": measured_traffic("k_step", "decode_2p7b"),
                         "alg_bytes_per_launch": alg, "avg_launch_us": round(ms * 1e3, 2)}}


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def cpu_baseline(args, syn, w):
    """The fp64 oracle as it stands, on the host cores, over a bounded sample
    of the headline workload: 16 of its 64 heads over its first 16384
    tokens, repeated for about --cpu-seconds of wall time; and one thread
    over 2 heads of the same tokens.  Reported in the headline's unit
    (a token being one position across all 64 heads)."""
    import oracle
    oracle.build()
    L, heads = 16384, 16
    inp = syn.make_inputs(w, seqlen=L)
    pairs = [(0, hh) for hh in range(0, w.heads, w.heads // heads)][:heads]
    cores = oracle.default_threads()

    def rate(prs, nthreads, seconds):
        passes = 0
        t0 = time.perf_counter()
        while True:
            oracle.scan(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp["D"],
                        inp["dt_bias"], io=inp["io"], pairs=prs, nthreads=nthreads)
            passes += 1
            if time.perf_counter() - t0 >= seconds:
                break
        dt_s = time.perf_counter() - t0
        return passes * len(prs) * L / w.heads / dt_s, passes, dt_s
    v, passes, dt_s = rate(pairs, cores, args.cpu_seconds)
    v1, p1, d1 = rate(pairs[:2], 1, max(args.cpu_seconds / 4, 2.0))
    log("oracle: %.4g tokens/s on %d threads, %.4g on one" % (v, cores, v1))
    return {"value": round(v, 1), "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "cpu_model": cpu_model(),
            "single_thread_value": round(v1, 1),
            "sample": "%d pass(es) over %d of %d heads x %d of %d tokens of the %s workload "
                      "(%.1f s wall); single thread: %d pass(es) over 2 heads (%.1f s)"
                      % (passes, len(pairs), w.heads, L, w.seqlen, w.name, dt_s, p1, d1)}


if __name__ == "__main__":
    main()
