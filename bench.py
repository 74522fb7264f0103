#!/usr/bin/env python3
"""Benchmark of the SSD scan on one MI355X.

One step = one ssd_chunk_scan over one batch of the Mamba2-130m-shaped
workload (batch 8, seqlen 2048, 24 heads, head_dim 64, state_dim 128,
1 group, chunk 256, bf16 io, fp32 state), inputs resident in HBM.  Steps
cycle through several independently drawn input/output sets so that the
working set exceeds the 256 MB Infinity Cache.  Printed: one JSON line with
tokens/s (value), the dominant kernel's roofline (HIP-event durations of
that kernel on its launch stream), the whole scan against its HBM roofline,
the decode step rate (ssd_step at batch 256, 80 heads, state from a
1024-token prefill), and the oracle timed on the host cores.

    python bench.py [--steps K] [--warmup W] [--gpus 1]
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

METRIC = "SSD scan tokens/sec at 1 GPU; % of MFMA/HBM roofline; decode steps/sec"
HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published
KERNEL_IDS = ("chunk_state", "state_scan", "chunk_out")
PROFILES = os.path.join(ROOT, "profiles")
KERNEL_SOURCES = ("mamba_ssd_chunked_chunk_amd/csrc/ssd_scan.hpp",
                  "mamba_ssd_chunked_chunk_amd/csrc/ssd_device.hpp",
                  "mamba_ssd_chunked_chunk_amd/csrc/ssd_plan.hpp")


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def source_digest() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


# ----------------------------------------------------------- byte counts ---
def plan_sizes(b, l, h, p, n, g, Q, T=32):
    """Chunks and padded rows per sequence, as the library plans them
    (32-row blocks that never straddle a chunk boundary)."""
    nc = -(-l // Q)
    lp = nc * (-(-Q // T) * T)
    return nc, lp


def bytes_scan_alg(b, l, h, p, n, g, Q, s, init=False, final=False):
    """Algorithmic bytes of the whole scan: inputs and outputs once plus one
    write and one read of the fp32 chunk-boundary-state tensor."""
    th = b * l * h
    per = 2 * p * s + 2 * n * s * g / h + s + 8.0 * n * p / Q
    extra = (4 * n * p * b * h) * (int(init) + int(final))
    return th * per + extra


def bytes_scan_min(b, l, h, p, n, g, Q, s, init=False, final=False):
    th = b * l * h
    return th * (2 * p * s + 2 * n * s * g / h + s) + 4 * n * p * b * h * (int(init) + int(final))


def bytes_kernel(name, b, l, h, p, n, g, Q, s, final=False, init=False, states=False):
    """Algorithmic bytes of one launch of a scan kernel: every operand of its
    step of the method moved once (per-row workspace arrays fp32; chunk
    states fp32 on the fp32 path and scaled fp16 on the bf16 path; boundary
    states in the read-out's operand type: fp16 on the bf16 path, fp32 on
    the fp32 path; with `states`, the state after every chunk written in
    fp32)."""
    nc, lp = plan_sizes(b, l, h, p, n, g, Q)
    th = b * l * h
    x = th * p * s                     # x (and y) in the io dtype
    BC = b * l * g * n * s             # B or C, once per group
    rows = b * h * lp * 4              # one per-row fp32 array (lcs, d or weight)
    so = 2 if s == 2 else 4            # boundary-state element
    se = 2 if s == 2 else 4            # chunk-state element (bf16 io: scaled fp16)
    # chunk states needed: the last chunk's only feeds the final state and
    # the state after the last chunk
    ns = nc if (final or states) else nc - 1
    sn = b * ns * h * n * p
    # boundary states stored and read: chunk 0's is the initial state, zero
    # (and neither stored nor read) when none is given
    sb = b * (nc if init else nc - 1) * h * n * p
    fin = b * h * n * p * 4 if final else 0
    sout = b * nc * h * n * p * 4 if states else 0
    if name == "chunk_state":
        # x, B and dt read; the per-row lcs, d and weights, the needed chunk
        # states, their decays (and on the bf16 path their scales) written
        return x + BC + th * s + 3 * rows + se * sn + b * h * ns * (8 if s == 2 else 4)
    if name == "state_scan":
        # needed chunk states and decays read, boundary states written; on the
        # bf16 path also B and C read once and their fp16 block images written
        img = 2 * BC + 2 * b * nc * g * (-(-Q // 32) * 32) * n * 2 if s == 2 else 0
        return se * sn + b * h * ns * (8 if s == 2 else 4) + so * sb + fin + img + sout
    if name == "chunk_out":
        # x, B and C (bf16 path: their fp16 block images, the same size), the
        # lcs, d and weight rows and the boundary states read, y written
        return x + 2 * BC + 3 * rows + so * sb + x
    raise KeyError(name)


def bytes_step(b, h, p, n, g, s):
    return b * h * (8 * n * p + 2 * p * s + s) + 2 * b * g * n * s + 12 * h


# --------------------------------------------------------------- traffic ---
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
        if kv.get("source_digest") != source_digest():
            return None
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


# ------------------------------------------------------------------ main ---
def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--sets", type=int, default=4, help="input/output sets cycled through")
    ap.add_argument("--decode-steps", type=int, default=128)
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-states", action="store_true",
                    help="skip the packed-sequence and state-output measurements")
    ap.add_argument("--no-neighbors", action="store_true",
                    help="skip the conv1d and gated-norm measurements")
    ap.add_argument("--no-backward", action="store_true",
                    help="skip the gradient-pass measurement")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--cpu-pairs", type=int, default=0, help="oracle sample size (0: all)")
    ap.add_argument("--traffic-probe", action="store_true",
                    help="run a few scans and a plain copy of known size, for counter runs")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the scan is built and measured on a single "
              "MI355X (no multi-GPU path); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import mamba_ssd_chunked_chunk_amd as ssd
    import ssd_synth as syn

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    w = syn.WORKLOADS["mamba2_130m"]
    b, l, h, p, n, g, Q = w.batch, w.seqlen, w.heads, w.head_dim, w.state_dim, w.groups, w.chunk
    s = 2

    def t(a):
        if a is None:
            return None
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(dev)

    log("generating %d input sets of %s" % (args.sets, w))
    sets = []
    host0 = None
    for k in range(args.sets):
        inp = syn.make_inputs(w.replace(seed=w.seed + 1000 * k))
        if k == 0:
            host0 = inp
        sets.append(dict(x=t(inp["x"]), dt=t(inp["dt"]), A=t(inp["A"]), B=t(inp["B"]),
                         C=t(inp["C"]), D=t(inp["D"]), bias=t(inp["dt_bias"]),
                         y=torch.empty((b, l, h, p), dtype=torch.bfloat16, device=dev)))
    wsb = ssd.workspace_bytes(b, l, h, p, n, g, Q)
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev)

    def run(i):
        S = sets[i % len(sets)]
        ssd.chunk_scan(S["x"], S["dt"], S["A"], S["B"], S["C"], S["D"], chunk_size=Q,
                       dt_bias=S["bias"], out=S["y"], workspace=ws)

    log("warmup", args.warmup)
    for i in range(args.warmup):
        run(i)
    torch.cuda.synchronize()

    if args.traffic_probe:
        # three scans, three decode steps on a decode-shaped state, then the
        # calibration kernels: a 256 MiB fill (writes only) and a sum over the
        # same 256 MiB (reads only)
        for i in range(3):
            run(i)
        wd = syn.WORKLOADS["decode_2p7b"]
        gen = torch.Generator(device=dev)
        gen.manual_seed(wd.seed)
        st = torch.randn(wd.batch, wd.heads, wd.state_dim, wd.head_dim, generator=gen,
                         device=dev)
        Ad = -torch.rand(wd.heads, generator=gen, device=dev) - 0.5
        Dd = torch.ones(wd.heads, device=dev)
        yd = torch.empty(wd.batch, wd.heads, wd.head_dim, dtype=torch.bfloat16, device=dev)
        for _ in range(3):
            xd = torch.randn(wd.batch, wd.heads, wd.head_dim, generator=gen, device=dev).bfloat16()
            dtd = torch.randn(wd.batch, wd.heads, generator=gen, device=dev).bfloat16()
            Bd = torch.randn(wd.batch, wd.groups, wd.state_dim, generator=gen, device=dev).bfloat16()
            Cd = torch.randn(wd.batch, wd.groups, wd.state_dim, generator=gen, device=dev).bfloat16()
            ssd.step(st, xd, dtd, Ad, Bd, Cd, Dd, out=yd)
        torch.cuda.synchronize()
        cal = torch.empty(64 << 20, dtype=torch.float32, device=dev)
        for _ in range(3):
            cal.fill_(1.0)
        tot = 0.0
        for _ in range(3):
            tot += float(cal.sum())
        torch.cuda.synchronize()
        print(json.dumps({"traffic_probe": True, "calibration_bytes": cal.numel() * 4,
                          "check": tot}))
        return

    log("timed", args.steps, "steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        run(i)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / args.steps
    value = b * l * args.steps / (t1 - t0)
    log("scan: %.3f ms/step, %.4g tokens/s" % (ms_step, value))

    kern = kernel_times(ssd, torch, run, args.steps,
                        lambda name: bytes_kernel(name, b, l, h, p, n, g, Q, s))
    dom = max(kern, key=lambda k: kern[k]["avg_us"])
    dk = kern[dom]
    achieved = dk["alg_bytes"] / (dk["avg_us"] * 1e-6) / 1e9
    for name, v in kern.items():
        v["GBs"] = round(v["alg_bytes"] / (v["avg_us"] * 1e-6) / 1e9, 1)
        v["avg_us"] = round(v["avg_us"], 2)
    log("kernels:", json.dumps(kern))
    traffic = measured_traffic("k_" + dom, w.name)
    roofline = {"kernel": "k_" + dom, "bound": "hbm", "achieved": round(achieved, 1),
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": traffic, "alg_bytes_per_launch": dk["alg_bytes"],
                "avg_launch_us": dk["avg_us"]}
    balg = bytes_scan_alg(b, l, h, p, n, g, Q, s)
    bmin = bytes_scan_min(b, l, h, p, n, g, Q, s)
    t_roof = balg / (HBM_PEAK_GBS * 1e9)
    scan_roof = {"bound": "hbm", "alg_bytes": balg, "min_bytes": bmin,
                 "t_roof_us": round(t_roof * 1e6, 2), "t_step_us": round(ms_step * 1e3, 2),
                 "frac_alg": round(t_roof / (ms_step * 1e-3), 4),
                 "frac_min": round(bmin / (HBM_PEAK_GBS * 1e9) / (ms_step * 1e-3), 4),
                 "kernels": kern}

    states = None
    if not args.no_states:
        states = bench_states(args, torch, ssd, np, sets, ws, w, dev)

    neighbors = None
    if not args.no_neighbors:
        neighbors = bench_neighbors(args, torch, ssd, syn, np, dev)

    backward = None
    if not args.no_backward:
        backward = bench_backward(args, torch, ssd, np, sets, w, dev)

    decode = None
    if not args.no_decode:
        decode = bench_decode(args, torch, ssd, syn, dev)

    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(args, host0, w)

    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) x/B/C/dt, A=-exp(U[0,ln16]), "
                "dt_bias=softplus^-1(loguniform[1e-3,0.1]), D=1, zero initial state)",
        "config": {"workload": "mamba2_130m", "batch": b, "seqlen": l, "heads": h,
                   "head_dim": p, "state_dim": n, "groups": g, "chunk": Q, "io": "bf16",
                   "state": "fp32", "input_sets": args.sets},
        "roofline": roofline,
        "scan_roofline": scan_roof,
        "states": states,
        "neighbors": neighbors,
        "backward": backward,
        "decode": decode,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out))


def kernel_times(ssd, torch, run, steps, alg_bytes):
    """Average duration of each scan kernel over `steps` calls of run(i),
    from HIP events the library records on its launch stream, with the
    kernel's algorithmic bytes and the rate they imply."""
    ssd.trace_enable(True)
    for name in KERNEL_IDS:
        ssd.trace_read(name)
    torch.cuda.synchronize()
    for i in range(steps):
        run(i)
    torch.cuda.synchronize()
    ssd.trace_enable(False)
    kern = {}
    for name in KERNEL_IDS:
        tot, cnt = ssd.trace_read(name)
        if cnt:
            kern[name] = dict(avg_us=1e3 * tot / cnt, launches=cnt, alg_bytes=alg_bytes(name))
    return kern


def doc_index(np, rng, b, l, lo=32, hi=2048):
    """Document index of packed rows: documents back to back, lengths
    log-uniform in [lo, hi] tokens, the last one cut at the row's end."""
    seq = np.zeros((b, l), np.int32)
    for bi in range(b):
        t = k = 0
        while t < l:
            m = int(round(math.exp(rng.uniform(math.log(lo), math.log(hi)))))
            seq[bi, t:t + m] = k
            t += m
            k += 1
    return seq


def bench_states(args, torch, ssd, np, sets, ws, w, dev):
    """The scan with packed documents (a per-token document index) and with
    the state after every chunk written, on the same workload and input sets
    as the headline; and the state after every token (chunk 1) on one batch
    row of it."""
    b, l, h, p, n, g, Q = w.batch, w.seqlen, w.heads, w.head_dim, w.state_dim, w.groups, w.chunk
    s = 2
    nc, _ = plan_sizes(b, l, h, p, n, g, Q)
    rng = np.random.default_rng(w.seed + 77)
    seqs = [torch.from_numpy(doc_index(np, rng, b, l)).to(dev) for _ in sets]
    docs = sum(int(q[:, -1].sum()) + b for q in seqs) / len(seqs)
    st_out = torch.empty((b, nc, h, n, p), dtype=torch.float32, device=dev)
    steps = max(args.steps // 2, 10)

    def measure(tag, run, alg_extra):
        for i in range(5):
            run(i)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            run(i)
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) * 1e3 / steps
        kern = kernel_times(ssd, torch, run, steps,
                            lambda k: bytes_kernel(k, b, l, h, p, n, g, Q, s,
                                                   states=tag == "chunk_states")
                            + alg_extra.get(k, 0))
        for v in kern.values():
            v["GBs"] = round(v["alg_bytes"] / (v["avg_us"] * 1e-6) / 1e9, 1)
            v["avg_us"] = round(v["avg_us"], 2)
        log("%s: %.4f ms/step %s" % (tag, ms, json.dumps(kern)))
        return {"value": round(b * l / (ms * 1e-3), 1), "unit": "tokens/s",
                "ms_per_step": round(ms, 4), "kernels": kern}

    def run_packed(i):
        S = sets[i % len(sets)]
        ssd.chunk_scan(S["x"], S["dt"], S["A"], S["B"], S["C"], S["D"], chunk_size=Q,
                       dt_bias=S["bias"], out=S["y"], workspace=ws, seq_idx=seqs[i % len(seqs)])

    def run_states(i):
        S = sets[i % len(sets)]
        ssd.chunk_scan(S["x"], S["dt"], S["A"], S["B"], S["C"], S["D"], chunk_size=Q,
                       dt_bias=S["bias"], out=S["y"], workspace=ws,
                       return_chunk_states=True, chunk_states_out=st_out)

    # the document index is read by the chunk-state pass and the chunk output
    # (4 bytes per token each); every chunk's state is written once (fp32)
    packed = measure("packed", run_packed, {"chunk_state": 4 * b * l, "chunk_out": 4 * b * l})
    packed["documents_per_step"] = round(docs, 1)
    packed["doc_lengths"] = "log-uniform in [32, 2048] tokens, seeded"
    chunks = measure("chunk_states", run_states, {})

    # the state after every token: chunk 1, one batch row, each token's
    # state written in fp32 (the rate that bounds this mode)
    S = sets[0]
    x1, dt1, B1, C1 = S["x"][:1], S["dt"][:1], S["B"][:1], S["C"][:1]
    y1 = torch.empty((1, l, h, p), dtype=torch.bfloat16, device=dev)
    tok_states = torch.empty((1, l, h, n, p), dtype=torch.float32, device=dev)
    ws1 = torch.empty(ssd.workspace_bytes(1, l, h, p, n, g, 1), dtype=torch.uint8, device=dev)

    def run_tok(i):
        ssd.chunk_scan(x1, dt1, S["A"], B1, C1, S["D"], chunk_size=1, dt_bias=S["bias"],
                       out=y1, workspace=ws1, return_chunk_states=True,
                       chunk_states_out=tok_states)
    for i in range(3):
        run_tok(i)
    torch.cuda.synchronize()
    nt = max(steps // 10, 5)
    t0 = time.perf_counter()
    for i in range(nt):
        run_tok(i)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / nt
    wbytes = l * h * n * p * 4
    log("per-token states: %.3f ms per row, %.0f GB/s of state written" %
        (ms, wbytes / (ms * 1e-3) / 1e9))
    per_token = {"value": round(l / (ms * 1e-3), 1), "unit": "tokens/s", "ms_per_call": round(ms, 4),
                 "config": {"batch": 1, "seqlen": l, "heads": h, "chunk": 1},
                 "state_bytes_written": wbytes,
                 "state_write_GBs": round(wbytes / (ms * 1e-3) / 1e9, 1)}
    return {"packed": packed, "chunk_states": chunks, "per_token": per_token}


def bench_neighbors(args, torch, ssd, syn, np, dev):
    """The steps around the scan at the 130m mixer's shape (8 x 2048 tokens,
    24 heads of 64, state 128, 1 group, bf16): the width-4 causal conv1d +
    SiLU + split of the 1792 projection channels, and the silu(z) gate with
    one RMS norm over the 1536 channels.  Each is one pass over HBM; its
    rate is priced on those bytes."""
    b, l, h, p, n, g, K = 8, 2048, 24, 64, 128, 1, 4
    ch = h * p + 2 * g * n
    steps = max(args.steps // 2, 10)
    sets = []
    for k in range(2):
        c = syn.conv_case(900 + k, b, l, h, p, n, g, K, io="bf16", with_init=False)
        nc = syn.norm_case(950 + k, b * l, h * p, io="bf16")

        def t16(a):
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        sets.append(dict(xbc=t16(c["xbc"]), w=torch.from_numpy(c["weight"]).to(dev),
                         bias=torch.from_numpy(c["bias"]).to(dev), y=t16(nc["y"]), z=t16(nc["z"]),
                         nw=torch.from_numpy(nc["weight"]).to(dev),
                         out=(torch.empty((b, l, h, p), dtype=torch.bfloat16, device=dev),
                              torch.empty((b, l, g, n), dtype=torch.bfloat16, device=dev),
                              torch.empty((b, l, g, n), dtype=torch.bfloat16, device=dev)),
                         nout=torch.empty((b * l, h * p), dtype=torch.bfloat16, device=dev)))

    def conv(i):
        S = sets[i % 2]
        ssd.conv1d_silu(S["xbc"], S["w"], h, p, n, g, bias=S["bias"], out=S["out"])

    def norm(i):
        S = sets[i % 2]
        ssd.gated_norm(S["y"], S["z"], S["nw"], eps=1e-5, out=S["nout"])

    res = {}
    for name, fn, tid, alg in (
            ("conv1d_silu", conv, "conv1d", 2 * b * l * ch * 2 + ch * (K + 1) * 4),
            ("gated_norm", norm, "gated_norm", 3 * b * l * h * p * 2 + h * p * 4)):
        for i in range(5):
            fn(i)
        torch.cuda.synchronize()
        ssd.trace_enable(True)
        ssd.trace_read(tid)
        for i in range(steps):
            fn(i)
        torch.cuda.synchronize()
        ssd.trace_enable(False)
        tot, cnt = ssd.trace_read(tid)
        us = 1e3 * tot / cnt
        gbs = alg / (us * 1e-6) / 1e9
        log("%s: %.2f us, %.0f GB/s" % (name, us, gbs))
        res[name] = {"avg_launch_us": round(us, 2), "alg_bytes_per_launch": alg,
                     "tokens_per_s": round(b * l / (us * 1e-6), 1),
                     "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                                  "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4)}}
    res["config"] = {"workload": "mamba2_130m mixer", "batch": b, "seqlen": l, "heads": h,
                     "head_dim": p, "state_dim": n, "groups": g, "conv_width": K,
                     "norm_groups": 1, "io": "bf16"}
    return res


def bench_backward(args, torch, ssd, np, sets, w, dev):
    """The gradient pass (ssd_chunk_scan_bwd) on the headline workload and
    input sets, with a final-state cotangent: tokens/s, and the call's time
    against the bytes any gradient pass must move (inputs x, dt, B, C, dy
    read once; dx, ddt, dB, dC written once; the final-state cotangent and
    d init once)."""
    b, l, h, p, n, g, Q = w.batch, w.seqlen, w.heads, w.head_dim, w.state_dim, w.groups, w.chunk
    gen = torch.Generator(device=dev)
    gen.manual_seed(w.seed + 99)
    dys = [torch.randn((b, l, h, p), generator=gen, device=dev).bfloat16() for _ in sets]
    dfin = torch.randn((b, h, n, p), generator=gen, device=dev)
    wsb = int(ssd._lib.load().ssd_chunk_scan_bwd_workspace_bytes(b, l, h, p, n, g, Q))
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
    steps = max(args.steps // 10, 5)

    def run(i):
        S = sets[i % len(sets)]
        ssd.chunk_scan_bwd(S["x"], S["dt"], S["A"], S["B"], S["C"], dys[i % len(dys)], D=S["D"],
                           chunk_size=Q, dt_bias=S["bias"], d_final=dfin, workspace=ws)
    for i in range(3):
        run(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        run(i)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    s = 2
    min_bytes = (2 * (2 * b * l * h * p * s + 2 * b * l * g * n * s + b * l * h * s)
                 + 2 * b * h * n * p * 4)
    gbs = min_bytes / (ms * 1e-3) / 1e9
    log("backward: %.3f ms per call, %.4g tokens/s, %.0f GB/s on the minimal bytes" %
        (ms, b * l / (ms * 1e-3), gbs))
    return {"metric": "gradient pass tokens/s", "value": round(b * l / (ms * 1e-3), 1),
            "unit": "tokens/s", "ms_per_call": round(ms, 4), "calls": steps,
            "workspace_bytes": wsb, "min_bytes": min_bytes,
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4)},
            "config": {"workload": "mamba2_130m", "io": "bf16", "d_final": True,
                       "deterministic": True}}


def bench_decode(args, torch, ssd, syn, dev):
    """Decode steps/s: batch 256, 80 heads, head_dim 64, state 128, bf16 io,
    fp32 state initialised by a 1024-token chunk-scan prefill."""
    w = syn.WORKLOADS["decode_2p7b"]
    b, l, h, p, n, g = w.batch, w.seqlen, w.heads, w.head_dim, w.state_dim, w.groups
    head = syn.make_inputs(w.replace(seqlen=1), batch=1)
    A = torch.from_numpy(head["A"]).to(dev)
    D = torch.from_numpy(head["D"]).to(dev)
    bias = torch.from_numpy(head["dt_bias"]).to(dev)
    gen = torch.Generator(device=dev)
    gen.manual_seed(w.seed)

    def rnd(*shape):
        return torch.randn(*shape, generator=gen, device=dev, dtype=torch.float32).bfloat16()

    log("decode prefill", b, "x", l)
    x, dt, B, C = rnd(b, l, h, p), rnd(b, l, h), rnd(b, l, g, n), rnd(b, l, g, n)
    _, st = ssd.chunk_scan(x, dt, A, B, C, D, chunk_size=w.chunk, dt_bias=bias,
                           return_final_state=True)
    del x, dt, B, C
    K = args.decode_steps
    xs, dts, Bs, Cs = rnd(K, b, h, p), rnd(K, b, h), rnd(K, b, g, n), rnd(K, b, g, n)
    y = torch.empty((b, h, p), dtype=torch.bfloat16, device=dev)
    for k in range(3):
        ssd.step(st, xs[k], dts[k], A, Bs[k], Cs[k], D, dt_bias=bias, out=y)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(K):
        ssd.step(st, xs[k], dts[k], A, Bs[k], Cs[k], D, dt_bias=bias, out=y)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    rate = K / (t1 - t0)
    ssd.trace_enable(True)
    ssd.trace_read("step")
    for k in range(K):
        ssd.step(st, xs[k], dts[k], A, Bs[k], Cs[k], D, dt_bias=bias, out=y)
    torch.cuda.synchronize()
    ssd.trace_enable(False)
    tot, cnt = ssd.trace_read("step")
    avg_us = 1e3 * tot / cnt
    alg = bytes_step(b, h, p, n, g, 2)
    achieved = alg / (avg_us * 1e-6) / 1e9
    log("decode: %.1f steps/s, kernel %.2f us, %.0f GB/s" % (rate, avg_us, achieved))
    return {"metric": "decode steps/s", "value": round(rate, 1), "unit": "steps/s",
            "tokens_per_s": round(rate * b, 1), "steps": K,
            "config": {"workload": "decode_2p7b", "batch": b, "heads": h, "head_dim": p,
                       "state_dim": n, "groups": g, "io": "bf16", "state": "fp32",
                       "prefill_tokens": l},
            "roofline": {"kernel": "k_step", "bound": "hbm", "achieved": round(achieved, 1),
                         "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(achieved / HBM_PEAK_GBS, 4),
                         "traffic": measured_traffic("k_step", "decode_2p7b"),
                         "alg_bytes_per_launch": alg, "avg_launch_us": round(avg_us, 2)}}


def cpu_baseline(args, inp, w, min_seconds=10.0, max_passes=500):
    """The fp64 oracle on the host cores over the same workload (all its
    (batch, head) pairs and tokens), repeated until about min_seconds of wall
    time have passed, reported in tokens/s (a token being one position across
    all heads)."""
    import oracle
    oracle.build()
    pairs_all = [(bb, hh) for bb in range(w.batch) for hh in range(w.heads)]
    k = args.cpu_pairs or len(pairs_all)
    pairs = pairs_all[:k]
    cores = oracle.default_threads()
    log("oracle on %d pairs, %d threads, >= %.0f s" % (len(pairs), cores, min_seconds))
    passes = 0
    t0 = time.perf_counter()
    while passes < max_passes:
        oracle.scan(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp["D"],
                    inp["dt_bias"], io=inp["io"], pairs=pairs, nthreads=cores)
        passes += 1
        if time.perf_counter() - t0 >= min_seconds:
            break
    dt_s = time.perf_counter() - t0
    tok = passes * len(pairs) * w.seqlen / w.heads
    log("oracle: %d passes in %.2f s" % (passes, dt_s))
    return {"value": round(tok / dt_s, 1), "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": "%d pass(es) over %d of %d (batch, head) pairs x %d tokens of the "
                      "mamba2_130m workload, %.1f s wall" % (passes, len(pairs),
                                                             len(pairs_all), w.seqlen, dt_s)}


if __name__ == "__main__":
    main()
