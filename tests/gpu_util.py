"""Helpers for the GPU parity tests: device transfer, the tolerance bar, and
sampled oracle comparisons.

Tolerance bar (elementwise, for y and for states):
  fp32 io:  |g - o| <= 1e-4 + 1e-4 |o|
  bf16 io:  |g - o| <= 2e-2 |o| + 2e-2 rms(o), asserted twice: with rms over
            the whole compared tensor, and with rms over each (batch, head)'s
            values (every head is its own recurrence: nnterp guide, "Mamba-2"
            page, opening section), so every element meets the stricter of
            the two floors.
with o the fp64 oracle value.  The pages' own step-vs-forward differences
(5.07e-5 in fp32 and 7.81e-3 in bf16 on an RTX 4090; mirror of
state-spaces/mamba issue 1024, "Mamba3 step() is non-deterministic ...")
sit inside these bounds.
"""
from __future__ import annotations

import math
import sys

import numpy as np

import ssd_synth as syn


def log(*a):
    print("[gpu-test]", *a, file=sys.stderr, flush=True)


def torch_mod():
    import torch
    return torch


def dev_tensor(a, io=None):
    """numpy -> cuda tensor; uint16 arrays are bf16 bit patterns."""
    torch = torch_mod()
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        t = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(a.astype(np.float32, copy=False))
    return t.to("cuda")


def to_f64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def bar(io):
    return (1e-4, 1e-4, 0.0) if io == "f32" else (0.0, 2e-2, 2e-2)


def check_close(g, o, io, what, rms_axes=None, floor=None):
    """Assert the elementwise bar; return (max_abs, max_rel, normwise).

    rms_axes: the axes that do NOT index a (batch, head) pair; with bf16 io
    the rms floor is then asserted both over the whole tensor and per pair
    (None: over the whole tensor only).  floor: the rms floor's factor
    instead of the io type's (the fp32 gradient terms that come out of a
    running sum)."""
    g = np.asarray(g, np.float64)
    o = np.asarray(o, np.float64)
    assert g.shape == o.shape, (what, g.shape, o.shape)
    assert np.isfinite(g).all(), "%s: non-finite values" % what
    atol, rtol, rmsf = bar(io)
    if floor is not None:
        rmsf = floor
    if o.size == 0:
        return (0.0, 0.0, 0.0)
    err = np.abs(g - o)
    rms_t = np.sqrt(np.mean(o * o))
    floors = [("tensor", rms_t)]
    if rms_axes is not None:
        floors.append(("head", np.sqrt(np.mean(o * o, axis=rms_axes, keepdims=True))))
    for kind, rms in floors:
        lim = atol + rtol * np.abs(o) + rmsf * rms
        bad = err > lim
        if bad.any():
            idx = np.unravel_index(np.argmax(err - lim), err.shape)
            raise AssertionError(
                "%s: %d of %d elements outside the %s bar (rms floor per %s); worst at %s: "
                "gpu %r oracle %r" % (what, int(bad.sum()), bad.size, io, kind, idx, g[idx], o[idx]))
        WORST.setdefault((what, kind), 0.0)
        if rmsf > 0:
            WORST[(what, kind)] = max(WORST[(what, kind)],
                                      float(np.max(err / (np.abs(o) + rms + 1e-300))))
    rms = rms_t
    den = np.maximum(np.abs(o), rms if rms > 0 else 1e-300)
    return (float(err.max()), float((err / den).max()),
            float(err.max() / max(np.abs(o).max(), 1e-300)))


# worst err / (|o| + rms) seen per (what, floor kind) in this process, for
# the logs
WORST = {}


# rms axes per layout: everything except the (batch, head) indices
Y_AXES = (1, 3)        # y [b, l, h, p]
STATE_AXES = (2, 3)    # state [b, h, n, p]
PAIR_AXES = (1, 2)     # per-pair stacks [k, l, p] / [k, n, p]


def gpu_inputs(inp):
    return dict(x=dev_tensor(inp["x"]), dt=dev_tensor(inp["dt"]), A=dev_tensor(inp["A"]),
                B=dev_tensor(inp["B"]), C=dev_tensor(inp["C"]), D=dev_tensor(inp["D"]),
                dt_bias=dev_tensor(inp["dt_bias"]),
                init=dev_tensor(inp["init_state"]) if inp["init_state"] is not None else None)


def run_scan(inp, chunk, final=True, dt_limit=(0.0, math.inf), dt_softplus=True, g=None):
    import mamba_ssd_chunked_chunk_amd as ssd
    torch = torch_mod()
    g = g or gpu_inputs(inp)
    out = ssd.chunk_scan(g["x"], g["dt"], g["A"], g["B"], g["C"], g["D"], chunk_size=chunk,
                         dt_bias=g["dt_bias"], dt_softplus=dt_softplus, dt_limit=dt_limit,
                         initial_state=g["init"], return_final_state=final)
    torch.cuda.synchronize()
    return out


def oracle_kw(inp, **over):
    kw = dict(x=inp["x"], dt=inp["dt"], A=inp["A"], B=inp["B"], C=inp["C"], D=inp["D"],
              dt_bias=inp["dt_bias"], init_state=inp["init_state"], io=inp["io"])
    kw.update(over)
    return kw


def sample_pairs(b, h, k, seed=0):
    """k (batch, head) pairs: the corners plus a seeded spread."""
    pairs = {(0, 0), (b - 1, h - 1), (0, h - 1), (b - 1, 0)}
    rng = np.random.default_rng(seed)
    while len(pairs) < min(k, b * h):
        pairs.add((int(rng.integers(b)), int(rng.integers(h))))
    return sorted(pairs)
