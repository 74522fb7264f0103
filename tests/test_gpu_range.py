"""GPU parity over the whole bf16 value range.

The bf16 path multiplies the inputs x, B and C on the matrix cores exactly
as given and splits every operand it forms (weighted x, masked scores,
carried state) into two bf16 terms, so any finite bf16 input is in its
domain, including magnitudes far outside fp16's.  The stored chunk and
boundary states carry a power-of-two scale, so states beyond 65504 or
below 2^-100 keep their precision.  Each case is checked element by
element against the fp64 oracle with the bf16 bar (both rms floors).

Values the pages fix: the recurrence and its tensor contract (nnterp guide,
"Mamba-2" page, opening section and "The values": bf16 io tensors, fp32
states).
"""
import math

import numpy as np
import pytest

import ssd_synth as syn
from gpu_util import (STATE_AXES, WORST, Y_AXES, check_close, log, oracle_kw, run_scan, to_f64,
                      torch_mod)

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _name(request):
    log("start", request.node.nodeid)
    yield


@pytest.fixture(scope="module")
def orc():
    import oracle
    oracle.build()
    return oracle


def _scaled(inp, sx, sB, sC):
    """The case with x, B, C multiplied by powers of two (exact in bf16 while
    the results stay inside bf16's range) and the initial state by sx sB."""
    out = dict(inp)
    for k, s in (("x", sx), ("B", sB), ("C", sC)):
        out[k] = syn.bf16_round(syn.as_f32(inp[k], "bf16") * np.float32(s))
    if inp["init_state"] is not None:
        out["init_state"] = (inp["init_state"] * np.float32(sx * sB)).astype(np.float32)
    return out


# (x, B, C) scales: all above fp16's largest value or below its smallest
# normal, and mixtures of both
SCALES = [(2.0 ** 12, 2.0 ** 12, 2.0 ** 12), (2.0 ** -16, 2.0 ** -16, 2.0 ** -16),
          (2.0 ** 20, 2.0 ** -20, 2.0 ** 10), (2.0 ** -30, 2.0 ** 25, 2.0 ** -5),
          (2.0 ** 40, 1.0, 2.0 ** -40)]


@pytest.mark.parametrize("scales", SCALES, ids=lambda s: "x%g_B%g_C%g" % tuple(math.log2(v) for v in s))
@pytest.mark.parametrize("shape", [(2, 600, 8, 64, 128, 2, 256), (1, 300, 4, 32, 64, 1, 100)],
                         ids=lambda s: "b%dl%dh%dp%dn%dg%dQ%d" % s)
def test_bf16_inputs_outside_fp16_range(orc, scales, shape):
    b, l, h, p, n, g, Q = shape
    inp = _scaled(syn.random_case(4100 + l, b, l, h, p, n, g, io="bf16", init_std=0.1), *scales)
    WORST.clear()
    y, fin = run_scan(inp, Q)
    yo, fo = orc.scan(**oracle_kw(inp))
    check_close(to_f64(y), yo, "bf16", "y", Y_AXES)
    check_close(to_f64(fin), fo, "bf16", "final_state", STATE_AXES)
    log("scales", scales, "worst err/(|o|+rms):", {"%s/%s" % k: "%.2e" % v for k, v in WORST.items()})


@pytest.mark.parametrize("init_std", [0.0, 1.0e5])
def test_states_beyond_fp16(orc, init_std):
    """A = 0 (causal linear attention: nothing decays) over 4096 tokens, and
    an initial state of order 1e5: the boundary states far exceed 65504."""
    b, l, h, p, n, g, Q = 1, 4096, 4, 64, 128, 1, 256
    inp = syn.random_case(4200, b, l, h, p, n, g, io="bf16", init_std=init_std)
    inp["A"] = np.zeros_like(inp["A"])
    # no decay and large steps: d = 2 for every token (no softplus, no bias)
    inp["dt"] = syn.bf16_round(np.full((b, l, h), 2.0, np.float32))
    inp["dt_bias"] = np.zeros_like(inp["dt_bias"])
    inp["x"] = syn.bf16_round(syn.as_f32(inp["x"], "bf16") * np.float32(1024.0))
    y, fin = run_scan(inp, Q, dt_softplus=False, dt_limit=(-math.inf, math.inf))
    assert float(fin.abs().max()) > 4 * 65504.0
    yo, fo = orc.scan(**oracle_kw(inp), dt_softplus=False, dt_limit=(-math.inf, math.inf))
    check_close(to_f64(y), yo, "bf16", "y", Y_AXES)
    check_close(to_f64(fin), fo, "bf16", "final_state", STATE_AXES)


def test_chunk_state_far_below_one(orc):
    """Chunks of 512 tokens whose last 256 carry x = 0 and a total log2 decay
    of about -120 over those rows: each chunk's own state ends near 2^-120 of
    its size after the first half (scale exponent clamped at 2^-100, so no
    inf or NaN), and the output still meets the bar."""
    b, l, h, p, n, g, Q = 1, 2048, 4, 64, 128, 1, 512
    inp = syn.random_case(4300, b, l, h, p, n, g, io="bf16", init_std=0.0)
    inp["A"] = np.full(h, -16.0, np.float32)
    # d = 0.0203 per token (no softplus, no bias): 256 tokens give
    # A d 256 log2(e) ~ -120
    inp["dt"] = syn.bf16_round(np.full((b, l, h), 0.0203, np.float32))
    inp["dt_bias"] = np.zeros_like(inp["dt_bias"])
    x = syn.as_f32(inp["x"], "bf16").copy()
    for c0 in range(0, l, Q):
        x[:, c0 + Q // 2: c0 + Q] = 0.0
    inp["x"] = syn.bf16_round(x)
    y, fin = run_scan(inp, Q, dt_softplus=False, dt_limit=(-math.inf, math.inf))
    torch = torch_mod()
    assert bool(torch.isfinite(y.float()).all()) and bool(torch.isfinite(fin).all())
    yo, fo = orc.scan(**oracle_kw(inp), dt_softplus=False, dt_limit=(-math.inf, math.inf))
    check_close(to_f64(y), yo, "bf16", "y", Y_AXES)
    check_close(to_f64(fin), fo, "bf16", "final_state", STATE_AXES)


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_kernel_events_time_each_kernel(orc, io):
    """Caller-owned events passed as kernel_events receive every launched
    kernel's start and end; the results are the same bits as without."""
    import mamba_ssd_chunked_chunk_amd as ssd
    torch = torch_mod()
    b, l, h, p, n, g, Q = 2, 1000, 8, 64, 128, 1, 256
    inp = syn.random_case(4400, b, l, h, p, n, g, io=io, init_std=0.1)
    y0, f0 = run_scan(inp, Q)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(8)]
    for e in evs:
        e.record()
    torch.cuda.synchronize()
    from gpu_util import gpu_inputs
    G = gpu_inputs(inp)
    y1, f1 = ssd.chunk_scan(G["x"], G["dt"], G["A"], G["B"], G["C"], G["D"], chunk_size=Q,
                            dt_bias=G["dt_bias"], initial_state=G["init"],
                            return_final_state=True,
                            kernel_events=[e.cuda_event for e in evs])
    torch.cuda.synchronize()
    assert torch.equal(y0, y1) and torch.equal(f0, f1)
    ms = [evs[2 * k].elapsed_time(evs[2 * k + 1]) for k in range(3)]
    log("kernel ms:", ms)
    assert all(0.0 < v < 1e3 for v in ms), ms
