"""GPU parity of the gradient pass (ssd_chunk_scan_bwd, through the C ABI)
against the fp64 gradient oracle (oracle/backward.py), and its
determinism."""
import math

import numpy as np
import pytest

import ssd_synth as syn
from gpu_util import STATE_AXES, Y_AXES, check_close, dev_tensor, gpu_inputs, log, to_f64, torch_mod

pytestmark = pytest.mark.gpu


def _seq(b, l, cuts_per_row):
    seq = np.zeros((b, l), np.int32)
    for bi, cuts in enumerate(cuts_per_row):
        for k, c in enumerate(cuts):
            seq[bi, c:] = 10 * (k + 1) + bi
    return seq


def _run(inp, cot, Q, seq=None, d_final=True, limit=(0.0, math.inf)):
    import mamba_ssd_chunked_chunk_amd as ssd
    torch = torch_mod()
    g = gpu_inputs(inp)
    sq = None if seq is None else torch.from_numpy(seq).to("cuda")
    out = ssd.chunk_scan_bwd(g["x"], g["dt"], g["A"], g["B"], g["C"], dev_tensor(cot["dy"]),
                             D=g["D"], chunk_size=Q, dt_bias=g["dt_bias"],
                             initial_state=g["init"],
                             d_final=dev_tensor(cot["d_final"]) if d_final else None,
                             dt_limit=limit, seq_idx=sq)
    torch.cuda.synchronize()
    return out


def _oracle(inp, cot, seq=None, d_final=True, limit=(0.0, math.inf)):
    from oracle import backward as bw
    io = inp["io"]
    f = lambda a: syn.as_f32(a, io)   # noqa: E731
    return bw.scan_grad(f(inp["x"]), f(inp["dt"]), inp["A"], f(inp["B"]), f(inp["C"]), inp["D"],
                        inp["dt_bias"], dt_limit=limit, init_state=inp["init_state"],
                        seq_idx=seq, dy=f(cot["dy"]),
                        d_final=cot["d_final"] if d_final else None)


AXES = dict(dx=Y_AXES, ddt=(1,), dB=Y_AXES, dC=Y_AXES, dA=None, dD=None, d_dt_bias=None,
            d_init=STATE_AXES)


# The time-step and decay gradients come from a reverse running sum of
# per-token terms u - v over a whole document, each term from an fp32 scan
# (relative error ~5e-6, the forward's own worst case); the sum's error grows
# like sqrt(tokens) * 5e-6 * |u|, with |u| up to ~10x the gradient's scale:
# ~1e-3 of the (batch, head)'s rms at a few hundred tokens.  fp32 io takes
# that rms floor on these three; bf16 io already has a 2e-2 floor.
FLOOR = dict(ddt=1e-3, dA=1e-3, d_dt_bias=1e-3)


def _compare(gpu, ref, io):
    for k, v in gpu.items():
        s = check_close(to_f64(v), ref[k], io, k, AXES[k],
                        floor=FLOOR.get(k) if io == "f32" else None)
        log("%s max_abs %.3g max_rel %.3g" % (k, s[0], s[1]))


# (batch, seqlen, heads, head_dim, state_dim, groups, chunk, init_std, d_final, resets per row)
BWD = [
    (2, 70, 4, 32, 32, 2, 32, 0.3, True, [(5, 40), ()]),
    (1, 130, 2, 64, 64, 1, 64, 0.0, False, [()]),
    (2, 100, 4, 64, 128, 1, 50, 0.2, False, [(33,), (1, 99)]),
    (1, 64, 2, 128, 32, 2, 16, 0.0, True, [()]),          # chunk below one block
    (1, 300, 3, 32, 64, 3, 256, 0.1, True, [(100, 101)]),  # one-token document
]


def _bid(c):
    return "b%d_l%d_h%d_p%d_n%d_g%d_Q%d" % c[:7]


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("case", BWD, ids=_bid)
def test_gradients_parity(case, io):
    b, l, h, p, n, g, Q, init, dfin, cuts = case
    inp = syn.random_case(5000 + sum(case[:7]), b, l, h, p, n, g, io=io, init_std=init)
    cot = syn.cotangent_case(5100 + sum(case[:7]), b, l, h, p, n, io=io)
    seq = _seq(b, l, cuts) if any(cuts) else None
    gpu = _run(inp, cot, Q, seq=seq, d_final=dfin)
    _compare(gpu, _oracle(inp, cot, seq=seq, d_final=dfin), io)


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_gradients_with_time_step_limit(io):
    """A clamp that binds on part of the tokens stops their time-step gradient."""
    inp = syn.random_case(5200, 2, 80, 4, 32, 64, 2, io=io, init_std=0.2)
    cot = syn.cotangent_case(5201, 2, 80, 4, 32, 64, io=io)
    lim = (0.004, 0.05)
    _compare(_run(inp, cot, 64, limit=lim), _oracle(inp, cot, limit=lim), io)


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_gradients_deterministic(io):
    """The same inputs give the same bits, call after call."""
    inp = syn.random_case(5300, 2, 300, 8, 64, 128, 2, io=io, init_std=0.2)
    cot = syn.cotangent_case(5301, 2, 300, 8, 64, 128, io=io)
    seq = _seq(2, 300, [(77, 200), ()])
    a = _run(inp, cot, 256, seq=seq)
    torch = torch_mod()
    for _ in range(2):
        bb = _run(inp, cot, 256, seq=seq)
        for k in a:
            assert torch.equal(a[k], bb[k]), k


# edge shapes: one token, fewer tokens than a chunk, one group per head,
# a document at every token, a long row at the bench head shape
EDGE = [
    (1, 1, 2, 32, 32, 1, 64, 0.3, True, [()]),
    (2, 20, 4, 64, 64, 4, 256, 0.0, True, [(), ()]),
    (1, 40, 2, 32, 32, 1, 32, 0.2, True, [tuple(range(1, 40))]),
    (1, 2048, 4, 64, 128, 1, 256, 0.1, True, [(700, 1500)]),
]


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("case", EDGE, ids=_bid)
def test_gradients_edge_shapes(case, io):
    b, l, h, p, n, g, Q, init, dfin, cuts = case
    inp = syn.random_case(5400 + sum(case[:7]), b, l, h, p, n, g, io=io, init_std=init)
    cot = syn.cotangent_case(5500 + sum(case[:7]), b, l, h, p, n, io=io)
    seq = _seq(b, l, cuts) if any(cuts) else None
    gpu = _run(inp, cot, Q, seq=seq, d_final=dfin)
    _compare(gpu, _oracle(inp, cot, seq=seq, d_final=dfin), io)


def test_gradients_joined_chunks():
    """A grid large enough that the bf16 pass stores its states every 2 of
    the caller's chunks in the adjoint scans (whose transposed one reads the
    other's states) and computes the transposed forward scan (one head per
    workgroup, four times the items) as one chunk per sequence: batch sized
    from the device's compute units; two batch rows (every head, so the
    group sums of dB and dC are whole) against the oracle run on those
    rows."""
    import mamba_ssd_chunked_chunk_amd as ssd
    torch = torch_mod()
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    l, h, p, n, g, Q = 2048, 16, 32, 64, 2, 256
    b = 3 * cus // ((l // Q // 2) * (h // 4))
    assert ssd.state_chunks(b, l, h, p, n, g, Q, io="bf16") == l // Q // 2
    inp = syn.random_case(5600, b, l, h, p, n, g, io="bf16", init_std=0.2)
    cot = syn.cotangent_case(5601, b, l, h, p, n, io="bf16")
    gpu = _run(inp, cot, Q)
    rows = [0, b - 1]
    sub = dict(inp)
    for k in ("x", "dt", "B", "C", "init_state"):
        sub[k] = inp[k][rows]
    csub = dict(dy=cot["dy"][rows], d_final=cot["d_final"][rows], io=cot["io"])
    ref = _oracle(sub, csub)
    for k in ("dx", "ddt", "dB", "dC", "d_init"):
        v = gpu[k][rows]
        s = check_close(to_f64(v), ref[k], "bf16", k, AXES[k])
        log("joined %s max_abs %.3g max_rel %.3g" % (k, s[0], s[1]))
