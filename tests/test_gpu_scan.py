"""GPU parity of ssd_chunk_scan against the fp64 oracle (through the C ABI).

Small cases compare every output element; they span several row blocks and
chunks, ragged last chunks, chunk lengths below / not a multiple of the row
block, grouped B/C, initial states and both io dtypes.  Workload-sized
cases are in test_gpu_workloads.py.
"""
import math

import numpy as np
import pytest

import ssd_synth as syn
from gpu_util import (STATE_AXES, Y_AXES, check_close, gpu_inputs, log, oracle_kw, run_scan,
                      to_f64, torch_mod)

pytestmark = pytest.mark.gpu

# (batch, seqlen, heads, head_dim, state_dim, groups, chunk, init_std)
SMALL = [
    (1, 256, 24, 64, 128, 1, 64, 0.0),    # the tiny fp32 workload's shape
    (2, 77, 4, 64, 128, 2, 64, 0.1),      # ragged last chunk, groups
    (1, 10, 8, 16, 64, 1, 16, 0.0),       # head_dim 16, state 64, chunk 16, 10 tokens
    (2, 300, 6, 32, 64, 3, 100, 0.5),     # chunk not a multiple of the row block
    (1, 129, 2, 128, 128, 1, 256, 0.1),   # sequence shorter than a chunk, head_dim 128
    (3, 40, 4, 64, 32, 4, 1, 0.2),        # one token per chunk
    (2, 1, 4, 64, 128, 1, 64, 0.3),       # a single token
    (16, 100, 32, 16, 128, 1, 32, 0.1),   # many heads: four heads per workgroup
    (1, 1000, 2, 64, 64, 2, 64, 0.0),     # 16 chunks through the state scan
    (1, 1500, 4, 64, 128, 1, 512, 0.1),   # long chunks: 16 row blocks carried per chunk
    (2, 1400, 2, 64, 128, 1, 700, 0.2),   # chunk of 700 rows, ragged blocks
    (1, 200, 3, 64, 128, 1, 64, 0.1),     # odd group size: one head (two waves) per workgroup
    (2, 130, 8, 32, 128, 2, 64, 0.1),     # head_dim 32, four heads per workgroup
]


def _id(c):
    return "b%d_l%d_h%d_p%d_n%d_g%d_Q%d" % c[:7]


@pytest.fixture(autouse=True)
def _name(request):
    log("start", request.node.nodeid)
    yield


@pytest.fixture(scope="module")
def orc():
    import oracle
    oracle.build()
    return oracle


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("case", SMALL, ids=_id)
def test_small_parity(orc, case, io):
    b, l, h, p, n, g, Q, init = case
    inp = syn.random_case(1000 + sum(case[:7]), b, l, h, p, n, g, io=io, init_std=init)
    y, fin = run_scan(inp, Q)
    yo, fo = orc.scan(**oracle_kw(inp))
    s1 = check_close(to_f64(y), yo, io, "y", Y_AXES)
    s2 = check_close(to_f64(fin), fo, io, "final_state", STATE_AXES)
    log("y max_abs %.3g max_rel %.3g | final max_abs %.3g" % (s1[0], s1[1], s2[0]))


# workgroups sharing B and C over several heads (head_dim 64 and 16) and
# one-head workgroups (group sizes that do not divide), ragged chunks
SHAPES = [
    (2, 300, 4, 64, 128, 1, 256, 0.1),    # two heads of one group per workgroup
    (1, 700, 8, 32, 64, 2, 100, 0.2),     # four heads per workgroup; ragged 100-row chunks
    (2, 200, 16, 16, 128, 4, 64, 0.0),    # four heads of head_dim 16 per workgroup
    (1, 520, 24, 64, 128, 1, 256, 0.0),   # the 130m shape, shorter
    (1, 333, 6, 64, 64, 3, 96, 0.3),      # group size 2: one head per workgroup
]


@pytest.mark.parametrize("case", SHAPES, ids=_id)
def test_bf16_shapes_and_determinism(orc, case):
    """bf16 scans over workgroup layouts and ragged chunks meet the bar
    against the oracle, and two calls give the same bits (every sum in a
    fixed order, nondeterminism being the complaint of the state-spaces/mamba
    issue 1024 mirror page)."""
    b, l, h, p, n, g, Q, init = case
    inp = syn.random_case(2000 + sum(case[:7]), b, l, h, p, n, g, io="bf16", init_std=init)
    y1, f1 = run_scan(inp, Q)
    y2, f2 = run_scan(inp, Q)
    torch = torch_mod()
    assert torch.equal(y1, y2)
    assert torch.equal(f1, f2)
    yo, fo = orc.scan(**oracle_kw(inp))
    check_close(to_f64(y1), yo, "bf16", "y", Y_AXES)
    check_close(to_f64(f1), fo, "bf16", "final_state", STATE_AXES)


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("init", [0.0, 0.3])
def test_outputs_independent_of_final_state_request(orc, io, init):
    """Without a requested final state the last chunk's own state is neither
    stored nor read, and without an initial state chunk 0's boundary state
    is neither stored nor read; y must not change with either choice."""
    inp = syn.random_case(31, 2, 700, 4, 64, 128, 2, io=io, init_std=init)
    g = gpu_inputs(inp)
    y_f, fin = run_scan(inp, 128, final=True, g=g)
    y_n = run_scan(inp, 128, final=False, g=g)
    if isinstance(y_n, tuple):
        y_n = y_n[0]
    assert torch_mod().equal(y_f, y_n)
    yo, fo = orc.scan(**oracle_kw(inp))
    check_close(to_f64(y_n), yo, io, "y", Y_AXES)
    check_close(to_f64(fin), fo, io, "final_state", STATE_AXES)


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_no_skip_no_bias_clamped(orc, io):
    inp = syn.random_case(7, 2, 150, 4, 64, 64, 2, io=io, init_std=0.2)
    inp["D"] = None
    inp["dt_bias"] = None
    y, fin = run_scan(inp, 64, dt_limit=(0.05, 0.5))
    yo, fo = orc.scan(**oracle_kw(inp, dt_limit=(0.05, 0.5)))
    check_close(to_f64(y), yo, io, "y", Y_AXES)
    check_close(to_f64(fin), fo, io, "final_state", STATE_AXES)


def test_raw_time_step_without_softplus(orc):
    inp = syn.random_case(8, 2, 90, 4, 32, 64, 1, io="f32")
    inp["dt"] = np.abs(inp["dt"]) * np.float32(0.1)
    inp["dt_bias"] = None
    y, fin = run_scan(inp, 32, dt_softplus=False)
    yo, fo = orc.scan(**oracle_kw(inp, dt_softplus=False))
    check_close(to_f64(y), yo, "f32", "y", Y_AXES)
    check_close(to_f64(fin), fo, "f32", "final_state", STATE_AXES)


def test_deterministic_bitwise():
    """Two runs on the same inputs give identical bits (no float atomics,
    fixed reduction order); nondeterminism is the complaint of the mirror of
    state-spaces/mamba issue 1024."""
    torch = torch_mod()
    inp = syn.random_case(9, 4, 700, 8, 64, 128, 2, io="bf16", init_std=0.1)
    g = gpu_inputs(inp)
    y1, f1 = run_scan(inp, 256, g=g)
    y2, f2 = run_scan(inp, 256, g=g)
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
    assert torch.equal(f1.view(torch.int32), f2.view(torch.int32))


def test_extreme_decays_stay_finite(orc):
    """A = -16 with large time steps (cumulative log decay far below -1e4):
    every output finite (kongchang "Mamba2": a NaN from a chunk-scan kernel
    was a numerical-stability defect) and equal to the oracle."""
    inp = syn.random_case(10, 2, 600, 4, 64, 128, 1, io="bf16", init_std=1.0)
    inp["A"] = np.full_like(inp["A"], -16.0)
    inp["dt"] = syn.bf16_round(np.abs(syn.bf16_to_f32(inp["dt"])) + np.float32(10.0))
    y, fin = run_scan(inp, 256)
    assert torch_mod().isfinite(y.float()).all() and torch_mod().isfinite(fin).all()
    yo, fo = orc.scan(**oracle_kw(inp))
    check_close(to_f64(y), yo, "bf16", "y", Y_AXES)
    check_close(to_f64(fin), fo, "bf16", "final_state", STATE_AXES)


def test_literal_dt_bias_reading_stress(orc):
    """The literal reading of 'dt_bias loguniform[1e-3, 0.1]' (no inverse
    softplus): larger time steps and decays."""
    inp = syn.random_case(11, 1, 2048, 16, 64, 128, 8, io="bf16", literal=True)
    y, fin = run_scan(inp, 256)
    yo, fo = orc.scan(**oracle_kw(inp))
    check_close(to_f64(y), yo, "bf16", "y", Y_AXES)
    check_close(to_f64(fin), fo, "bf16", "final_state", STATE_AXES)


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_split_forward_equals_one_forward(orc, io):
    """scan(l1) -> final as init -> scan(l2) equals scan(l1 + l2): the
    boundary state is a function of the initial state (nnterp, "The state
    after every token"), so a prompt can be resumed."""
    inp = syn.random_case(12, 2, 333, 4, 64, 128, 1, io=io, init_std=0.1)
    l1 = 140
    first = {k: (v[:, :l1] if k in ("x", "dt", "B", "C") else v) for k, v in inp.items()}
    second = {k: (v[:, l1:] if k in ("x", "dt", "B", "C") else v) for k, v in inp.items()}
    y1, f1 = run_scan(first, 64)
    g2 = gpu_inputs(second)
    g2["init"] = f1
    y2, f2 = run_scan(second, 64, g=g2)
    yo, fo = orc.scan(**oracle_kw(inp))
    check_close(np.concatenate([to_f64(y1), to_f64(y2)], axis=1), yo, io, "y", Y_AXES)
    check_close(to_f64(f2), fo, io, "final_state", STATE_AXES)


def test_final_state_may_alias_initial_state(orc):
    import mamba_ssd_chunked_chunk_amd as ssd
    inp = syn.random_case(13, 2, 200, 4, 64, 128, 1, io="bf16", init_std=0.3)
    g = gpu_inputs(inp)
    st = g["init"].clone()
    y, fin = ssd.chunk_scan(g["x"], g["dt"], g["A"], g["B"], g["C"], g["D"], chunk_size=64,
                            dt_bias=g["dt_bias"], initial_state=st, return_final_state=True,
                            final_out=st)
    torch_mod().cuda.synchronize()
    assert fin.data_ptr() == st.data_ptr()
    yo, fo = orc.scan(**oracle_kw(inp))
    check_close(to_f64(y), yo, "bf16", "y", Y_AXES)
    check_close(to_f64(st), fo, "bf16", "final_state", STATE_AXES)


def test_group_expansion():
    """g groups equal h groups with B, C repeated over each group's contiguous
    heads (the head -> group map hh // (heads // groups))."""
    torch = torch_mod()
    inp = syn.random_case(14, 2, 300, 8, 64, 128, 2, io="f32", init_std=0.1)
    y, fin = run_scan(inp, 64)
    rep = dict(inp, B=np.repeat(inp["B"], 4, axis=2), C=np.repeat(inp["C"], 4, axis=2))
    yr, fr = run_scan(rep, 64)
    assert torch.allclose(y, yr, rtol=1e-5, atol=1e-5)
    assert torch.allclose(fin, fr, rtol=1e-5, atol=1e-5)


def test_nan_stays_in_its_head():
    """A NaN in one (batch, head)'s x reaches only that (batch, head)."""
    torch = torch_mod()
    inp = syn.random_case(15, 2, 300, 4, 64, 128, 1, io="f32")
    inp["x"] = inp["x"].copy()
    inp["x"][1, 77, 2, 5] = np.nan
    y, fin = run_scan(inp, 64)
    bad = ~torch.isfinite(y)
    assert bad[1, 77:, 2].any()
    bad[1, :, 2] = False
    assert not bad.any()
    fb = ~torch.isfinite(fin)
    fb[1, 2] = False
    assert not fb.any()


def test_empty_sequence_and_batch():
    import mamba_ssd_chunked_chunk_amd as ssd
    torch = torch_mod()
    inp = syn.random_case(16, 3, 5, 4, 64, 128, 1, io="bf16", init_std=0.5)
    g = gpu_inputs(inp)
    empty = {k: (v[:, :0].contiguous() if k in ("x", "dt", "B", "C") else v) for k, v in g.items()}
    y, fin = ssd.chunk_scan(empty["x"], empty["dt"], g["A"], empty["B"], empty["C"], g["D"],
                            chunk_size=64, dt_bias=g["dt_bias"], initial_state=g["init"],
                            return_final_state=True)
    torch.cuda.synchronize()
    assert y.shape == (3, 0, 4, 64)
    assert torch.equal(fin, g["init"])
    y, fin = ssd.chunk_scan(empty["x"], empty["dt"], g["A"], empty["B"], empty["C"], g["D"],
                            chunk_size=64, return_final_state=True)
    torch.cuda.synchronize()
    assert torch.count_nonzero(fin) == 0
    z = {k: (v[:0].contiguous() if k in ("x", "dt", "B", "C") else v) for k, v in g.items()}
    y, fin = ssd.chunk_scan(z["x"], z["dt"], g["A"], z["B"], z["C"], g["D"], chunk_size=64,
                            return_final_state=True)
    torch.cuda.synchronize()
    assert y.shape[0] == 0 and fin.shape[0] == 0


def test_workspace_contents_ignored(orc):
    """The workspace is filled with NaN bytes before the call: nothing the
    scan reads from it may come from an earlier call or be left unwritten."""
    import mamba_ssd_chunked_chunk_amd as ssd
    torch = torch_mod()
    b, l, h, p, n, g, Q = 2, 300, 4, 64, 128, 2, 64
    for io in ("f32", "bf16"):
        inp = syn.random_case(19, b, l, h, p, n, g, io=io, init_std=0.2)
        G = gpu_inputs(inp)
        ws = torch.full((ssd.workspace_bytes(b, l, h, p, n, g, Q),), 0xFF, dtype=torch.uint8,
                        device="cuda")
        y, fin = ssd.chunk_scan(G["x"], G["dt"], G["A"], G["B"], G["C"], G["D"], chunk_size=Q,
                                dt_bias=G["dt_bias"], initial_state=G["init"],
                                return_final_state=True, workspace=ws)
        torch.cuda.synchronize()
        yo, fo = orc.scan(**oracle_kw(inp))
        check_close(to_f64(y), yo, io, "y", Y_AXES)
        check_close(to_f64(fin), fo, io, "final state", STATE_AXES)


def test_invalid_arguments_raise():
    import mamba_ssd_chunked_chunk_amd as ssd
    inp = syn.random_case(17, 1, 64, 4, 64, 128, 1, io="bf16")
    g = gpu_inputs(inp)
    with pytest.raises(ssd.SsdError):
        ssd.chunk_scan(g["x"], g["dt"], g["A"], g["B"], g["C"], g["D"], chunk_size=0)
    with pytest.raises(ValueError):
        ssd.chunk_scan(g["x"], g["dt"], g["A"], g["B"], g["C"].float(), g["D"])
    with pytest.raises(ssd.SsdError):
        ssd.chunk_scan(g["x"], g["dt"], g["A"], g["B"], g["C"], g["D"], chunk_size=64,
                       workspace=torch_mod().empty(256, dtype=torch_mod().uint8, device="cuda"))


def _ws_layout(b, l, h, n, p, Q):
    """Workspace offsets (bytes) as the library lays them out (include/ssd.h):
    four per-row fp32 arrays, boundary states, chunk states, chunk log2
    decays, chunk-state maxima, then the boundary-state scales."""
    T = 32   # rows per block
    nc = -(-l // Q)
    Qp = -(-Q // T) * T
    lp = nc * Qp
    a256 = lambda v: (v + 255) // 256 * 256
    off = {"lcs": 0}
    off["dtp"] = a256(b * h * lp * 4)
    off["wgt"] = off["dtp"] + a256(b * h * lp * 4)
    off["sgr"] = off["wgt"] + a256(b * h * lp * 4)
    off["hb"] = off["sgr"] + a256(b * h * lp * 4)
    off["st"] = off["hb"] + a256(b * nc * h * n * p * 4)
    off["lam"] = off["st"] + a256(b * nc * h * n * p * 4)
    off["scl"] = off["lam"] + a256(b * h * nc * 4)
    off["hs"] = off["scl"] + a256(b * h * nc * 4)   # no short-chunk states here
    return T, nc, Qp, lp, off


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_stage_intermediates(orc, io):
    """Intermediates read back from the workspace against the chunked fp64
    steps: the boundary states (fp32 on the fp32 path; fp16 times their
    power-of-two scale per (batch, chunk, head) on the bf16 path), and on the
    fp32 path the per-row time step, cumulative log decay and state weights
    (the bf16 kernels compute those on chip and store none)."""
    import mamba_ssd_chunked_chunk_amd as ssd
    from oracle import chunked
    torch = torch_mod()
    T = 32
    # a grid small enough (under four workgroups per compute unit) that the
    # bf16 scan stores the state at every one of the caller's chunks
    b, l, h, p, n, g, Q = 4, 5 * T + 11, 128, 16, 32, 4, T
    inp = syn.random_case(18, b, l, h, p, n, g, io=io, init_std=0.1)
    G = gpu_inputs(inp)
    wsb = ssd.workspace_bytes(b, l, h, p, n, g, Q)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    ssd.chunk_scan(G["x"], G["dt"], G["A"], G["B"], G["C"], G["D"], chunk_size=Q,
                   dt_bias=G["dt_bias"], initial_state=G["init"], workspace=ws)
    torch.cuda.synchronize()
    T, nc, Qp, lp, off = _ws_layout(b, l, h, n, p, Q)
    wsf = ws.view(torch.float32)
    _, _, inter = chunked.chunked_scan(**oracle_kw(inp), chunk=Q)
    # boundary states are stored transposed: [b, chunks, heads, head_dim, state_dim]
    if io == "bf16":
        hb = ws[off["hb"]: off["hb"] + 2 * b * nc * h * n * p].view(torch.float16).float()
        sc = wsf[off["hs"] // 4: off["hs"] // 4 + b * h * nc].view(b, h, nc)
        hb = hb.view(b, nc, h, p, n) * sc.transpose(1, 2)[..., None, None]
    else:
        hb = wsf[off["hb"] // 4: off["hb"] // 4 + b * nc * h * n * p].view(b, nc, h, p, n)
    hb = hb.transpose(3, 4)
    check_close(to_f64(hb), inter["H_prev"], io, "boundary states", (1, 3, 4))
    if io == "bf16":
        return
    field = lambda k: wsf[off[k] // 4: off[k] // 4 + b * h * lp].view(b, h, nc, Qp)[..., :Q] \
        .reshape(b, h, nc * Q)[..., :l]
    lcs, dtp, wgt = field("lcs"), field("dtp"), field("wgt")
    check_close(to_f64(dtp), inter["d"], "f32", "processed time step")
    # per-chunk cumsum (natural log) == lcs / log2(e) since blocks == chunks
    cs = to_f64(lcs) / math.log2(math.e)
    err = np.abs(cs - inter["cs"])
    assert (err <= 1e-5 * (1 + np.abs(inter["cs"]))).all(), err.max()
    # weight of each row in the state at its block's (here: chunk's) end:
    # exp(cs[last row of the chunk] - cs[row]) d[row]
    cs_o = inter["cs"]
    last = np.minimum(np.arange(l) // Q * Q + Q, l) - 1
    w_o = np.exp(cs_o[..., last] - cs_o) * inter["d"]
    check_close(to_f64(wgt), w_o, "f32", "row weights")


def test_graph_capture_replays_match_eager(orc):
    """One ssd_chunk_scan call captured in a HIP graph (preallocated output,
    final state and workspace; the library allocates and clears nothing) and
    replayed several times with eager work in between: every replay equals
    the eager call bit for bit."""
    import mamba_ssd_chunked_chunk_amd as ssd
    torch = torch_mod()
    inp = syn.random_case(41, 2, 600, 8, 64, 128, 2, io="bf16", init_std=0.2)
    g = gpu_inputs(inp)
    b, l, h, p = g["x"].shape
    n = g["B"].shape[3]
    Q = 256
    ws = torch.empty(ssd.workspace_bytes(b, l, h, p, n, 2, Q), dtype=torch.uint8, device="cuda")
    y = torch.empty_like(g["x"])
    fin = torch.empty((b, h, n, p), dtype=torch.float32, device="cuda")

    def call():
        ssd.chunk_scan(g["x"], g["dt"], g["A"], g["B"], g["C"], g["D"], chunk_size=Q,
                       dt_bias=g["dt_bias"], initial_state=g["init"], return_final_state=True,
                       out=y, final_out=fin, workspace=ws)
    call()
    torch.cuda.synchronize()
    y_ref, f_ref = y.clone(), fin.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call()                      # warm the path on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    for k in range(3):
        y.zero_()
        fin.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), y_ref.view(torch.int16)), k
        assert torch.equal(fin.view(torch.int32), f_ref.view(torch.int32)), k
        call()                      # eager work between replays
        torch.cuda.synchronize()
    yo, fo = orc.scan(**oracle_kw(inp))
    check_close(to_f64(y), yo, "bf16", "y", Y_AXES)
