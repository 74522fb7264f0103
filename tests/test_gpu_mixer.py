"""GPU tests of ssd_mixer_forward (conv1d + SiLU + split, the chunk scan and
the gated RMS norm in one call, through the C ABI): against the chain of
fp64 oracles, and bit for bit against the three separate entry points."""
import numpy as np
import pytest

import ssd_synth as syn
from gpu_util import STATE_AXES, Y_AXES, check_close, dev_tensor, log, to_f64, torch_mod

pytestmark = pytest.mark.gpu


def _dev_int(a):
    return torch_mod().from_numpy(np.ascontiguousarray(a, np.int32)).to("cuda")


def _case(seed, b, l, h, p, n, g, K, io, init=True, docs=False, z=True, init_std=0.0):
    c = syn.conv_case(seed, b, l, h, p, n, g, K, io=io, with_init=init)
    sc = syn.random_case(seed + 1, b, l, h, p, n, g, io=io, init_std=init_std)
    nc = syn.norm_case(seed + 2, b * l, h * p, io=io)
    seq = syn.doc_index(seed + 3, b, l, lo=16, hi=max(l // 2, 17)) if docs else None
    return dict(c=c, sc=sc, z=nc["z"].reshape(b, l, h * p) if z else None, nw=nc["weight"],
                seq=seq, dims=(b, l, h, p, n, g, K))


def _mixer(case, Q, G, normalize=True, final=True):
    import mamba_ssd_chunked_chunk_amd as ssd
    c, sc = case["c"], case["sc"]
    b, l, h, p, n, g, K = case["dims"]
    r = ssd.mixer_forward(
        dev_tensor(c["xbc"]), dev_tensor(sc["dt"]), dev_tensor(sc["A"]), dev_tensor(c["weight"]),
        h, p, n, g, z=None if case["z"] is None else dev_tensor(case["z"]),
        conv_bias=dev_tensor(c["bias"]), conv_init=dev_tensor(c["conv_init"]),
        D=dev_tensor(sc["D"]), dt_bias=dev_tensor(sc["dt_bias"]),
        initial_state=dev_tensor(sc["init_state"]),
        seq_idx=None if case["seq"] is None else _dev_int(case["seq"]),
        norm_weight=dev_tensor(case["nw"]), norm_group=G, eps=1e-5, normalize=normalize,
        chunk_size=Q, return_final_state=final, return_conv_state=final)
    torch_mod().cuda.synchronize()
    return r


def _chain(case, Q, G, normalize=True):
    """The same mixer through the three separate entry points."""
    import mamba_ssd_chunked_chunk_amd as ssd
    c, sc = case["c"], case["sc"]
    b, l, h, p, n, g, K = case["dims"]
    seq = None if case["seq"] is None else _dev_int(case["seq"])
    x, B, C, cfin = ssd.conv1d_silu(dev_tensor(c["xbc"]), dev_tensor(c["weight"]), h, p, n, g,
                                    bias=dev_tensor(c["bias"]),
                                    conv_init=dev_tensor(c["conv_init"]), seq_idx=seq,
                                    return_conv_state=True)
    y, fin = ssd.chunk_scan(x, dev_tensor(sc["dt"]), dev_tensor(sc["A"]), B, C,
                            dev_tensor(sc["D"]), chunk_size=Q, dt_bias=dev_tensor(sc["dt_bias"]),
                            initial_state=dev_tensor(sc["init_state"]), seq_idx=seq,
                            return_final_state=True)
    zz = None if case["z"] is None else dev_tensor(case["z"]).reshape(b * l, h * p)
    out = ssd.gated_norm(y.reshape(b * l, h * p), zz, dev_tensor(case["nw"]), group_size=G,
                         eps=1e-5, normalize=normalize)
    torch_mod().cuda.synchronize()
    return out.reshape(b, l, h, p), fin, cfin


def _oracle(case, G, normalize=True):
    """The chain of fp64 oracles, each scan input rounded to the io type as
    the conv stores it (as a layer feeds the scan)."""
    import oracle
    from oracle import neighbors as nb
    c, sc = case["c"], case["sc"]
    io = c["io"]
    b, l, h, p, n, g, K = case["dims"]
    xo, Bo, Co, cfo = nb.conv1d_silu(syn.as_f32(c["xbc"], io), c["weight"], h, p, n, g,
                                     bias=c["bias"], conv_init=c["conv_init"],
                                     seq_idx=case["seq"])
    r = (lambda a: syn.bf16_round(np.asarray(a, np.float32))) if io == "bf16" else \
        (lambda a: np.asarray(a, np.float32))
    yo, fo = oracle.scan(r(xo), sc["dt"], sc["A"], r(Bo), r(Co), sc["D"], sc["dt_bias"],
                         init_state=sc["init_state"], io=io, seq_idx=case["seq"])
    zz = None if case["z"] is None else syn.as_f32(case["z"], io).reshape(b * l, h * p)
    oo = nb.gated_norm(yo.reshape(b * l, h * p), zz, case["nw"], group_size=G, eps=1e-5,
                       normalize=normalize)
    return oo.reshape(b, l, h, p), fo, cfo


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("shape", [
    # b, l, h, p, n, g, K, Q, norm group, packed documents
    (2, 300, 4, 64, 64, 2, 4, 128, 128, False),
    (1, 700, 8, 64, 128, 2, 4, 256, 512, True),
    (3, 129, 6, 32, 64, 3, 3, 64, 64, True),
])
def test_mixer_matches_oracle_chain(io, shape):
    b, l, h, p, n, g, K, Q, G, docs = shape
    case = _case(7100 + l, b, l, h, p, n, g, K, io, docs=docs, init_std=0.1)
    out, fin, cfin = _mixer(case, Q, G)
    oo, fo, cfo = _oracle(case, G)
    log("mixer %s %s io=%s" % (shape, "docs" if docs else "", io))
    check_close(to_f64(out), oo, io, "mixer out", Y_AXES)
    check_close(to_f64(fin), fo, io, "mixer final state", STATE_AXES)
    check_close(to_f64(cfin), cfo, "f32", "mixer conv state")


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_mixer_equals_separate_calls_bitwise(io):
    """One call gives the bits of the three entry points in a row."""
    torch = torch_mod()
    case = _case(7200, 2, 1000, 8, 64, 128, 1, 4, io, docs=True, init_std=0.1)
    out, fin, cfin = _mixer(case, 256, 256)
    o2, f2, c2 = _chain(case, 256, 256)
    assert torch.equal(out, o2)
    assert torch.equal(fin, f2)
    assert torch.equal(cfin, c2)


def test_mixer_without_gate_or_norm_is_the_scan():
    """z None and normalize off: out is the scan's y of the conv's outputs."""
    torch = torch_mod()
    case = _case(7300, 2, 513, 4, 64, 64, 1, 4, "bf16", z=False)
    out, fin, _ = _mixer(case, 256, 256, normalize=False)
    o2, f2, _ = _chain(case, 256, 256, normalize=False)
    assert torch.equal(out, o2)
    assert torch.equal(fin, f2)


def test_mixer_at_the_130m_mixer_shape():
    """8 x 2048 tokens, 24 heads of 64, state 128, conv width 4 over 1792
    channels, one RMS norm over the 1536 channels (bf16): bit for bit the
    separate calls, each of which the oracle pins at this shape elsewhere;
    plus sampled rows of batch row 0 against the oracle chain."""
    torch = torch_mod()
    b, l, h, p, n, g, K = 8, 2048, 24, 64, 128, 1, 4
    case = _case(7400, b, l, h, p, n, g, K, "bf16", init=False)
    out, fin, _ = _mixer(case, 256, h * p)
    o2, f2, _ = _chain(case, 256, h * p)
    assert torch.equal(out, o2)
    assert torch.equal(fin, f2)
    # the first batch row through the oracle chain
    one = dict(case)
    one["c"] = dict(case["c"], xbc=case["c"]["xbc"][:1])
    one["sc"] = {k: (v[:1] if k in ("x", "dt", "B", "C") and v is not None else v)
                 for k, v in case["sc"].items()}
    one["sc"]["init_state"] = None
    one["z"] = case["z"][:1]
    one["dims"] = (1, l, h, p, n, g, K)
    oo, _, _ = _oracle(one, h * p)
    check_close(to_f64(out[:1]), oo, "bf16", "mixer out (130m shape, row 0)", Y_AXES)


def test_mixer_with_no_tokens_passes_the_states_through():
    import mamba_ssd_chunked_chunk_amd as ssd
    torch = torch_mod()
    b, h, p, n, g, K = 2, 4, 64, 64, 1, 4
    ch = h * p + 2 * g * n
    xbc = torch.zeros((b, 0, ch), dtype=torch.bfloat16, device="cuda")
    dt = torch.zeros((b, 0, h), dtype=torch.bfloat16, device="cuda")
    A = -torch.ones(h, device="cuda")
    w = torch.ones((ch, K), device="cuda")
    init = torch.randn((b, h, n, p), device="cuda")
    cinit = torch.randn((b, K - 1, ch), device="cuda")
    out, fin, cfin = ssd.mixer_forward(xbc, dt, A, w, h, p, n, g, conv_init=cinit,
                                       initial_state=init, return_final_state=True,
                                       return_conv_state=True)
    torch.cuda.synchronize()
    assert out.shape == (b, 0, h, p)
    assert torch.equal(fin, init)
    assert torch.equal(cfin, cinit)


def test_mixer_graph_capture_replays_match_eager():
    """One ssd_mixer_forward call (conv, scan and norm: kernel launches only,
    nothing allocated or cleared by the library) captured in a HIP graph and
    replayed several times with eager work in between: every replay equals
    the eager call bit for bit."""
    import mamba_ssd_chunked_chunk_amd as ssd
    torch = torch_mod()
    b, l, h, p, n, g, K, Q = 2, 700, 8, 64, 128, 2, 4, 256
    case = _case(7500, b, l, h, p, n, g, K, "bf16", docs=True, init_std=0.1)
    c, sc = case["c"], case["sc"]
    T = {k: dev_tensor(v) for k, v in (("xbc", c["xbc"]), ("w", c["weight"]), ("cb", c["bias"]),
                                       ("ci", c["conv_init"]), ("dt", sc["dt"]), ("A", sc["A"]),
                                       ("D", sc["D"]), ("bias", sc["dt_bias"]),
                                       ("init", sc["init_state"]), ("z", case["z"]),
                                       ("nw", case["nw"]))}
    seq = _dev_int(case["seq"])
    out = torch.empty((b, l, h, p), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(ssd.mixer_workspace_bytes(b, l, h, p, n, g, Q), dtype=torch.uint8,
                     device="cuda")

    def call():
        ssd.mixer_forward(T["xbc"], T["dt"], T["A"], T["w"], h, p, n, g, z=T["z"],
                          conv_bias=T["cb"], conv_init=T["ci"], D=T["D"], dt_bias=T["bias"],
                          initial_state=T["init"], seq_idx=seq, norm_weight=T["nw"],
                          norm_group=256, chunk_size=Q, out=out, workspace=ws)
    call()
    torch.cuda.synchronize()
    ref = out.clone()
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
        out.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), k
        call()                      # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), k
