"""GPU parity of the steps around the scan (ssd_conv1d_silu, ssd_gated_norm,
through the C ABI) against the fp64 oracle in oracle/neighbors.py."""
import numpy as np
import pytest

import ssd_synth as syn
from gpu_util import Y_AXES, check_close, dev_tensor, log, to_f64, torch_mod

pytestmark = pytest.mark.gpu


def _seq(b, l, cuts_per_row):
    seq = np.zeros((b, l), np.int32)
    for bi, cuts in enumerate(cuts_per_row):
        for k, c in enumerate(cuts):
            seq[bi, c:] = 10 * (k + 1) + bi
    return seq


def _dev_int(a):
    return torch_mod().from_numpy(np.ascontiguousarray(a, np.int32)).to("cuda")


def _conv(case, seq=None, bias=True, init=True, silu=True):
    import mamba_ssd_chunked_chunk_amd as ssd
    from oracle import neighbors as nb
    io = case["io"]
    xbc32 = syn.as_f32(case["xbc"], io)
    h, p, n, g = case["heads"], case["head_dim"], case["state_dim"], case["groups"]
    ci = case["conv_init"] if init else None
    x, B, C, fin = ssd.conv1d_silu(dev_tensor(case["xbc"]), dev_tensor(case["weight"]), h, p, n, g,
                                   bias=dev_tensor(case["bias"]) if bias else None,
                                   conv_init=dev_tensor(ci),
                                   seq_idx=None if seq is None else _dev_int(seq),
                                   apply_silu=silu, return_conv_state=True)
    torch_mod().cuda.synchronize()
    xo, Bo, Co, fo = nb.conv1d_silu(xbc32, case["weight"], h, p, n, g,
                                    bias=case["bias"] if bias else None, conv_init=ci,
                                    seq_idx=seq, apply_silu=silu)
    s = check_close(to_f64(x), xo, io, "x", Y_AXES)
    check_close(to_f64(B), Bo, io, "B", Y_AXES)
    check_close(to_f64(C), Co, io, "C", Y_AXES)
    # the final conv state is a copy of inputs: exact
    np.testing.assert_array_equal(to_f64(fin), fo)
    return s


# (batch, seqlen, heads, head_dim, state_dim, groups, width)
CONV = [
    (1, 50, 2, 16, 32, 1, 4),
    (2, 37, 4, 64, 128, 2, 4),     # ragged last run
    (3, 5, 2, 32, 64, 1, 3),       # one partial run
    (1, 2, 2, 16, 32, 2, 4),       # fewer tokens than the window
    (2, 100, 3, 128, 64, 1, 2),
    (1, 64, 2, 16, 32, 1, 1),      # no history
    (2, 45, 3, 12, 36, 1, 4),      # bf16 x, B widths not multiples of 8: 4-channel threads
    (1, 300, 2, 64, 64, 1, 4),     # many runs, the last one ragged
]


def _cid(c):
    return "b%d_l%d_h%d_p%d_n%d_g%d_w%d" % c


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("case", CONV, ids=_cid)
def test_conv_parity(case, io):
    c = syn.conv_case(4000 + sum(case), *case, io=io)
    _conv(c)
    _conv(c, bias=False, init=False)


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_conv_without_silu(io):
    c = syn.conv_case(4100, 2, 40, 2, 32, 64, 1, 4, io=io)
    _conv(c, silu=False)


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_conv_packed_documents(io):
    c = syn.conv_case(4200, 2, 70, 4, 64, 32, 2, 4, io=io)
    seq = _seq(2, 70, [(1, 2, 3, 16, 17, 40), (69,)])
    _conv(c, seq=seq)
    # the last document shorter than the window: earlier rows drop out of the final state
    seq2 = _seq(2, 70, [(68,), (69,)])
    _conv(c, seq=seq2)


def test_conv_bench_shape():
    """The 130m mixer's projection: 8 x 2048 tokens, 24 heads of 64, state 128,
    1 group, width 4, bf16."""
    c = syn.conv_case(4300, 8, 2048, 24, 64, 128, 1, 4, io="bf16")
    s = _conv(c)
    log("conv bench shape: max_abs %.3g max_rel %.3g" % (s[0], s[1]))


@pytest.mark.parametrize("init", [False, True])
def test_conv_no_tokens(init):
    """Zero tokens: the final conv state is the initial one (or zeros)."""
    import mamba_ssd_chunked_chunk_amd as ssd
    torch = torch_mod()
    c = syn.conv_case(4400, 2, 0, 2, 16, 32, 1, 4, io="f32")
    ci = dev_tensor(syn.conv_case(4401, 2, 1, 2, 16, 32, 1, 4)["conv_init"]) if init else None
    x, B, C, fin = ssd.conv1d_silu(dev_tensor(c["xbc"]), dev_tensor(c["weight"]), 2, 16, 32, 1,
                                   conv_init=ci, return_conv_state=True)
    torch.cuda.synchronize()
    assert x.numel() == 0
    if init:
        assert torch.equal(fin, ci)
    else:
        assert torch.count_nonzero(fin) == 0


def _norm(case, z=True, weight=True, normalize=True, G=None, inplace=False):
    import mamba_ssd_chunked_chunk_amd as ssd
    from oracle import neighbors as nb
    io = case["io"]
    y = dev_tensor(case["y"])
    zt = dev_tensor(case["z"]) if z else None
    wt = dev_tensor(case["weight"]) if weight else None
    out = ssd.gated_norm(y, zt, wt, group_size=G, eps=1e-5, normalize=normalize,
                         out=y if inplace else None)
    torch_mod().cuda.synchronize()
    o = nb.gated_norm(syn.as_f32(case["y"], io), syn.as_f32(case["z"], io) if z else None,
                      case["weight"] if weight else None, group_size=G, eps=1e-5,
                      normalize=normalize)
    return check_close(to_f64(out), o, io, "gated norm", (1,))


# (rows, dim, group_size)
NORM = [(7, 1536, 1536), (5, 64, 16), (3, 4096, 512), (2, 8, 4), (33, 1536, 192),
        (3, 3072, 1024),   # 4 steps of 256 channels in registers
        (2, 2048, 2048),   # 8 steps
        (4, 1400, 700),    # 3 steps, held as 4 with the last masked
        (3, 5008, 1252),   # 5 steps, held as 6
        (2, 6144, 3072)]   # beyond registers: two passes


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("case", NORM, ids=lambda c: "r%d_d%d_g%d" % c)
def test_norm_parity(case, io):
    rows, dim, G = case
    c = syn.norm_case(4500 + rows + dim + G, rows, dim, io=io)
    _norm(c, G=G)
    _norm(c, z=False, G=G)
    _norm(c, weight=False, G=G)
    _norm(c, normalize=False, G=G)


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_norm_in_place(io):
    c = syn.norm_case(4600, 9, 512, io=io)
    _norm(c, G=128, inplace=True)
    c = syn.norm_case(4601, 5, 1400, io=io)
    _norm(c, G=700, inplace=True)


def test_norm_bench_shape():
    """y of the 130m mixer: 8 x 2048 tokens of 24 x 64 channels, one group, bf16."""
    c = syn.norm_case(4700, 8 * 2048, 1536, io="bf16")
    s = _norm(c)
    log("gated norm bench shape: max_abs %.3g max_rel %.3g" % (s[0], s[1]))


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_mixer_chain_matches_composed_oracles(io):
    """conv1d + SiLU -> chunk scan -> gate + RMS norm on the GPU against the
    same chain of oracles (each GPU stage fed by the previous GPU stage, as
    in a layer; the oracle chain in fp64, its scan inputs rounded like the
    GPU's)."""
    import mamba_ssd_chunked_chunk_amd as ssd
    import oracle
    from oracle import neighbors as nb
    torch = torch_mod()
    b, l, h, p, n, g, K, Q = 2, 300, 4, 64, 64, 2, 4, 128
    c = syn.conv_case(4800, b, l, h, p, n, g, K, io=io, with_init=False)
    sc = syn.random_case(4801, b, l, h, p, n, g, io=io)
    z = syn.norm_case(4802, b * l, h * p, io=io)
    x, B, C = ssd.conv1d_silu(dev_tensor(c["xbc"]), dev_tensor(c["weight"]), h, p, n, g,
                              bias=dev_tensor(c["bias"]))
    y = ssd.chunk_scan(x, dev_tensor(sc["dt"]), dev_tensor(sc["A"]), B, C, dev_tensor(sc["D"]),
                       chunk_size=Q, dt_bias=dev_tensor(sc["dt_bias"]))
    out = ssd.gated_norm(y.reshape(b * l, h * p), dev_tensor(z["z"]), dev_tensor(z["weight"]),
                         eps=1e-5)
    torch.cuda.synchronize()
    # the oracle chain: its conv in fp64, rounded to the io type as the GPU
    # stores it, then the fp64 scan, then the fp64 gate and norm
    xo, Bo, Co, _ = nb.conv1d_silu(syn.as_f32(c["xbc"], io), c["weight"], h, p, n, g,
                                   bias=c["bias"])
    r = (lambda a: syn.bf16_round(np.asarray(a, np.float32))) if io == "bf16" else \
        (lambda a: np.asarray(a, np.float32))
    yo, _ = oracle.scan(r(xo), sc["dt"], sc["A"], r(Bo), r(Co), sc["D"], sc["dt_bias"], io=io)
    oo = nb.gated_norm(yo.reshape(b * l, h * p), syn.as_f32(z["z"], io), z["weight"], eps=1e-5)
    check_close(to_f64(out), oo, io, "mixer chain", (1,))
