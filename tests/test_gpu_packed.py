"""GPU parity of the packed-sequence reset and of the state after every
chunk (ssd_chunk_scan_ex, through the C ABI) against the fp64 oracle.

Packed rows hold several documents back to back; wherever the per-token
document index changes, the next token starts from a zero state (the
sample-packing reset of the Mamba2 news page).  The state after every chunk
boundary is the nnterp guide's "state after every token" with chunk 1.
"""
import numpy as np
import pytest

import ssd_synth as syn
from gpu_util import (STATE_AXES, Y_AXES, check_close, gpu_inputs, log, oracle_kw, to_f64,
                      torch_mod)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def orc():
    import oracle
    oracle.build()
    return oracle


def _seq(b, l, cuts_per_row):
    seq = np.zeros((b, l), np.int32)
    for bi, cuts in enumerate(cuts_per_row):
        for k, c in enumerate(cuts):
            seq[bi, c:] = 10 * (k + 1) + bi
    return seq


def _run(inp, Q, seq=None, states=False, final=True):
    import mamba_ssd_chunked_chunk_amd as ssd
    torch = torch_mod()
    g = gpu_inputs(inp)
    sq = None if seq is None else torch.from_numpy(seq).to("cuda")
    out = ssd.chunk_scan(g["x"], g["dt"], g["A"], g["B"], g["C"], g["D"], chunk_size=Q,
                         dt_bias=g["dt_bias"], initial_state=g["init"],
                         return_final_state=final, seq_idx=sq,
                         return_chunk_states=states)
    torch.cuda.synchronize()
    return out


# (batch, seqlen, heads, head_dim, state_dim, groups, chunk, init_std, resets per row)
PACKED = [
    (2, 300, 4, 64, 128, 2, 64, 0.2, [(5, 40, 41, 64, 200), (1, 299)]),  # chunk starts, one-token documents
    (1, 520, 24, 64, 128, 1, 256, 0.0, [(17, 256, 300, 513)]),         # bench shape, reset at a chunk start
    (2, 130, 8, 32, 64, 2, 100, 0.1, [(31, 32, 33, 99), ()]),          # ragged chunks, block edges
    (3, 77, 4, 16, 32, 4, 16, 0.0, [(1,), (7, 8, 9, 10), (76,)]),      # short chunks, resets on the last token
    (1, 200, 3, 128, 128, 1, 64, 0.3, [(63, 64, 65, 128)]),            # head_dim 128, odd group size
]


def _pid(c):
    return "b%d_l%d_h%d_p%d_n%d_g%d_Q%d" % c[:7]


# sequences of one chunk without per-chunk states: the bf16 scan runs its
# chunk output alone (initial state in, final state out)
ONE_CHUNK = [
    (2, 200, 8, 64, 128, 2, 256, 0.3, [(3, 50, 51, 199), ()]),
    (1, 256, 4, 128, 64, 1, 256, 0.2, [(128, 129)]),
    (3, 70, 4, 32, 32, 4, 128, 0.0, [(1,), (), (33, 69)]),
]


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("case", ONE_CHUNK, ids=_pid)
def test_packed_one_chunk(orc, case, io):
    b, l, h, p, n, g, Q, init, cuts = case
    inp = syn.random_case(3100 + sum(case[:7]), b, l, h, p, n, g, io=io, init_std=init)
    seq = _seq(b, l, cuts) if any(cuts) else None
    y, fin = _run(inp, Q, seq=seq)
    yo, fo = orc.scan(**oracle_kw(inp), seq_idx=seq)
    check_close(to_f64(y), yo, io, "y", Y_AXES)
    check_close(to_f64(fin), fo, io, "final_state", STATE_AXES)


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("case", PACKED, ids=_pid)
def test_packed_sequences_parity(orc, case, io):
    b, l, h, p, n, g, Q, init, cuts = case
    inp = syn.random_case(3000 + sum(case[:7]), b, l, h, p, n, g, io=io, init_std=init)
    seq = _seq(b, l, cuts)
    y, fin, st = _run(inp, Q, seq=seq, states=True)
    yo, fo, so = orc.scan(**oracle_kw(inp), seq_idx=seq, states_chunk=Q)
    s1 = check_close(to_f64(y), yo, io, "y", Y_AXES)
    check_close(to_f64(fin), fo, io, "final_state", STATE_AXES)
    check_close(to_f64(st), so, io, "chunk states", (1, 3, 4))
    log("y max_abs %.3g max_rel %.3g" % (s1[0], s1[1]))


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("init", [0.0, 0.4])
@pytest.mark.parametrize("Q,l", [(64, 300), (100, 250), (256, 256), (32, 33)])
def test_chunk_states_parity(orc, io, init, Q, l):
    """The state after every chunk boundary, [b, chunks, h, n, p]; the last
    one equals the final state."""
    inp = syn.random_case(3100 + Q + l, 2, l, 4, 64, 64, 2, io=io, init_std=init)
    y, fin, st = _run(inp, Q, states=True)
    assert st.shape[1] == -(-l // Q)
    assert torch_mod().equal(st[:, -1], fin)
    yo, fo, so = orc.scan(**oracle_kw(inp), states_chunk=Q)
    check_close(to_f64(y), yo, io, "y", Y_AXES)
    check_close(to_f64(st), so, io, "chunk states", (1, 3, 4))


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_per_token_states(orc, io):
    """chunk 1: the state after every token (nnterp guide, "The state after
    every token"), with packed documents as well."""
    inp = syn.random_case(3200, 2, 40, 4, 32, 64, 1, io=io, init_std=0.2)
    seq = _seq(2, 40, [(9, 10, 30), ()])
    y, st = _run(inp, 1, seq=seq, states=True, final=False)
    assert tuple(st.shape) == (2, 40, 4, 64, 32)
    yo, fo, so = orc.scan(**oracle_kw(inp), seq_idx=seq, states_chunk=1)
    check_close(to_f64(y), yo, io, "y", Y_AXES)
    check_close(to_f64(st), so, io, "per-token states", (1, 3, 4))


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_constant_document_index_changes_nothing(io):
    """A document index that never changes gives the same bits as none."""
    inp = syn.random_case(3300, 2, 333, 4, 64, 128, 2, io=io, init_std=0.1)
    seq = np.full((2, 333), 5, np.int32)
    y0, f0 = _run(inp, 64)
    y1, f1 = _run(inp, 64, seq=seq)
    torch = torch_mod()
    assert torch.equal(y0, y1)
    assert torch.equal(f0, f1)


@pytest.mark.parametrize("case", PACKED[:2], ids=_pid)
def test_packed_is_deterministic(orc, case):
    """Packed documents: two calls give the same bits."""
    b, l, h, p, n, g, Q, init, cuts = case
    inp = syn.random_case(3400 + sum(case[:7]), b, l, h, p, n, g, io="bf16", init_std=init)
    seq = _seq(b, l, cuts)
    y1, f1 = _run(inp, Q, seq=seq)[:2]
    y2, f2 = _run(inp, Q, seq=seq)[:2]
    torch = torch_mod()
    assert torch.equal(y1, y2)
    assert torch.equal(f1, f2)


# (chunk, seqlen, head_dim, state_dim): chunks shorter than one 32-row block
# are computed as whole multiples of themselves, and the states at the
# caller's boundaries are stepped token by token from the computed chunks'
# boundary states
SHORT = [(1, 70, 16, 64), (3, 100, 32, 128), (7, 70, 128, 32), (16, 64, 64, 128),
         (31, 200, 64, 64)]


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("Qs,l,p,n", SHORT, ids=lambda c: str(c))
def test_short_chunk_states(orc, io, Qs, l, p, n):
    inp = syn.random_case(3500 + Qs + l + p + n, 2, l, 4, p, n, 2, io=io, init_std=0.3)
    seq = _seq(2, l, [(5, l // 2, l // 2 + 1), ()])
    y, fin, st = _run(inp, Qs, seq=seq, states=True)
    assert st.shape[1] == -(-l // Qs)
    # the last state is stepped token by token, the final state comes from
    # the chunked pass: equal up to rounding, each checked against the oracle
    yo, fo, so = orc.scan(**oracle_kw(inp), seq_idx=seq, states_chunk=Qs)
    check_close(to_f64(y), yo, io, "y", Y_AXES)
    check_close(to_f64(fin), fo, io, "final_state", STATE_AXES)
    check_close(to_f64(st), so, io, "chunk states", (1, 3, 4))


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_short_chunk_output_independent_of_states_request(io):
    """y and the final state are the same bits whether or not the states
    after every (short) chunk are asked for."""
    inp = syn.random_case(3600, 2, 90, 4, 64, 64, 2, io=io, init_std=0.2)
    y0, f0 = _run(inp, 5)
    y1, f1, _ = _run(inp, 5, states=True)
    torch = torch_mod()
    assert torch.equal(y0, y1)
    assert torch.equal(f0, f1)


def _bench_inputs():
    w = syn.WORKLOADS["mamba2_130m"]
    return w, syn.make_inputs(w)


def test_bench_workload_packed_documents_sampled(orc):
    """bench.py's packed call at full size: 8 x 2048 tokens of the 130m
    shape with its seeded document lengths, the state after every chunk
    written; sampled (batch, head) pairs against the oracle."""
    from gpu_util import PAIR_AXES, sample_pairs
    w, inp = _bench_inputs()
    seq = syn.doc_index(w.seed + 77, w.batch, w.seqlen)
    y, fin, st = _run(inp, w.chunk, seq=seq, states=True)
    pairs = sample_pairs(w.batch, w.heads, 6, seed=11)
    pr = np.asarray(pairs)
    yo, fo, so = orc.scan(**oracle_kw(inp), seq_idx=seq, pairs=pairs, states_chunk=w.chunk)
    torch = torch_mod()
    bi = torch.as_tensor(pr[:, 0], device="cuda")
    hi = torch.as_tensor(pr[:, 1], device="cuda")
    check_close(to_f64(y[bi, :, hi]), yo, "bf16", "y", PAIR_AXES)
    check_close(to_f64(fin[bi, hi]), fo, "bf16", "final_state", PAIR_AXES)
    check_close(to_f64(st[bi, :, hi]), so, "bf16", "chunk states", (1, 2, 3))


def test_bench_workload_per_token_states_sampled(orc):
    """bench.py's per-token call: one 2048-token row of the 130m shape at
    chunk 1 (1.6 GB of states); two heads against the oracle."""
    import mamba_ssd_chunked_chunk_amd as ssd
    w, _ = _bench_inputs()
    inp = syn.make_inputs(w, batch=1)
    torch = torch_mod()
    g = gpu_inputs(inp)
    y, st = ssd.chunk_scan(g["x"], g["dt"], g["A"], g["B"], g["C"], g["D"], chunk_size=1,
                           dt_bias=g["dt_bias"], return_chunk_states=True)
    torch.cuda.synchronize()
    assert tuple(st.shape) == (1, w.seqlen, w.heads, w.state_dim, w.head_dim)
    pairs = [(0, 0), (0, w.heads - 1)]
    yo, fo, so = orc.scan(**oracle_kw(inp), pairs=pairs, states_chunk=1)
    for k, (_, hh) in enumerate(pairs):
        check_close(to_f64(st[0, :, hh]), so[k], "bf16", "per-token states head %d" % hh,
                    (1, 2))
        check_close(to_f64(y[0, :, hh]), yo[k], "bf16", "y head %d" % hh)
    del st
