"""Pins of the fp64 oracle against facts fixed by the pages and by mathematics.

Nothing here compares the oracle with itself: every check is a hand-derived
worked example, an independent closed form (the dual matrix form, causal
linear attention), an exact invariant the nnterp "Mamba-2" page states, or an
algebraic identity of a linear recurrence.  Each is chosen so that a
plausible slip in the oracle (a dropped term, a wrong sign or index, a
transposed operand, read-before-write) fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest

import ssd_synth as syn
from oracle import chunked, quadratic

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_examples.json")


def _lim(v):
    return math.inf if v == "inf" else float(v)


def _case_arrays(c):
    d = c["dims"]
    b, l, h, p, n, g = (d[k] for k in "blhpng")
    arr = lambda v, s: np.array(v, np.float32).reshape(s)
    init = None if c["init_state"] is None else arr(c["init_state"], (b, h, n, p))
    return dict(x=arr(c["x"], (b, l, h, p)), dt=arr(c["dt"], (b, l, h)),
                A=arr(c["A"], (h,)), B=arr(c["B"], (b, l, g, n)),
                C=arr(c["C"], (b, l, g, n)), D=arr(c["D"], (h,)),
                dt_bias=None if c["dt_bias"] is None else arr(c["dt_bias"], (h,)),
                dt_softplus=c["dt_softplus"],
                dt_limit=(_lim(c["dt_limit"][0]), _lim(c["dt_limit"][1])),
                init_state=init)


def _cases():
    with open(GOLDEN) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _cases(), ids=lambda c: c["name"])
def test_worked_examples(oracle_mod, case):
    a = _case_arrays(case)
    y, fin = oracle_mod.scan(**a, io="f32")
    np.testing.assert_allclose(y.reshape(-1), case["y"], rtol=1e-15, atol=1e-15)
    np.testing.assert_allclose(fin.reshape(-1), case["final"], rtol=1e-15, atol=1e-15)


def _small(seed, b=2, l=37, h=4, p=5, n=6, g=2, init=0.3, literal=False, io="f32"):
    return syn.random_case(seed, b, l, h, p, n, g, io=io, init_std=init, literal=literal)


def _kw(inp, **over):
    kw = dict(x=inp["x"], dt=inp["dt"], A=inp["A"], B=inp["B"], C=inp["C"], D=inp["D"],
              dt_bias=inp["dt_bias"], init_state=inp["init_state"], io=inp["io"])
    kw.update(over)
    return kw


def _close(a, b, tol=1e-12):
    scale = max(np.abs(b).max(), 1e-300)
    assert np.abs(a - b).max() <= tol * scale, (np.abs(a - b).max(), scale)


@pytest.mark.parametrize("seed,shape", [
    (11, dict(b=2, l=37, h=4, p=5, n=6, g=2)),
    (12, dict(b=1, l=64, h=3, p=4, n=3, g=3)),
    (13, dict(b=3, l=9, h=6, p=2, n=7, g=1)),
    (14, dict(b=1, l=1, h=2, p=3, n=2, g=2)),
])
@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_matches_dual_form(oracle_mod, seed, shape, io):
    inp = _small(seed, io=io, **shape)
    y, fin = oracle_mod.scan(**_kw(inp))
    yq, fq = quadratic.dual_form(**_kw(inp))
    _close(y, yq)
    _close(fin, fq)


def test_dual_form_with_clamp_and_no_bias(oracle_mod):
    inp = _small(21)
    kw = _kw(inp, dt_bias=None, dt_limit=(0.2, 0.9), D=None)
    _close(oracle_mod.scan(**kw)[0], quadratic.dual_form(**kw)[0])
    kw = _kw(inp, dt_softplus=False, dt_limit=(0.0, math.inf),
             dt=np.abs(inp["dt"]).astype(np.float32))
    _close(oracle_mod.scan(**kw)[0], quadratic.dual_form(**kw)[0])


def test_zero_decay_is_causal_linear_attention(oracle_mod):
    """A = 0: the scan is causal linear attention (nnterp: "linear attention
    with one scalar decay per head"), checked with plain matrix products."""
    inp = _small(31, init=0.5)
    A0 = np.zeros_like(inp["A"])
    y, fin = oracle_mod.scan(**_kw(inp, A=A0))
    d, _ = oracle_mod.process_dt(inp["dt"], A0, inp["dt_bias"])
    # independent time step: numpy logaddexp
    d2 = np.logaddexp(0.0, inp["dt"].astype(np.float64) + inp["dt_bias"].astype(np.float64))
    np.testing.assert_allclose(d, d2, rtol=1e-15)
    yl, fl = quadratic.linear_attention(
        inp["x"].astype(np.float64), inp["B"].astype(np.float64),
        inp["C"].astype(np.float64), d2, D=inp["D"].astype(np.float64),
        init_state=inp["init_state"].astype(np.float64), groups=2)
    _close(y, yl)
    _close(fin, fl)


@pytest.mark.parametrize("Q", [1, 2, 7, 16, 64, 256])
@pytest.mark.parametrize("l", [64, 77])
def test_chunked_equals_sequential(oracle_mod, Q, l):
    inp = _small(41, l=l, b=2, h=4, p=8, n=16, g=2)
    y, fin = oracle_mod.scan(**_kw(inp))
    yc, fc, inter = chunked.chunked_scan(**_kw(inp), chunk=Q)
    _close(yc, y)
    _close(fc, fin)
    # boundary states are the sequential state after each chunk's last token
    nc = -(-l // Q)
    for c in range(1, nc):
        _, fc_prefix = oracle_mod.scan(**_kw(inp, x=inp["x"][:, :c * Q], dt=inp["dt"][:, :c * Q],
                                             B=inp["B"][:, :c * Q], C=inp["C"][:, :c * Q]))
        _close(inter["H_prev"][:, c], fc_prefix)


def test_zero_time_step_is_exact_skip(oracle_mod):
    """dt = 0 writes nothing and decays nothing: the state after token t equals
    the state after t - 1 exactly (nnterp, "betas and decays are one argument")."""
    inp = _small(51, l=12)
    dt = np.abs(inp["dt"]).astype(np.float32)
    dt[:, 5, :] = 0.0
    kw = dict(dt_softplus=False, dt_bias=None)
    _, f5 = oracle_mod.scan(**_kw(inp, x=inp["x"][:, :5], dt=dt[:, :5], B=inp["B"][:, :5],
                                  C=inp["C"][:, :5], **kw))
    _, f6 = oracle_mod.scan(**_kw(inp, x=inp["x"][:, :6], dt=dt[:, :6], B=inp["B"][:, :6],
                                  C=inp["C"][:, :6], **kw))
    assert np.array_equal(f5, f6)


def test_all_zero_decays_keep_zero_state(oracle_mod):
    """decays = 0 everywhere (dt = 0) from a zero state: the state stays zero
    through the prompt and y = D x (nnterp, "Writing decays rewrites betas")."""
    inp = _small(52, init=0.0)
    dt = np.zeros_like(inp["dt"])
    y, fin = oracle_mod.scan(**_kw(inp, dt=dt, dt_softplus=False, dt_bias=None))
    assert np.all(fin == 0.0)
    assert np.array_equal(y, inp["D"][None, None, :, None].astype(np.float64) *
                          inp["x"].astype(np.float64))


def test_decays_nonpositive_and_dt_positive(oracle_mod):
    """Under softplus with A < 0: d > 0 and A d <= 0 (nnterp, "The values":
    decays are non-positive; the printed dt.min() > 0 check)."""
    inp = syn.make_inputs(syn.WORKLOADS["tiny_fp32"])
    d, a = oracle_mod.process_dt(inp["dt"], inp["A"], inp["dt_bias"])
    assert d.min() > 0 and a.max() <= 0


def test_step_continuation_equals_long_forward(oracle_mod):
    """forward(l1) then l2 single steps equals forward(l1 + l2); the state
    handed from one call to the next is continuous (nnterp, "The state
    between steps")."""
    inp = _small(61, l=20)
    l1 = 13
    y, fin = oracle_mod.scan(**_kw(inp))
    y1, st = oracle_mod.scan(**_kw(inp, x=inp["x"][:, :l1], dt=inp["dt"][:, :l1],
                                   B=inp["B"][:, :l1], C=inp["C"][:, :l1]))
    np.testing.assert_array_equal(y1, y[:, :l1])
    for t in range(l1, 20):
        yt, st = oracle_mod.step(st, inp["x"][:, t], inp["dt"][:, t], inp["A"],
                                 inp["B"][:, t], inp["C"][:, t], inp["D"], inp["dt_bias"])
        np.testing.assert_array_equal(yt, y[:, t])
    np.testing.assert_array_equal(st, fin)


def test_split_forward_with_init_state(oracle_mod):
    inp = _small(62, l=30)
    y, fin = oracle_mod.scan(**_kw(inp))
    ya, sa = oracle_mod.scan(**_kw(inp, x=inp["x"][:, :11], dt=inp["dt"][:, :11],
                                   B=inp["B"][:, :11], C=inp["C"][:, :11]))
    yb, sb = oracle_mod.scan(**_kw(inp, x=inp["x"][:, 11:], dt=inp["dt"][:, 11:],
                                   B=inp["B"][:, 11:], C=inp["C"][:, 11:], init_state=sa))
    np.testing.assert_array_equal(np.concatenate([ya, yb], 1), y)
    np.testing.assert_array_equal(sb, fin)


def test_linearity_and_superposition(oracle_mod):
    inp = _small(71, init=0.0)
    y, f = oracle_mod.scan(**_kw(inp))
    y3, f3 = oracle_mod.scan(**_kw(inp, x=(4.0 * inp["x"]).astype(np.float32)))
    _close(y3, 4.0 * y)
    _close(f3, 4.0 * f)
    H0 = (0.7 * np.random.default_rng(1).standard_normal(f.shape)).astype(np.float32)
    yh, fh = oracle_mod.scan(**_kw(inp, init_state=H0))
    y0, f0 = oracle_mod.scan(**_kw(inp, x=np.zeros_like(inp["x"]), init_state=H0))
    _close(yh, y + y0)
    _close(fh, f + f0)


def test_batch_and_head_permutation(oracle_mod):
    inp = _small(72, b=3, h=4, g=1)
    y, f = oracle_mod.scan(**_kw(inp))
    pb, ph = np.array([2, 0, 1]), np.array([3, 1, 0, 2])
    kw = _kw(inp, x=inp["x"][pb][:, :, ph], dt=inp["dt"][pb][:, :, ph], B=inp["B"][pb],
             C=inp["C"][pb], A=inp["A"][ph], D=inp["D"][ph], dt_bias=inp["dt_bias"][ph],
             init_state=inp["init_state"][pb][:, ph])
    yp, fp = oracle_mod.scan(**kw)
    np.testing.assert_array_equal(yp, y[pb][:, :, ph])
    np.testing.assert_array_equal(fp, f[pb][:, ph])


def test_group_expansion(oracle_mod):
    """g groups equal h groups with each group's B, C repeated for its
    contiguous block of heads (np.repeat defines the head -> group map)."""
    inp = _small(73, h=6, g=3)
    y, f = oracle_mod.scan(**_kw(inp))
    rep = 2
    yx, fx = oracle_mod.scan(**_kw(inp, B=np.repeat(inp["B"], rep, axis=2),
                                   C=np.repeat(inp["C"], rep, axis=2)))
    np.testing.assert_array_equal(y, yx)
    np.testing.assert_array_equal(f, fx)


def test_extreme_decays_stay_finite(oracle_mod):
    """A = -16 with large dt: cumulative log decay below -1e4; everything stays
    finite and the state decays (kongchang "Mamba2": a NaN in a chunk-scan
    kernel was a numerical-stability defect)."""
    inp = _small(81, l=200, init=1.0)
    A = np.full_like(inp["A"], -16.0)
    dt = (np.abs(inp["dt"]) + 10.0).astype(np.float32)
    y, f = oracle_mod.scan(**_kw(inp, A=A, dt=dt))
    d, a = oracle_mod.process_dt(dt, A, inp["dt_bias"])
    assert a.sum(axis=1).max() < -1e4
    assert np.isfinite(y).all() and np.isfinite(f).all()


def test_oracle_time_step_large_and_small_arguments(oracle_mod):
    """softplus(z) -> z for large z and -> e^z for very negative z, without
    overflow; clamps apply after the softplus."""
    dt = np.array([[[800.0, -50.0, 0.0]]], np.float32)
    A = np.array([-1.0, -1.0, -2.0], np.float32)
    d, a = oracle_mod.process_dt(dt, A)
    assert d[0, 0, 0] == 800.0
    assert d[0, 0, 1] == pytest.approx(math.exp(-50.0), rel=1e-12)
    assert d[0, 0, 2] == pytest.approx(math.log(2.0), rel=1e-15)
    assert a[0, 0, 2] == pytest.approx(-2.0 * math.log(2.0), rel=1e-15)
    d, _ = oracle_mod.process_dt(dt, A, dt_limit=(0.5, 10.0))
    np.testing.assert_array_equal(d[0, 0], [10.0, 0.5, math.log(2.0)])


def test_softplus_closed_forms():
    from oracle import quadratic as q
    z = np.array([-30.0, -1.0, 0.0, math.log(math.e - 1.0), 1.0, 25.0, 700.0])
    d = q.time_step(z, None, True, (0.0, math.inf))
    assert d[2] == pytest.approx(math.log(2.0), rel=1e-15)
    assert d[3] == pytest.approx(1.0, rel=1e-15)
    assert d[-1] == 700.0
    # inverse used for dt_bias: softplus(softplus_inv(y)) = y
    ys = np.exp(np.linspace(math.log(1e-3), math.log(0.1), 50))
    np.testing.assert_allclose(q.time_step(syn.softplus_inv(ys), None, True,
                                           (0.0, math.inf)), ys, rtol=1e-14)


def test_bf16_rounding_matches_torch():
    import torch
    v = np.random.default_rng(5).standard_normal(100000).astype(np.float32) * 7
    v[:4] = [0.0, -0.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8]   # ties
    ours = syn.bf16_round(v)
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)
    np.testing.assert_array_equal(syn.bf16_to_f32(ours),
                                  torch.from_numpy(ref.view(np.int16)).view(torch.bfloat16)
                                  .float().numpy())


def test_synth_deterministic_and_distributions():
    w = syn.WORKLOADS["tiny_fp32"]
    a, b = syn.make_inputs(w), syn.make_inputs(w)
    for k in ("x", "dt", "A", "B", "C", "dt_bias"):
        np.testing.assert_array_equal(a[k], b[k])
    assert a["A"].min() >= -16.0 and a["A"].max() <= -1.0
    lo, hi = syn.softplus_inv(1e-3), syn.softplus_inv(0.1)
    assert a["dt_bias"].min() >= lo - 1e-5 and a["dt_bias"].max() <= hi + 1e-5
    s = syn.make_step_inputs(syn.WORKLOADS["decode_2p7b"], 3, batch=2)
    assert s["x"].shape == (2, 80, 64) and s["x"].dtype == np.uint16


# ---------------------------------------------------------------------------
# Packed sequences and the chunk-boundary states output.

def _slice(inp, t0, t1):
    return dict(x=inp["x"][:, t0:t1], dt=inp["dt"][:, t0:t1], B=inp["B"][:, t0:t1],
                C=inp["C"][:, t0:t1])


@pytest.mark.parametrize("cuts", [(11,), (5, 6, 30), (1, 36)])
def test_packed_sequences_equal_separate_runs(oracle_mod, cuts):
    """Documents packed into one row with a per-token document index behave
    as if run one by one: the first from the initial state, every later one
    from a zero state; the final state is the last document's.  (Sample
    packing with a reset at document boundaries, the packing fix on the
    Mamba2 news page.)  Includes a one-token document."""
    inp = _small(81, l=37)
    b, l = inp["x"].shape[:2]
    edges = (0,) + tuple(cuts) + (l,)
    seq = np.zeros((b, l), np.int32)
    for k in range(len(edges) - 1):
        seq[:, edges[k]:edges[k + 1]] = 3 * k + 1
    y, fin = oracle_mod.scan(**_kw(inp), seq_idx=seq)
    init = inp["init_state"]
    for k in range(len(edges) - 1):
        t0, t1 = edges[k], edges[k + 1]
        yk, fk = oracle_mod.scan(**_kw(inp, **_slice(inp, t0, t1),
                                       init_state=init if k == 0 else None))
        np.testing.assert_array_equal(y[:, t0:t1], yk)
    np.testing.assert_array_equal(fin, fk)


def test_constant_document_index_changes_nothing(oracle_mod):
    inp = _small(82)
    y, fin = oracle_mod.scan(**_kw(inp))
    seq = np.full(inp["x"].shape[:2], 7, np.int32)
    ys, fs = oracle_mod.scan(**_kw(inp), seq_idx=seq)
    np.testing.assert_array_equal(ys, y)
    np.testing.assert_array_equal(fs, fin)


@pytest.mark.parametrize("chunk", [1, 5, 37, 64])
def test_chunk_states_are_prefix_final_states(oracle_mod, chunk):
    """The state after every chunk boundary is the final state of the prompt
    cut at that boundary, and the last one is the final state (nnterp, "The
    state after every token": states[:, -1] equals the final state)."""
    inp = _small(83, l=37)
    l = inp["x"].shape[1]
    y, fin, states = oracle_mod.scan(**_kw(inp), states_chunk=chunk)
    assert states.shape[1] == -(-l // chunk)
    np.testing.assert_array_equal(states[:, -1], fin)
    for c in range(states.shape[1]):
        t1 = min((c + 1) * chunk, l)
        _, fc = oracle_mod.scan(**_kw(inp, **_slice(inp, 0, t1)))
        np.testing.assert_array_equal(states[:, c], fc)


def test_per_token_states_hold_at_a_zero_time_step(oracle_mod):
    """With one state per token, a zero time step at token 3 leaves the state
    after token 3 equal to the state after token 2 (nnterp, "The state after
    every token": held[:, 3] equals held[:, 2] with betas[:, 3] = 0)."""
    inp = _small(84, l=10)
    dt = np.abs(inp["dt"]).astype(np.float32)
    dt[:, 3, :] = 0.0
    _, _, states = oracle_mod.scan(**_kw(inp, dt=dt, dt_softplus=False, dt_bias=None),
                                   states_chunk=1)
    np.testing.assert_array_equal(states[:, 3], states[:, 2])
    assert not np.array_equal(states[:, 4], states[:, 3])


def test_chunk_states_with_packed_sequences(oracle_mod):
    """Chunk states of a packed row are the prefix states of the same packed
    row, and a boundary state right after a document ends is that
    document's final state."""
    inp = _small(85, l=30)
    seq = np.zeros(inp["x"].shape[:2], np.int32)
    seq[:, 10:] = 1
    _, fin, states = oracle_mod.scan(**_kw(inp), seq_idx=seq, states_chunk=10)
    _, f_doc0 = oracle_mod.scan(**_kw(inp, **_slice(inp, 0, 10)))
    np.testing.assert_array_equal(states[:, 0], f_doc0)
    np.testing.assert_array_equal(states[:, -1], fin)
    _, f20 = oracle_mod.scan(**_kw(inp, **_slice(inp, 0, 20)), seq_idx=seq[:, :20])
    np.testing.assert_array_equal(states[:, 1], f20)
