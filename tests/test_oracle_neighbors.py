"""Pins of the fp64 oracle of the convolution before the scan and the gated
norm after it, against library routines, closed forms and invariants."""
import math

import numpy as np
import pytest

from oracle import neighbors as nb

H, P, N, G = 2, 4, 3, 1          # heads, head_dim, state_dim, groups
CH = H * P + 2 * G * N           # 14 channels


def _rand(seed, *shape):
    return np.random.default_rng(seed).standard_normal(shape)


def _pre(xbc, w, bias=None, **kw):
    """Pre-activation conv output as one [b, l, ch] array."""
    x, B, C, fin = nb.conv1d_silu(xbc, w, H, P, N, G, bias=bias, apply_silu=False, **kw)
    b, l = xbc.shape[:2]
    return np.concatenate([x.reshape(b, l, -1), B.reshape(b, l, -1), C.reshape(b, l, -1)], -1), fin


def test_silu_values():
    assert nb.silu(0.0) == 0.0
    assert nb.silu(1.0) == pytest.approx(1.0 / (1.0 + math.exp(-1.0)), rel=1e-15)
    assert nb.silu(-1.0) == pytest.approx(-1.0 / (1.0 + math.e), rel=1e-15)
    assert nb.silu(50.0) == pytest.approx(50.0, rel=1e-20)
    assert abs(nb.silu(-800.0)) == 0.0


@pytest.mark.parametrize("K", [1, 2, 4])
def test_conv_equals_numpy_convolve(K):
    """Each channel is a causal FIR filter: numpy's full convolution with the
    taps reversed, truncated to the first l outputs."""
    xbc = _rand(1, 2, 37, CH)
    w = _rand(2, CH, K)
    out, _ = _pre(xbc, w)
    for bi in range(2):
        for c in range(CH):
            ref = np.convolve(xbc[bi, :, c], w[c, ::-1])[:37]
            np.testing.assert_allclose(out[bi, :, c], ref, rtol=1e-13, atol=1e-13)


def test_impulse_response():
    """A unit input at token t0 of channel c leaves tap width-1-j at token
    t0 + j (plus the bias), and the bias elsewhere."""
    K, l, t0, c = 4, 12, 5, 9
    xbc = np.zeros((1, l, CH))
    xbc[0, t0, c] = 1.0
    w = _rand(3, CH, K)
    bias = _rand(4, CH)
    out, _ = _pre(xbc, w, bias=bias)
    exp = np.broadcast_to(bias, (l, CH)).copy()
    for j in range(K):
        exp[t0 + j, c] += w[c, K - 1 - j]
    np.testing.assert_allclose(out[0], exp, rtol=0, atol=1e-15)


def test_causal():
    K = 4
    xbc = _rand(5, 1, 30, CH)
    w = _rand(6, CH, K)
    a, _ = _pre(xbc, w)
    xbc2 = xbc.copy()
    xbc2[:, 17:] = _rand(7, 1, 13, CH)
    b2, _ = _pre(xbc2, w)
    np.testing.assert_array_equal(a[:, :17], b2[:, :17])
    assert not np.allclose(a[:, 17:], b2[:, 17:])


def test_split_order():
    """Channel order: x (head-major), then B, then C (group-major)."""
    l = 3
    xbc = np.zeros((1, l, CH))
    xbc[0, :, :] = np.arange(CH)[None, :]
    w = np.zeros((CH, 2))
    w[:, 1] = 1.0     # identity filter
    x, B, C, _ = nb.conv1d_silu(xbc, w, H, P, N, G, apply_silu=False)
    np.testing.assert_array_equal(x[0, 0], np.arange(H * P).reshape(H, P))
    np.testing.assert_array_equal(B[0, 0], np.arange(H * P, H * P + N).reshape(G, N))
    np.testing.assert_array_equal(C[0, 0], np.arange(H * P + N, CH).reshape(G, N))


def test_silu_applied_elementwise():
    xbc = _rand(8, 1, 20, CH)
    w = _rand(9, CH, 4)
    pre, _ = _pre(xbc, w)
    x, B, C, _ = nb.conv1d_silu(xbc, w, H, P, N, G)
    post = np.concatenate([x.reshape(1, 20, -1), B.reshape(1, 20, -1), C.reshape(1, 20, -1)], -1)
    np.testing.assert_allclose(post, pre / (1 + np.exp(-pre)), rtol=1e-15)


def test_continuation_with_conv_state():
    """Convolving a prefix and then the rest from the prefix's final conv
    state equals convolving the whole sequence at once."""
    K = 4
    xbc = _rand(10, 2, 40, CH)
    w = _rand(11, CH, K)
    bias = _rand(12, CH)
    whole, fin_whole = _pre(xbc, w, bias=bias)
    a, fa = _pre(xbc[:, :23], w, bias=bias)
    np.testing.assert_array_equal(fa, xbc[:, 23 - (K - 1):23])
    b2, fb = _pre(xbc[:, 23:], w, bias=bias, conv_init=fa)
    np.testing.assert_allclose(np.concatenate([a, b2], 1), whole, rtol=1e-14, atol=1e-14)
    np.testing.assert_array_equal(fb, fin_whole)


def test_packed_documents_equal_separate_runs():
    K = 4
    xbc = _rand(13, 1, 50, CH)
    w = _rand(14, CH, K)
    bias = _rand(15, CH)
    init = _rand(16, 1, K - 1, CH)
    cuts = [0, 2, 19, 20, 50]      # documents of 2, 17, 1 and 30 tokens
    seq = np.zeros((1, 50), np.int32)
    for k in range(len(cuts) - 1):
        seq[0, cuts[k]:cuts[k + 1]] = 7 * k
    out, fin = _pre(xbc, w, bias=bias, conv_init=init, seq_idx=seq)
    for k in range(len(cuts) - 1):
        lo, hi = cuts[k], cuts[k + 1]
        sep, sfin = _pre(xbc[:, lo:hi], w, bias=bias, conv_init=init if k == 0 else None)
        np.testing.assert_allclose(out[:, lo:hi], sep, rtol=1e-14, atol=1e-14)
    np.testing.assert_array_equal(fin, sfin)


def test_constant_document_index_changes_nothing():
    xbc = _rand(17, 2, 25, CH)
    w = _rand(18, CH, 3)
    init = _rand(19, 2, 2, CH)
    a, fa = _pre(xbc, w, conv_init=init)
    b2, fb = _pre(xbc, w, conv_init=init, seq_idx=np.full((2, 25), 3, np.int32))
    np.testing.assert_array_equal(a, b2)
    np.testing.assert_array_equal(fa, fb)


def test_norm_unit_rms_per_group():
    y = _rand(20, 5, 24)
    out = nb.gated_norm(y, group_size=8, eps=0.0)
    rms = np.sqrt(np.mean(out.reshape(5, 3, 8) ** 2, axis=2))
    np.testing.assert_allclose(rms, 1.0, rtol=1e-14)


def test_norm_scale_invariant_per_group():
    y = _rand(21, 4, 16)
    s = np.abs(_rand(22, 4, 2)) + 0.5
    ys = (y.reshape(4, 2, 8) * s[:, :, None]).reshape(4, 16)
    np.testing.assert_allclose(nb.gated_norm(ys, group_size=8, eps=0.0),
                               nb.gated_norm(y, group_size=8, eps=0.0), rtol=1e-13)


def test_norm_groups_are_separate_norms():
    y = _rand(23, 3, 12)
    w = _rand(24, 12)
    whole = nb.gated_norm(y, weight=w, group_size=4, eps=1e-3)
    for k in range(3):
        part = nb.gated_norm(y[:, 4 * k:4 * k + 4], weight=w[4 * k:4 * k + 4], eps=1e-3)
        np.testing.assert_allclose(whole[:, 4 * k:4 * k + 4], part, rtol=1e-15)


def test_norm_closed_form_two_channels():
    """[3, 4]: rms = sqrt(12.5 + eps)."""
    out = nb.gated_norm(np.array([[3.0, 4.0]]), weight=np.array([2.0, -1.0]), eps=0.5)
    np.testing.assert_allclose(out, [[6.0 / math.sqrt(13.0), -4.0 / math.sqrt(13.0)]], rtol=1e-15)


def test_gate_limits():
    """silu(z) -> z for large z, -> 0 for very negative z; gate before norm."""
    y = _rand(25, 2, 8)
    big = np.full((2, 8), 60.0)
    np.testing.assert_allclose(nb.gated_norm(y, big, normalize=False), 60.0 * y, rtol=1e-15)
    assert np.all(nb.gated_norm(y, -big * 20, normalize=False) == 0.0)
    z = _rand(26, 2, 8)
    g = y * z / (1 + np.exp(-z))
    np.testing.assert_allclose(nb.gated_norm(y, z, group_size=8, eps=0.0),
                               g / np.sqrt(np.mean(g * g, axis=1, keepdims=True)), rtol=1e-14)
