"""The sequence-segment identity the segment entry points rely on, checked
with the oracle alone: segments scanned from a zero state, combined through
entry_{k+1} = exp(L_k) entry_k + S_k, and scanned again from their entry
states, give one pass's y and final state."""
import math

import numpy as np
import pytest

import oracle
import ssd_synth as syn


def _d(dt, bias):
    z = np.asarray(dt, np.float64) + np.asarray(bias, np.float64)[None, None, :]
    return np.maximum(z, 0) + np.log1p(np.exp(-np.abs(z)))


@pytest.mark.parametrize("init", [0.0, 0.3])
@pytest.mark.parametrize("packed", [False, True])
def test_segments_recompose_one_pass(init, packed):
    b, l, h, p, n, g = 2, 200, 3, 8, 4, 1
    inp = syn.random_case(61, b, l, h, p, n, g, init_std=init)
    seq = None
    if packed:
        seq = np.zeros((b, l), np.int32)
        seq[0, 40:] = 1
        seq[0, 150:] = 2     # a document starting exactly at a segment start
        seq[1, 90:] = 5      # one crossing a segment boundary
    cuts = [0, 70, 150, 200]
    yf, ff = oracle.scan(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp["D"],
                         inp["dt_bias"], init_state=inp["init_state"], seq_idx=seq)
    d = _d(inp["dt"], inp["dt_bias"])
    cur = np.zeros((b, h, n, p)) if inp["init_state"] is None else inp["init_state"].astype(np.float64)
    for k in range(len(cuts) - 1):
        lo, hi = cuts[k], cuts[k + 1]
        part = {key: inp[key][:, lo:hi] for key in ("x", "dt", "B", "C")}
        sq = None if seq is None else seq[:, lo:hi]
        if seq is not None and lo > 0:
            cur = cur * (seq[:, lo] == seq[:, lo - 1])[:, None, None, None]
        # pass 1: from zero
        _, S = oracle.scan(part["x"], part["dt"], inp["A"], part["B"], part["C"], inp["D"],
                           inp["dt_bias"], seq_idx=sq)
        L = np.sum(inp["A"][None, None, :] * d[:, lo:hi], axis=1)
        if sq is not None:
            L = np.where((sq[:, 1:] != sq[:, :-1]).any(axis=1)[:, None], -np.inf, L)
        # pass 2: from the entry state
        y2, f2 = oracle.scan(part["x"], part["dt"], inp["A"], part["B"], part["C"], inp["D"],
                             inp["dt_bias"], init_state=cur, seq_idx=sq)
        np.testing.assert_allclose(y2, yf[:, lo:hi], rtol=1e-9, atol=1e-9)
        nxt = np.exp(L)[:, :, None, None] * cur + S
        np.testing.assert_allclose(nxt, f2, rtol=1e-9, atol=1e-9)
        cur = nxt
    np.testing.assert_allclose(cur, ff, rtol=1e-9, atol=1e-9)
