"""Pins of the fp64 gradient oracle (oracle/backward.py): its forward against
the C oracle, every gradient against central finite differences of the
forward, packed documents against separate runs, and linearity in the
cotangents."""
import math

import numpy as np
import pytest

import oracle
from oracle import backward as bw


def _case(seed, b=2, l=9, h=2, p=3, n=2, g=1, init=True, seq=True):
    r = np.random.default_rng(seed)
    c = dict(x=r.standard_normal((b, l, h, p)), dt=r.standard_normal((b, l, h)) * 0.7,
             A=-np.exp(r.uniform(0, math.log(4), h)), B=r.standard_normal((b, l, g, n)),
             C=r.standard_normal((b, l, g, n)), D=r.standard_normal(h),
             dt_bias=r.uniform(-1, 0.5, h))
    if init:
        c["init_state"] = r.standard_normal((b, h, n, p))
    if seq:
        s = np.zeros((b, l), np.int64)
        s[0, 4:] = 1          # two documents in row 0
        c["seq_idx"] = s
    cot = dict(dy=r.standard_normal((b, l, h, p)), d_final=r.standard_normal((b, h, n, p)))
    return c, cot


def _loss(c, cot, **kw):
    y, hs, _, _, _ = bw.forward_states(**{**c, **kw})
    return float(np.sum(cot["dy"] * y) + np.sum(cot["d_final"] * hs[:, -1]))


def test_forward_matches_c_oracle():
    c, _ = _case(1, b=2, l=17, h=4, p=4, n=3, g=2)
    # the C oracle takes fp32 inputs: give both sides the same fp32 values
    c = {k: (v if k == "seq_idx" else np.asarray(v, np.float32).astype(np.float64))
         for k, v in c.items()}
    y, hs, _, _, _ = bw.forward_states(**c)
    f = {k: np.asarray(v, np.float32) for k, v in c.items() if k != "seq_idx"}
    yo, fo = oracle.scan(f["x"], f["dt"], f["A"], f["B"], f["C"], f["D"], f["dt_bias"],
                         init_state=c["init_state"], seq_idx=c["seq_idx"])
    np.testing.assert_allclose(y, yo, rtol=1e-10, atol=1e-10)
    np.testing.assert_allclose(hs[:, -1], fo, rtol=1e-10, atol=1e-10)


@pytest.mark.parametrize("limit", [(0.0, math.inf), (0.05, 0.6)])
@pytest.mark.parametrize("softplus", [True, False])
def test_gradients_match_finite_differences(limit, softplus):
    c, cot = _case(2)
    if not softplus:
        c["dt"] = np.abs(c["dt"]) + 0.1   # d = dt + bias stays positive
        c["dt_bias"] = np.abs(c["dt_bias"]) * 0.1
    kw = dict(dt_softplus=softplus, dt_limit=limit)
    gr = bw.scan_grad(**c, **kw, **cot)
    names = dict(x="dx", dt="ddt", A="dA", B="dB", C="dC", D="dD", dt_bias="d_dt_bias",
                 init_state="d_init")
    eps = 1e-6
    for name, gname in names.items():
        base = c[name]
        num = np.zeros_like(base)
        for idx in np.ndindex(base.shape):
            hi = base.copy()
            lo = base.copy()
            hi[idx] += eps
            lo[idx] -= eps
            num[idx] = (_loss({**c, name: hi}, cot, **kw) - _loss({**c, name: lo}, cot, **kw)) / (2 * eps)
        scale = max(1.0, float(np.abs(num).max()))
        np.testing.assert_allclose(gr[gname], num, rtol=0, atol=2e-7 * scale, err_msg=name)


def test_clamp_stops_the_time_step_gradient():
    c, cot = _case(3, init=False, seq=False)
    gr = bw.scan_grad(**c, dt_limit=(10.0, 20.0), **cot)   # every d clamped to 10
    assert np.all(gr["ddt"] == 0.0) and np.all(gr["d_dt_bias"] == 0.0)


def test_packed_documents_equal_separate_runs():
    c, cot = _case(4, b=1, l=12, seq=False)
    cut = 5
    seq = np.zeros((1, 12), np.int64)
    seq[0, cut:] = 3
    gp = bw.scan_grad(**c, seq_idx=seq, **cot)
    first = {k: (v[:, :cut] if k in ("x", "dt", "B", "C") else v) for k, v in c.items()}
    second = {k: (v[:, cut:] if k in ("x", "dt", "B", "C") else v) for k, v in c.items()
              if k != "init_state"}
    g1 = bw.scan_grad(**first, dy=cot["dy"][:, :cut], d_final=None)
    g2 = bw.scan_grad(**second, dy=cot["dy"][:, cut:], d_final=cot["d_final"])
    for k in ("dx", "ddt", "dB", "dC"):
        np.testing.assert_allclose(gp[k], np.concatenate([g1[k], g2[k]], 1), rtol=1e-12,
                                   atol=1e-12, err_msg=k)
    for k in ("dA", "dD", "d_dt_bias"):
        np.testing.assert_allclose(gp[k], g1[k] + g2[k], rtol=1e-12, atol=1e-12, err_msg=k)
    np.testing.assert_allclose(gp["d_init"], g1["d_init"], rtol=1e-12, atol=1e-12)


def test_linear_in_cotangents():
    c, cot = _case(5)
    _, cot2 = _case(6)
    ga = bw.scan_grad(**c, **cot)
    gb = bw.scan_grad(**c, **cot2)
    gab = bw.scan_grad(**c, dy=2 * cot["dy"] - cot2["dy"],
                       d_final=2 * cot["d_final"] - cot2["d_final"])
    for k in ga:
        np.testing.assert_allclose(gab[k], 2 * ga[k] - gb[k], rtol=1e-10, atol=1e-10, err_msg=k)
