"""fp64 CPU oracle of the gradients of the Mamba-2 SSD scan.

TEST INFRASTRUCTURE ONLY: the test suite and the benchmark's CPU-baseline
leg are the only users.  The product path never imports, loads or calls
anything here, and nothing here imports the product package.

The forward is the per-head recurrence of the nnterp guide's "Mamba-2"
page (opening section):

    d_t = clamp(softplus(dt_t + dt_bias)),   alpha_t = exp(A d_t)
    h_t = alpha_t h_{t-1} + d_t B_t x_t^T    (h_{t-1} = 0 where a new
                                             document starts)
    y_t = C_t^T h_t + D x_t

For cotangents dy (of every y_t) and d_final (of the last state), the
gradients follow from the adjoint state g_t = dL/dh_t, stepped backwards:

    g_t = C_t dy_t^T + alpha_{t+1} g_{t+1}   (the second term only when
                                             token t+1 continues t's document;
                                             g_{l-1} also receives d_final)

and each input's gradient is read off g_t and the forward states:

    dx_t  = D dy_t + d_t g_t^T B_t          dB_t = d_t g_t x_t (summed over
    dC_t  = h_t dy_t                               the group's heads; dC too)
    da_t  = alpha_t <g_t, h_{t-1}>          (the log decay a_t = A d_t)
    dd_t  = <g_t, B_t x_t^T> + A da_t       dA  = sum d_t da_t
    ddt_t = dd_t * [clamp passes] * softplus'(dt_t + dt_bias)
    d dt_bias = sum ddt,  dD = sum dy . x,  d init = alpha_0 g_0

Readings (the pages give no backward; this is the derivative of the
forward above): the clamp passes the gradient where dt_min <= softplus(z)
<= dt_max (inclusive ends), softplus'(z) = sigmoid(z).
"""
from __future__ import annotations

import math

import numpy as np


def _softplus(z):
    return np.maximum(z, 0.0) + np.log1p(np.exp(-np.abs(z)))


def _sigmoid(z):
    return 0.5 * (1.0 + np.tanh(0.5 * z))


def forward_states(x, dt, A, B, C, D=None, dt_bias=None, dt_softplus=True,
                   dt_limit=(0.0, math.inf), init_state=None, seq_idx=None):
    """The forward in fp64 with every state kept: returns y [b,l,h,p], the
    states after every token hs [b,l,h,n,p], the states the decays act on
    hp [b,l,h,n,p] (h_{t-1}, zero at document starts), d and alpha [b,l,h]."""
    x, dt, B, C = (np.asarray(a, np.float64) for a in (x, dt, B, C))
    A = np.asarray(A, np.float64)
    b, l, h, p = x.shape
    g, n = B.shape[2], B.shape[3]
    hpg = h // g
    z = dt + (0.0 if dt_bias is None else np.asarray(dt_bias, np.float64)[None, None, :])
    sp = _softplus(z) if dt_softplus else z
    d = np.clip(sp, dt_limit[0], dt_limit[1])
    alpha = np.exp(A[None, None, :] * d)
    Dv = np.zeros(h) if D is None else np.asarray(D, np.float64)
    y = np.empty((b, l, h, p))
    hs = np.empty((b, l, h, n, p))
    hprev = np.empty((b, l, h, n, p))
    for bi in range(b):
        for hh in range(h):
            gi = hh // hpg
            H = np.zeros((n, p)) if init_state is None else np.array(init_state[bi, hh], np.float64)
            for t in range(l):
                if seq_idx is not None and t > 0 and seq_idx[bi, t] != seq_idx[bi, t - 1]:
                    H = np.zeros((n, p))
                hprev[bi, t, hh] = H
                H = alpha[bi, t, hh] * H + d[bi, t, hh] * np.outer(B[bi, t, gi], x[bi, t, hh])
                hs[bi, t, hh] = H
                y[bi, t, hh] = C[bi, t, gi] @ H + Dv[hh] * x[bi, t, hh]
    return y, hs, hprev, d, alpha


def scan_grad(x, dt, A, B, C, D=None, dt_bias=None, dt_softplus=True,
              dt_limit=(0.0, math.inf), init_state=None, seq_idx=None, dy=None, d_final=None):
    """Gradients of L = sum(dy * y) + sum(d_final * final_state).

    Inputs as values (float arrays; bf16 inputs widened exactly by the
    caller).  Returns a dict of fp64 arrays: dx [b,l,h,p], ddt [b,l,h],
    dA [h], dB and dC [b,l,g,n], dD [h], d_dt_bias [h], d_init [b,h,n,p]."""
    x, dt, B, C = (np.asarray(a, np.float64) for a in (x, dt, B, C))
    A = np.asarray(A, np.float64)
    b, l, h, p = x.shape
    g, n = B.shape[2], B.shape[3]
    hpg = h // g
    dy = np.zeros((b, l, h, p)) if dy is None else np.asarray(dy, np.float64)
    Dv = np.zeros(h) if D is None else np.asarray(D, np.float64)
    _, hs, hprev, d, alpha = forward_states(x, dt, A, B, C, D, dt_bias, dt_softplus, dt_limit,
                                            init_state, seq_idx)
    z = dt + (0.0 if dt_bias is None else np.asarray(dt_bias, np.float64)[None, None, :])
    sp = _softplus(z) if dt_softplus else z
    gate = ((sp >= dt_limit[0]) & (sp <= dt_limit[1])).astype(np.float64)
    dsp = _sigmoid(z) if dt_softplus else np.ones_like(z)

    out = dict(dx=np.zeros((b, l, h, p)), ddt=np.zeros((b, l, h)), dA=np.zeros(h),
               dB=np.zeros((b, l, g, n)), dC=np.zeros((b, l, g, n)), dD=np.zeros(h),
               d_dt_bias=np.zeros(h), d_init=np.zeros((b, h, n, p)))
    for bi in range(b):
        for hh in range(h):
            gi = hh // hpg
            # the cotangent arriving from beyond token t (decayed), then g_t
            Gn = np.zeros((n, p)) if d_final is None else np.array(d_final[bi, hh], np.float64)
            for t in range(l - 1, -1, -1):
                G = np.outer(C[bi, t, gi], dy[bi, t, hh]) + Gn
                dt_ = d[bi, t, hh]
                out["dx"][bi, t, hh] = Dv[hh] * dy[bi, t, hh] + dt_ * (B[bi, t, gi] @ G)
                out["dB"][bi, t, gi] += dt_ * (G @ x[bi, t, hh])
                out["dC"][bi, t, gi] += hs[bi, t, hh] @ dy[bi, t, hh]
                da = alpha[bi, t, hh] * np.sum(G * hprev[bi, t, hh])
                dd = float(B[bi, t, gi] @ G @ x[bi, t, hh]) + A[hh] * da
                out["dA"][hh] += dt_ * da
                ddt = dd * gate[bi, t, hh] * dsp[bi, t, hh]
                out["ddt"][bi, t, hh] = ddt
                out["d_dt_bias"][hh] += ddt
                out["dD"][hh] += float(dy[bi, t, hh] @ x[bi, t, hh])
                cut = seq_idx is not None and t > 0 and seq_idx[bi, t] != seq_idx[bi, t - 1]
                Gn = np.zeros((n, p)) if cut else alpha[bi, t, hh] * G
            out["d_init"][bi, hh] = Gn
    return out
