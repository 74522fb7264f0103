"""The SSD scan as one masked matrix product per head (fp64, numpy).

TEST INFRASTRUCTURE ONLY (pins the sequential oracle on small inputs).

Unrolling the recurrence of the nnterp guide, "Mamba-2" page, opening
section (h_t = exp(a_t) h_{t-1} + d_t B_t x_t^T, y_t = C_t^T h_t + D x_t,
with a_t = A d_t the log decay of section "The values") gives the closed
"dual" form that the kongchang "Mamba2" page calls the matrix-multiplication
form:

    y_t   = sum_{j<=t} (C_t . B_j) exp(sum_{k=j+1..t} a_k) d_j x_j
            + exp(sum_{k<=t} a_k) C_t^T H0 + D x_t
    final = sum_j exp(sum_{k>j} a_k) d_j B_j x_j^T + exp(sum_k a_k) H0

This module evaluates exactly that: a lower-triangular l x l decay matrix
built from explicit segment sums, an l x l score matrix C B^T, and numpy
matrix products.  The processed time step uses numpy's logaddexp(0, z) for
softplus.  It shares no code with ssd_oracle.c.
"""
from __future__ import annotations

import math

import numpy as np


def _widen(a, io):
    a = np.asarray(a)
    if io == "bf16":
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def time_step(dt_raw, dt_bias, dt_softplus, dt_limit):
    """d = clamp(softplus(dt + dt_bias)) with softplus(z) = log(e^0 + e^z)."""
    z = dt_raw + (0.0 if dt_bias is None else dt_bias)
    d = np.logaddexp(0.0, z) if dt_softplus else z
    return np.clip(d, dt_limit[0], dt_limit[1])


def segment_sums(a):
    """seg[t, j] = sum_{k=j+1..t} a_k for j <= t (explicit sums), -inf above."""
    l = a.shape[0]
    seg = np.full((l, l), -np.inf)
    for j in range(l):
        seg[j, j] = 0.0
        if j + 1 < l:
            seg[j + 1:, j] = np.cumsum(a[j + 1:])
    return seg


def dual_form(x, dt, A, B, C, D=None, dt_bias=None, dt_softplus=True,
              dt_limit=(0.0, math.inf), init_state=None, io="f32"):
    """Returns y [b,l,h,p] and final [b,h,n,p], both fp64."""
    X = _widen(x, io)
    Bm = _widen(B, io)
    Cm = _widen(C, io)
    raw = _widen(dt, io)
    b, l, h, p = X.shape
    g, n = Bm.shape[2], Bm.shape[3]
    A = np.asarray(A, np.float64)
    bias = None if dt_bias is None else np.asarray(dt_bias, np.float64)
    Dv = np.zeros(h) if D is None else np.asarray(D, np.float64)
    y = np.zeros((b, l, h, p))
    fin = np.zeros((b, h, n, p))
    per_group = h // g
    for bi in range(b):
        d_all = time_step(raw[bi], bias, dt_softplus, dt_limit)          # [l, h]
        for hh in range(h):
            gi = hh // per_group
            d = d_all[:, hh]
            a = A[hh] * d
            seg = segment_sums(a)
            decay = np.exp(seg)                                           # 0 above diagonal
            H0 = np.zeros((n, p)) if init_state is None else \
                np.asarray(init_state, np.float64)[bi, hh]
            Cg, Bg, Xh = Cm[bi, :, gi, :], Bm[bi, :, gi, :], X[bi, :, hh, :]
            scores = Cg @ Bg.T                                            # [l, l]
            total = np.cumsum(a)                                          # sum_{k<=t} a_k
            y[bi, :, hh, :] = (scores * decay * d[None, :]) @ Xh \
                + np.exp(total)[:, None] * (Cg @ H0) + Dv[hh] * Xh
            if l:
                tail = seg[l - 1, :]                                      # sum_{k>j} a_k
                fin[bi, hh] = (Bg * (np.exp(tail) * d)[:, None]).T @ Xh \
                    + np.exp(total[-1]) * H0
            else:
                fin[bi, hh] = H0
    return y, fin


def linear_attention(x, B, C, d, D=None, init_state=None, groups=1):
    """A = 0 special case: causal linear attention (textbook form).

    Y = tril(C B^T) diag(d) X + D X,  final = B^T diag(d) X + H0, per head.
    x [b,l,h,p] fp64, B, C [b,l,g,n] fp64, d [b,l,h] fp64.
    """
    b, l, h, p = x.shape
    n = B.shape[3]
    y = np.zeros_like(x)
    fin = np.zeros((b, h, n, p))
    for bi in range(b):
        for hh in range(h):
            gi = hh // (h // groups)
            Cg, Bg = C[bi, :, gi], B[bi, :, gi]
            H0 = np.zeros((n, p)) if init_state is None else init_state[bi, hh]
            Xd = d[bi, :, hh][:, None] * x[bi, :, hh]
            y[bi, :, hh] = np.tril(Cg @ Bg.T) @ Xd + Cg @ H0
            if D is not None:
                y[bi, :, hh] += D[hh] * x[bi, :, hh]
            fin[bi, hh] = Bg.T @ Xd + H0
    return y, fin
