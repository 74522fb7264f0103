"""The two-stage chunked SSD algorithm, step by step in fp64 (numpy).

TEST INFRASTRUCTURE ONLY.  It follows the chunked form described on the
kongchang "Mamba2" page (chunk-scan entry: parallel inside a chunk, serial
across chunks; matrix-multiplication form) and the nnterp guide, "Mamba-2"
page, section "The state after every token" (the scan holds the state at
every chunk boundary, each obtained cumulatively from the initial state).
The steps, in order, for chunk c of length Q (the last one may be shorter):

  1. d = clamp(softplus(dt + dt_bias)), a = A d, and cs = inclusive cumsum
     of a restarted at each chunk start;
  2. S_c = B_c^T diag(exp(cs_last - cs) d) X_c       (chunk state from zero);
  3. H_prev[c] = H; H = exp(cs_last) H + S_c        (serial over chunks);
  4. Y_diag = ((C_c B_c^T) o L o d_j) X_c with L_ij = exp(cs_i - cs_j), j <= i;
  5. y = Y_diag + exp(cs_i) C_c^T H_prev[c] + D x.

The intermediates (cs, S, H_prev, Y_diag) are returned so that a stage of a
faster implementation can be compared with the matching step here.  Its only
tie to the sequential oracle is the test asserting both agree.
"""
from __future__ import annotations

import math

import numpy as np


def _widen(a, io):
    a = np.asarray(a)
    if io == "bf16":
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def chunked_scan(x, dt, A, B, C, D=None, dt_bias=None, dt_softplus=True,
                 dt_limit=(0.0, math.inf), init_state=None, io="f32", chunk=64):
    X = _widen(x, io)
    Bm = _widen(B, io)
    Cm = _widen(C, io)
    raw = _widen(dt, io)
    b, l, h, p = X.shape
    g, n = Bm.shape[2], Bm.shape[3]
    Q = int(chunk)
    nc = -(-l // Q)
    A = np.asarray(A, np.float64)
    z = raw + (0.0 if dt_bias is None else np.asarray(dt_bias, np.float64))
    # softplus(z) = max(z, 0) + log(1 + exp(-|z|))
    d = (np.maximum(z, 0.0) + np.log1p(np.exp(-np.abs(z)))) if dt_softplus else z
    d = np.minimum(np.maximum(d, dt_limit[0]), dt_limit[1])          # [b,l,h]
    a = d * A[None, None, :]
    # head-major views, [b,h,l]
    dh = np.transpose(d, (0, 2, 1))
    ah = np.transpose(a, (0, 2, 1))
    grp = np.arange(h) // (h // g)
    Bh = Bm[:, :, grp, :]                                              # [b,l,h,n]
    Ch = Cm[:, :, grp, :]

    # step 1: per-chunk inclusive cumsum
    cs = np.zeros((b, h, l))
    for c in range(nc):
        r0, r1 = c * Q, min(l, (c + 1) * Q)
        cs[:, :, r0:r1] = np.cumsum(ah[:, :, r0:r1], axis=2)

    # step 2: chunk states from zero
    S = np.zeros((b, nc, h, n, p))
    cs_last = np.zeros((b, h, nc))
    for c in range(nc):
        r0, r1 = c * Q, min(l, (c + 1) * Q)
        last = cs[:, :, r1 - 1]                                        # [b,h]
        cs_last[:, :, c] = last
        w = np.exp(last[:, :, None] - cs[:, :, r0:r1]) * dh[:, :, r0:r1]   # [b,h,q]
        S[:, c] = np.einsum("bqhn,bhq,bqhp->bhnp", Bh[:, r0:r1], w, X[:, r0:r1])

    # step 3: serial state passing
    H = np.zeros((b, h, n, p)) if init_state is None else np.array(init_state, np.float64)
    Hprev = np.zeros((b, nc, h, n, p))
    for c in range(nc):
        Hprev[:, c] = H
        H = np.exp(cs_last[:, :, c])[:, :, None, None] * H + S[:, c]
    final = H

    # steps 4-5: per-chunk outputs
    Ydiag = np.zeros((b, l, h, p))
    y = np.zeros((b, l, h, p))
    Dv = np.zeros(h) if D is None else np.asarray(D, np.float64)
    for c in range(nc):
        r0, r1 = c * Q, min(l, (c + 1) * Q)
        q = r1 - r0
        csq = cs[:, :, r0:r1]                                          # [b,h,q]
        tri = np.tril(np.ones((q, q), bool))
        diff = np.where(tri, csq[:, :, :, None] - csq[:, :, None, :], -np.inf)
        L = np.exp(diff)                                               # select, then exp
        G = np.einsum("bihn,bjhn->bhij", Ch[:, r0:r1], Bh[:, r0:r1])
        M = G * L * dh[:, :, None, r0:r1]
        Ydiag[:, r0:r1] = np.einsum("bhij,bjhp->bihp", M, X[:, r0:r1])
        off = np.einsum("bihn,bhnp->bihp", Ch[:, r0:r1], Hprev[:, c])
        y[:, r0:r1] = Ydiag[:, r0:r1] + np.exp(np.transpose(csq, (0, 2, 1)))[..., None] * off \
            + Dv[None, None, :, None] * X[:, r0:r1]
    inter = dict(d=dh, cs=cs, cs_last=cs_last, S=S, H_prev=Hprev, Y_diag=Ydiag)
    return y, final, inter
