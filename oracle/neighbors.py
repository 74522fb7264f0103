"""fp64 CPU oracle of the two steps around the scan in a Mamba-2 mixer.

TEST INFRASTRUCTURE ONLY: the test suite and the benchmark's CPU-baseline
leg are the only users.  The product path never imports, loads or calls
anything here, and nothing here imports the product package.

* `conv1d_silu` -- the short causal convolution in front of the scan (the
  transformers issue page on the two paths of a Mamba-2 layer: the causal
  conv1d, then the chunk scan, or both fused with the split of its output).
  Each channel of the packed x | B | C projection is convolved over time
  with its own taps, shifted by a bias, passed through SiLU and split into
  the scan's x, B and C.
* `gated_norm` -- the steps after the scan (nnterp guide: the heads' y is
  read before the gated norm and the output projection; on Falcon-H1 with
  its RMS norm off, y is gated by silu(z)): y * silu(z), then an RMS norm
  over groups of channels with a per-channel weight.

The pages name these steps without defining them; the readings taken (the
plainest ones the rest supports) are:

* the convolution is depthwise and causal: output t of channel c is
  bias[c] + sum_k weight[c, k] * input[t - (width - 1) + k, c], inputs
  before token 0 being the `conv_init` rows (zeros if absent);
* channels are ordered x (heads * head_dim, head-major), then B, then C
  (groups * state_dim each, group-major), as the scan's inputs are laid out;
* with a per-token document index, a tap reads zero where its source token
  belongs to another document (packed documents do not see each other, as
  in the scan); the `conv_init` rows belong to the row's first document;
* `conv_final` holds the last width - 1 inputs as the next token's window
  sees them (rows of earlier documents zero);
* the gate is y * silu(z) with silu(v) = v / (1 + exp(-v)); the norm divides
  each group of `group_size` consecutive channels by sqrt(mean(v^2) + eps)
  and multiplies by the channel's weight (gate first, then the norm).

Parity unpinned: none of these conventions is fixed by a page example; the
pins in tests/test_oracle_neighbors.py check the arithmetic against library
routines, closed forms and invariants.
"""
from __future__ import annotations

from typing import Optional

import numpy as np


def silu(v):
    """v / (1 + exp(-v)) in fp64 (exp overflows to inf for v << 0: the
    quotient is then -0)."""
    v = np.asarray(v, np.float64)
    with np.errstate(over="ignore"):
        return v / (1.0 + np.exp(-v))


def conv1d_silu(xbc, weight, heads, head_dim, state_dim, groups, bias=None, conv_init=None,
                seq_idx=None, apply_silu=True):
    """Causal depthwise convolution over time, SiLU, split.

    xbc        [b, l, ch] (ch = heads*head_dim + 2*groups*state_dim), values
               at the io precision
    weight     [ch, width] taps; tap width-1 multiplies the current token
    bias       [ch] or None
    conv_init  [b, width-1, ch] inputs before token 0, oldest first, or None
    seq_idx    [b, l] document index, or None
    Returns x [b,l,h,p], B [b,l,g,n], C [b,l,g,n], conv_final [b,width-1,ch]
    (all fp64).
    """
    xbc = np.asarray(xbc, np.float64)
    w = np.asarray(weight, np.float64)
    b, l, ch = xbc.shape
    K = w.shape[1]
    hp, gn = heads * head_dim, groups * state_dim
    assert ch == hp + 2 * gn and w.shape[0] == ch
    init = np.zeros((b, K - 1, ch)) if conv_init is None else np.asarray(conv_init, np.float64)
    # the inputs with the K-1 rows before token 0 in front: row s + K - 1 is token s
    src = np.concatenate([init, xbc], axis=1)
    if seq_idx is not None:
        seq = np.asarray(seq_idx)
        # document of every source row (the init rows belong to token 0's)
        doc = np.concatenate([np.repeat(seq[:, :1], K - 1, axis=1), seq], axis=1)
    out = np.zeros((b, l, ch))
    if bias is not None:
        out += np.asarray(bias, np.float64)[None, None, :]
    for k in range(K):
        # tap k reads token t - (K-1) + k, i.e. source row t + k
        term = w[None, None, :, k] * src[:, k:k + l, :]
        if seq_idx is not None:
            same = doc[:, k:k + l] == seq
            term = term * same[:, :, None]
        out += term
    if apply_silu:
        out = silu(out)
    x = out[:, :, :hp].reshape(b, l, heads, head_dim)
    B = out[:, :, hp:hp + gn].reshape(b, l, groups, state_dim)
    C = out[:, :, hp + gn:].reshape(b, l, groups, state_dim)
    fin = src[:, l:l + K - 1, :].copy()
    if seq_idx is not None:
        last = doc[:, l:l + K - 1] == seq[:, -1:]
        fin *= last[:, :, None]
    return x, B, C, fin


def gated_norm(y, z=None, weight=None, group_size=None, eps=1e-5, normalize=True):
    """y [rows, dim] (heads' outputs, flattened), z [rows, dim] or None.

    v = y * silu(z) (v = y without z); with normalize, each group of
    group_size channels is divided by sqrt(mean(v^2) + eps) and multiplied
    by weight (ones if None)."""
    v = np.asarray(y, np.float64)
    if z is not None:
        v = v * silu(z)
    if not normalize:
        return v
    rows, dim = v.shape
    G = dim if group_size is None else group_size
    assert dim % G == 0
    vg = v.reshape(rows, dim // G, G)
    r = np.sqrt(np.mean(vg * vg, axis=2, keepdims=True) + eps)
    out = (vg / r).reshape(rows, dim)
    if weight is not None:
        out = out * np.asarray(weight, np.float64)[None, :]
    return out
