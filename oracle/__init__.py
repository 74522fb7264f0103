"""fp64 CPU oracle for the Mamba-2 SSD scan.

TEST INFRASTRUCTURE ONLY: the test suite, the package smoke check and the
benchmark's CPU-baseline leg are the only users.  The product path never
imports, loads or calls anything here, and nothing here imports the product
package.

Three independent fp64 formulations live here:

* `scan` / `step` -- the sequential recurrence, token by token, in plain C
  (ssd_oracle.c).  This is the oracle proper (nnterp guide, "Mamba-2" page,
  opening section: h = exp(dt A) h + dt B x^T, y = C^T h + D x).  Options:
  packed sequences (a per-token document index; a zero state wherever it
  changes -- the sample-packing reset of the Mamba2 news page) and the state
  after every chunk boundary (nnterp, "The state after every token").
* `oracle.quadratic.dual_form` -- the same result written as one masked
  matrix product per head (the "matrix multiplication form" of the kongchang
  "Mamba2" page), derived by unrolling the recurrence.  Used only to pin the
  C code on small inputs.
* `oracle.chunked.chunked_scan` -- the two-stage chunked algorithm (kongchang
  "Mamba2" page, chunk-scan entry; nnterp "The state after every token"),
  step by step in fp64, returning its intermediates.  Pinned to `scan`.

Parity unpinned (documented conventions, not facts the pages fix): the head
to group mapping hh -> hh // (heads // groups), and the default time-step
limit (0, +inf).
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ssd_oracle.c")
_SO = os.path.join(_HERE, "libssd_oracle.so")
_lib = None

IO_CODES = {"f32": 0, "bf16": 1}


def build(force: bool = False) -> str:
    """Compile ssd_oracle.c into oracle/libssd_oracle.so with gcc -O2."""
    if force or not os.path.exists(_SO) or os.path.getmtime(_SO) < os.path.getmtime(_SRC):
        tmp = _SO + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fPIC", "-shared", "-std=c99",
                               "-D_GNU_SOURCE", "-o", tmp, _SRC, "-lm", "-lpthread"])
        os.replace(tmp, _SO)
    return _SO


def _bind(lib):
    """Declare the C signatures on a loaded oracle library."""
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    lib.ssd_oracle_scan.restype = ctypes.c_int
    lib.ssd_oracle_scan.argtypes = [P, P, P, P, P, P, P, ctypes.c_int,
                                    ctypes.c_double, ctypes.c_double, P,
                                    I64, I64, I64, I64, I64, I64, ctypes.c_int,
                                    P, I64, P, P, P, I64, P, ctypes.c_int]
    lib.ssd_oracle_dt.restype = ctypes.c_int
    lib.ssd_oracle_dt.argtypes = [P, P, P, ctypes.c_int, ctypes.c_double,
                                  ctypes.c_double, I64, I64, I64, ctypes.c_int, P, P]
    return lib


def _load():
    global _lib
    if _lib is None:
        _lib = _bind(ctypes.CDLL(build()))
    return _lib


def default_threads() -> int:
    """Host threads for the oracle: the CPUs this process may run on, capped
    by OMP_NUM_THREADS when that is set (a machine's share of its cores)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    cap = os.environ.get("OMP_NUM_THREADS", "")
    if cap.isdigit() and int(cap) > 0:
        n = min(n, int(cap))
    return max(1, n)


def _c(a, dtype):
    return None if a is None else np.ascontiguousarray(a, dtype=dtype)


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _io_arr(a, io):
    return np.ascontiguousarray(a, dtype=np.uint16 if io == "bf16" else np.float32)


def scan(x, dt, A, B, C, D=None, dt_bias=None, dt_softplus=True,
         dt_limit=(0.0, math.inf), init_state=None, io="f32",
         pairs: Optional[Sequence] = None, nthreads: Optional[int] = None,
         seq_idx=None, states_chunk: Optional[int] = None):
    """Sequential fp64 recurrence.

    x [b,l,h,p], dt [b,l,h], B, C [b,l,g,n] as stored (float32, or uint16
    bf16 bits when io == "bf16"); A, D, dt_bias [h]; init_state [b,h,n,p]
    (any float dtype; None -> zeros).  seq_idx [b,l] integers or None:
    packed sequences, a zero state wherever the index changes from one token
    to the next.

    pairs None: returns y [b,l,h,p] fp64 and final [b,h,n,p] fp64.
    pairs [(b, h), ...]: returns y [k,l,p] and final [k,n,p] for those pairs.
    states_chunk c: also returns the state after the last token of every
    chunk of c tokens, [b, ceil(l/c), h, n, p] (pairs: [k, ceil(l/c), n, p]).
    """
    x, dt, B, C = (_io_arr(a, io) for a in (x, dt, B, C))
    b, l, h, p = x.shape
    g, n = B.shape[2], B.shape[3]
    full = pairs is None
    if full:
        pr = np.array([(bi, hi) for bi in range(b) for hi in range(h)], np.int64)
    else:
        pr = np.asarray(pairs, np.int64).reshape(-1, 2)
    k = pr.shape[0]
    init = None
    if init_state is not None:
        ist = np.asarray(init_state)
        init = np.ascontiguousarray(ist[pr[:, 0], pr[:, 1]], dtype=np.float64)
    y = np.empty((k, l, p), np.float64)
    st = np.empty((k, n, p), np.float64)
    A = _c(A, np.float32)
    D = _c(D, np.float32)
    dt_bias = _c(dt_bias, np.float32)
    seq = None if seq_idx is None else np.ascontiguousarray(np.asarray(seq_idx).reshape(b, l),
                                                            dtype=np.int32)
    nc = 0
    states = None
    if states_chunk is not None:
        nc = -(-l // int(states_chunk))
        states = np.empty((k, nc, n, p), np.float64)
    rc = _load().ssd_oracle_scan(
        _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(dt_bias),
        int(bool(dt_softplus)), float(dt_limit[0]), float(dt_limit[1]), _ptr(init),
        b, l, h, p, n, g, IO_CODES[io], _ptr(pr), k, _ptr(y), _ptr(st), _ptr(seq),
        int(states_chunk or 0), _ptr(states), int(nthreads or default_threads()))
    if rc != 0:
        raise ValueError("ssd_oracle_scan rejected its arguments")
    if full:
        y = y.reshape(b, h, l, p).transpose(0, 2, 1, 3).copy()
        st = st.reshape(b, h, n, p)
        if states is not None:
            states = states.reshape(b, h, nc, n, p).transpose(0, 2, 1, 3, 4).copy()
    if states is not None:
        return y, st, states
    return y, st


def step(state, x, dt, A, B, C, D=None, dt_bias=None, dt_softplus=True,
         dt_limit=(0.0, math.inf), io="f32", nthreads: Optional[int] = None):
    """One decode step: exactly one iteration of the recurrence.

    state [b,h,n,p] (fp64 carried state); x [b,h,p]; dt [b,h]; B, C [b,g,n].
    Returns (y [b,h,p] fp64, new state [b,h,n,p] fp64).
    """
    x = np.asarray(x)
    b, h, p = x.shape
    y, st = scan(x.reshape(b, 1, h, p), np.asarray(dt).reshape(b, 1, h), A,
                 np.asarray(B)[:, None], np.asarray(C)[:, None], D, dt_bias,
                 dt_softplus, dt_limit, init_state=np.asarray(state, np.float64),
                 io=io, nthreads=nthreads)
    return y[:, 0], st


def process_dt(dt, A, dt_bias=None, dt_softplus=True, dt_limit=(0.0, math.inf),
               io="f32"):
    """Processed time step d and log-decay a = A d, each [b,l,h] fp64."""
    dt = _io_arr(dt, io)
    b, l, h = dt.shape
    d = np.empty((b, l, h), np.float64)
    a = np.empty((b, l, h), np.float64)
    A = _c(A, np.float32)
    dt_bias = _c(dt_bias, np.float32)
    rc = _load().ssd_oracle_dt(_ptr(dt), _ptr(A), _ptr(dt_bias), int(bool(dt_softplus)),
                               float(dt_limit[0]), float(dt_limit[1]), b, l, h,
                               IO_CODES[io], _ptr(d), _ptr(a))
    if rc != 0:
        raise ValueError("ssd_oracle_dt rejected its arguments")
    return d, a


def widen(a, io):
    """Stored io array -> fp64 values (exact)."""
    a = np.asarray(a)
    if io == "bf16":
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return a.astype(np.float64)
