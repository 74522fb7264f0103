"""Seeded synthetic inputs for the Mamba-2 SSD scan.

This module only draws random numbers and rounds them to the storage
precision. It holds none of the scan's arithmetic and is shared, as the
single input source, by the fp64 oracle's tests, the GPU parity tests and
the benchmark.

Shapes and distributions follow the Mamba-2 SSD tensor contract of the
nnterp guide, "Mamba-2" page, section "The values": x [b, l, h, p],
dt [b, l, h], B and C [b, l, g, n], states [b, h, n, p].  The dt_bias draw
is the inverse softplus of a log-uniform time step, as described on Bud's
Wiki, "Mamba-2 dt_bias initialization bug", section "Method" (the page's
"log(uniform(...)) (softplus-inverted)" is read as softplus^-1 applied to
exp(U[log tmin, log tmax])).

Draw order for one workload (generator PCG64 seeded with the workload seed):
A[h], dt_bias[h], then for each batch row b in order: x[b], dt[b], B[b],
C[b]; then init_state (when the workload has one).  All values are drawn in
fp32; bf16 workloads round them to bf16 with round-to-nearest-even here,
before either the oracle or the GPU sees them.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

F32 = "f32"
BF16 = "bf16"


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic SSD scan workload (shapes, io dtype, chunk, init state)."""
    name: str
    batch: int
    seqlen: int
    heads: int
    head_dim: int
    state_dim: int
    groups: int
    chunk: int
    io: str = BF16
    init_std: float = 0.0          # 0 -> zero initial state (passed as None)
    return_final: bool = True
    dt_bias_literal: bool = False  # stress reading: dt_bias = loguniform itself
    seed: int = 0

    @property
    def tokens(self) -> int:
        return self.batch * self.seqlen

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five workloads of the scan (tiny fp32; Mamba2-130m-shaped; 2.7B-shaped
# with an initial state; grouped long context; decode after a prefill).
WORKLOADS = {
    "tiny_fp32": Workload("tiny_fp32", 1, 256, 24, 64, 128, 1, 64, io=F32, seed=0),
    "mamba2_130m": Workload("mamba2_130m", 8, 2048, 24, 64, 128, 1, 256, seed=1,
                            return_final=False),
    "mamba2_2p7b": Workload("mamba2_2p7b", 4, 4096, 80, 64, 128, 1, 256,
                            init_std=0.1, seed=2),
    "grouped_long": Workload("grouped_long", 1, 65536, 64, 64, 128, 8, 256, seed=3,
                             return_final=False),
    # decode workload: the prefill that seeds the state, then DECODE_STEPS steps
    "decode_2p7b": Workload("decode_2p7b", 256, 1024, 80, 64, 128, 1, 256, seed=4),
}
DECODE_STEPS = 128


def bf16_round(a: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest, ties to even."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    r = ((u + bias) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(a)
    if nan.any():
        r[nan] = np.uint16(0x7FC0)
    return r


def bf16_to_f32(u: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> fp32, exact."""
    return (np.ascontiguousarray(u, dtype=np.uint16).astype(np.uint32)
            << np.uint32(16)).view(np.float32)


def softplus_inv(y: np.ndarray) -> np.ndarray:
    """Inverse of softplus(z) = log(1 + e^z) for y > 0: z = y + log(-expm1(-y))."""
    y = np.asarray(y, dtype=np.float64)
    return y + np.log(-np.expm1(-y))


def _store(a32: np.ndarray, io: str) -> np.ndarray:
    """fp32 draw -> the stored io representation (float32, or uint16 bf16 bits)."""
    return bf16_round(a32) if io == BF16 else np.ascontiguousarray(a32, np.float32)


def _normal(rng, shape, std=1.0) -> np.ndarray:
    v = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        v *= np.float32(std)
    return v


def _head_params(rng, heads: int, literal: bool):
    # A_h = -exp(U[log 1, log 16])  ->  A in [-16, -1]
    A = -np.exp(rng.uniform(0.0, math.log(16.0), size=heads)).astype(np.float32)
    # dt0 = exp(U[log 1e-3, log 0.1]); dt_bias = softplus^-1(dt0)
    dt0 = np.exp(rng.uniform(math.log(1e-3), math.log(0.1), size=heads))
    dt_bias = (dt0 if literal else softplus_inv(dt0)).astype(np.float32)
    return A, dt_bias


def make_inputs(w: Workload, seqlen: Optional[int] = None, batch: Optional[int] = None):
    """Draw one workload's inputs.  Returns a dict of numpy arrays.

    x, dt, B, C are float32 (f32 io) or uint16 bf16 bit patterns (bf16 io).
    A, D, dt_bias and init_state are float32.  init_state is None when the
    workload starts from the zero state.  `seqlen` / `batch` override the
    workload's sizes (same draw order, smaller arrays).
    """
    L = w.seqlen if seqlen is None else seqlen
    Bt = w.batch if batch is None else batch
    h, p, n, g = w.heads, w.head_dim, w.state_dim, w.groups
    rng = np.random.Generator(np.random.PCG64(w.seed))
    A, dt_bias = _head_params(rng, h, w.dt_bias_literal)
    sdt = np.uint16 if w.io == BF16 else np.float32
    x = np.empty((Bt, L, h, p), sdt)
    dt = np.empty((Bt, L, h), sdt)
    Bm = np.empty((Bt, L, g, n), sdt)
    Cm = np.empty((Bt, L, g, n), sdt)
    for b in range(Bt):
        x[b] = _store(_normal(rng, (L, h, p)), w.io)
        dt[b] = _store(_normal(rng, (L, h)), w.io)
        Bm[b] = _store(_normal(rng, (L, g, n)), w.io)
        Cm[b] = _store(_normal(rng, (L, g, n)), w.io)
    init = None
    if w.init_std > 0:
        init = _normal(rng, (Bt, h, n, p), w.init_std)
    D = np.ones(h, np.float32)
    return dict(x=x, dt=dt, A=A, B=Bm, C=Cm, D=D, dt_bias=dt_bias,
                init_state=init, io=w.io)


def make_step_inputs(w: Workload, step: int, batch: Optional[int] = None):
    """Inputs of decode step `step` (x [b,h,p], dt [b,h], B, C [b,g,n]).

    Each step has its own generator, PCG64 seeded with (workload seed, 1,
    step), so any step can be drawn without drawing the ones before it.
    """
    Bt = w.batch if batch is None else batch
    h, p, n, g = w.heads, w.head_dim, w.state_dim, w.groups
    rng = np.random.Generator(np.random.PCG64([w.seed, 1, step]))
    x = _store(_normal(rng, (Bt, h, p)), w.io)
    dt = _store(_normal(rng, (Bt, h)), w.io)
    Bm = _store(_normal(rng, (Bt, g, n)), w.io)
    Cm = _store(_normal(rng, (Bt, g, n)), w.io)
    return dict(x=x, dt=dt, B=Bm, C=Cm)


def random_case(seed: int, batch: int, seqlen: int, heads: int, head_dim: int,
                state_dim: int, groups: int, io: str = F32, init_std: float = 0.0,
                literal: bool = False):
    """A small case with the workload distributions and arbitrary shapes."""
    w = Workload("case", batch, seqlen, heads, head_dim, state_dim, groups, 1,
                 io=io, init_std=init_std, dt_bias_literal=literal, seed=seed)
    return make_inputs(w)


def as_f32(a: np.ndarray, io: str) -> np.ndarray:
    """Stored io array -> float32 values (exact widening for bf16)."""
    return bf16_to_f32(a) if io == BF16 else np.asarray(a, np.float32)


def conv_case(seed: int, batch: int, seqlen: int, heads: int, head_dim: int, state_dim: int,
              groups: int, width: int, io: str = F32, with_init: bool = True):
    """Inputs of the short convolution before the scan: the projection's
    x | B | C channels ~ N(0, 1) (stored in io), taps and bias
    ~ U(-1/sqrt(width), 1/sqrt(width)) (a depthwise filter's fan-in is its
    width), and width-1 earlier input rows ~ N(0, 1) at io precision, in
    fp32."""
    rng = np.random.Generator(np.random.PCG64([seed, 7]))
    ch = heads * head_dim + 2 * groups * state_dim
    bound = 1.0 / math.sqrt(width)
    xbc = _store(_normal(rng, (batch, seqlen, ch)), io)
    weight = rng.uniform(-bound, bound, (ch, width)).astype(np.float32)
    bias = rng.uniform(-bound, bound, ch).astype(np.float32)
    init = None
    if with_init:
        init = np.ascontiguousarray(as_f32(_store(_normal(rng, (batch, width - 1, ch)), io), io))
    return dict(xbc=xbc, weight=weight, bias=bias, conv_init=init, io=io, heads=heads,
                head_dim=head_dim, state_dim=state_dim, groups=groups)


def norm_case(seed: int, rows: int, dim: int, io: str = F32):
    """Inputs of the gate and norm after the scan: y, z ~ N(0, 1) (stored in
    io) and a per-channel weight 1 + N(0, 0.1^2)."""
    rng = np.random.Generator(np.random.PCG64([seed, 8]))
    y = _store(_normal(rng, (rows, dim)), io)
    z = _store(_normal(rng, (rows, dim)), io)
    weight = (1.0 + 0.1 * rng.standard_normal(dim)).astype(np.float32)
    return dict(y=y, z=z, weight=weight, io=io)



def doc_index(seed: int, batch: int, seqlen: int, lo: int = 32, hi: int = 2048) -> np.ndarray:
    """Document index [batch, seqlen] int32 of packed rows: documents back to
    back, lengths log-uniform in [lo, hi] tokens (PCG64 seeded with
    (seed, 10)), the last one cut at the row's end."""
    rng = np.random.Generator(np.random.PCG64([seed, 10]))
    seq = np.zeros((batch, seqlen), np.int32)
    for bi in range(batch):
        t = k = 0
        while t < seqlen:
            m = int(round(math.exp(rng.uniform(math.log(lo), math.log(hi)))))
            seq[bi, t:t + m] = k
            t += m
            k += 1
    return seq


def cotangent_case(seed: int, batch: int, seqlen: int, heads: int, head_dim: int,
                   state_dim: int, io: str = F32):
    """Cotangents for the gradient pass: dy ~ N(0, 1) (stored in io) and
    d_final ~ N(0, 1) (fp32)."""
    rng = np.random.Generator(np.random.PCG64([seed, 9]))
    dy = _store(_normal(rng, (batch, seqlen, heads, head_dim)), io)
    d_final = _normal(rng, (batch, heads, state_dim, head_dim))
    return dict(dy=dy, d_final=d_final, io=io)
