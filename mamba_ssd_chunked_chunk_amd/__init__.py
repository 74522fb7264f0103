"""Mamba-2 SSD selective-state-space scan on AMD MI355X (gfx950).

Thin Python binding over libssd.so (include/ssd.h).  Every step of the scan
runs in the library's HIP kernels; this module only checks and marshals
arguments.  torch supplies device memory and the current HIP stream.

    y = chunk_scan(x, dt, A, B, C, D, chunk_size=256)
    y, final = chunk_scan(..., initial_state=h0, return_final_state=True)
    y = step(state, x_t, dt_t, A, B_t, C_t, D)        # state updated in place

Tensor contract (nnterp guide, "Mamba-2" page, section "The values"):
x [b, l, h, p], dt [b, l, h], B and C [b, l, g, n], states [b, h, n, p]
(fp32), A, D, dt_bias [h] (fp32).  x, dt, B, C share one io dtype
(torch.float32 or torch.bfloat16); y has that dtype.
"""
from __future__ import annotations

import ctypes
import math
from typing import Optional, Tuple

from . import _lib
from ._lib import LibraryMissing, load, status_string  # noqa: F401

__all__ = ["chunk_scan", "chunk_scan_noalloc", "chunk_scan_bwd", "step", "conv1d_silu", "gated_norm",
           "mixer_forward", "mixer_workspace_bytes",
           "segment_log_decay", "combine_segments",
           "workspace_bytes", "state_chunks", "abi_version",
           "LibraryMissing", "SsdError"]


class SsdError(RuntimeError):
    def __init__(self, fn: str, code: int):
        super().__init__("%s failed: %s (status %d)" % (fn, status_string(code), code))
        self.code = code


def _torch():
    import torch
    return torch


def _io_code(dtype) -> int:
    torch = _torch()
    if dtype == torch.float32:
        return _lib.SSD_F32
    if dtype == torch.bfloat16:
        return _lib.SSD_BF16
    raise ValueError("io dtype must be torch.float32 or torch.bfloat16, got %s" % (dtype,))


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _check(name, t, dtype=None, shape=None, device=None):
    if t is None:
        return
    if dtype is not None and t.dtype != dtype:
        raise ValueError("%s must have dtype %s, got %s" % (name, dtype, t.dtype))
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if device is not None and t.device != device:
        raise ValueError("%s is on %s, expected %s" % (name, t.device, device))


def abi_version() -> int:
    return int(load().ssd_abi_version())


def workspace_bytes(batch, seqlen, heads, head_dim, state_dim, groups, chunk) -> int:
    return int(load().ssd_chunk_scan_workspace_bytes(batch, seqlen, heads, head_dim,
                                                     state_dim, groups, chunk))


def state_chunks(batch, seqlen, heads, head_dim, state_dim, groups, chunk, io="bf16",
                 with_chunk_states=False) -> int:
    """Chunks per sequence whose boundary states a chunk_scan call with these
    sizes stores on the current device (ssd_chunk_scan_state_chunks)."""
    code = {"f32": 0, "bf16": 1}[io]
    v = int(load().ssd_chunk_scan_state_chunks(batch, seqlen, heads, head_dim, state_dim,
                                                 groups, chunk, code, int(bool(with_chunk_states))))
    if v < 0:
        raise SsdError("ssd_chunk_scan_state_chunks", v)
    return v


def chunk_scan(x, dt, A, B, C, D=None, chunk_size: int = 256, dt_bias=None,
               dt_softplus: bool = True, dt_limit: Tuple[float, float] = (0.0, math.inf),
               initial_state=None, return_final_state: bool = False, out=None,
               final_out=None, workspace=None, seq_idx=None,
               return_chunk_states: bool = False, chunk_states_out=None, kernel_events=None):
    """The chunked SSD scan of a whole sequence (ssd_chunk_scan_ex).

    Returns y, followed by final_state when return_final_state and by the
    state after every chunk [b, ceil(l / chunk_size), h, n, p] when
    return_chunk_states (a tuple when either is asked for).  seq_idx
    [b, l] int32: packed documents, a zero state wherever the index changes
    from one token to the next.  `out`, `final_out`, `chunk_states_out` and
    `workspace` (uint8, at least workspace_bytes(...)) may be given to avoid
    allocations; final_out may alias initial_state.  kernel_events: None, or
    8 raw hipEvent_t handles (ints; 0 for none) that receive the start and
    end of the call's kernel in each slot of _lib.EVENT_SLOTS.
    """
    torch = _torch()
    lib = load()
    if x.dim() != 4:
        raise ValueError("x must be [batch, seqlen, heads, head_dim]")
    b, l, h, p = x.shape
    if B.dim() != 4:
        raise ValueError("B must be [batch, seqlen, groups, state_dim]")
    g, n = B.shape[2], B.shape[3]
    dev = x.device
    if dev.type != "cuda":
        raise ValueError("x must be a GPU tensor")
    io = x.dtype
    _io_code(io)
    _check("x", x, io)
    _check("dt", dt, io, (b, l, h), dev)
    _check("B", B, io, (b, l, g, n), dev)
    _check("C", C, io, (b, l, g, n), dev)
    _check("A", A, torch.float32, (h,), dev)
    _check("D", D, torch.float32, (h,), dev)
    _check("dt_bias", dt_bias, torch.float32, (h,), dev)
    _check("initial_state", initial_state, torch.float32, (b, h, n, p), dev)
    _check("seq_idx", seq_idx, torch.int32, (b, l), dev)
    y = torch.empty_like(x) if out is None else out
    _check("out", y, io, (b, l, h, p), dev)
    fin = None
    if return_final_state:
        fin = torch.empty((b, h, n, p), dtype=torch.float32, device=dev) \
            if final_out is None else final_out
        _check("final_out", fin, torch.float32, (b, h, n, p), dev)
    states = None
    if return_chunk_states:
        nck = -(-l // int(chunk_size)) if chunk_size > 0 else 0
        states = torch.empty((b, nck, h, n, p), dtype=torch.float32, device=dev) \
            if chunk_states_out is None else chunk_states_out
        _check("chunk_states_out", states, torch.float32, (b, nck, h, n, p), dev)
    wsb = int(lib.ssd_chunk_scan_workspace_bytes(b, l, h, p, n, g, int(chunk_size)))
    ws = workspace
    if ws is None:
        ws = torch.empty(max(wsb, 256), dtype=torch.uint8, device=dev)
    _check("workspace", ws, torch.uint8, None, dev)
    ev = None
    if kernel_events is not None:
        if len(kernel_events) != 2 * len(_lib.EVENT_SLOTS):
            raise ValueError("kernel_events must hold %d handles" % (2 * len(_lib.EVENT_SLOTS)))
        ev = (ctypes.c_void_p * len(kernel_events))(*[int(e) or None for e in kernel_events])
    stream = torch.cuda.current_stream(dev).cuda_stream
    rc = lib.ssd_chunk_scan_ex(
        _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(dt_bias),
        int(bool(dt_softplus)), float(dt_limit[0]), float(dt_limit[1]),
        _ptr(initial_state), _ptr(seq_idx), _ptr(y), _ptr(fin), _ptr(states), b, l, h, p, n,
        g, int(chunk_size), _io_code(io), _ptr(ws), ws.numel() * ws.element_size(), stream, ev)
    if rc != 0:
        raise SsdError("ssd_chunk_scan_ex", rc)
    if not return_final_state and not return_chunk_states:
        return y
    return (y,) + ((fin,) if return_final_state else ()) + \
        ((states,) if return_chunk_states else ())


def chunk_scan_noalloc(x, dt, A, B, C, y, D=None, chunk_size: int = 256, dt_bias=None,
                       dt_softplus: bool = True, dt_limit: Tuple[float, float] = (0.0, math.inf),
                       initial_state=None, final_state=None, seq_idx=None, chunk_states=None):
    """chunk_scan on the library's static device scratch (ssd_chunk_scan_noalloc):
    no workspace, and nothing allocated here either -- the caller passes the
    outputs y, and optionally final_state [b, h, n, p] and chunk_states
    [b, ceil(l / chunk_size), h, n, p] (fp32).  Sizes whose workspace_bytes
    exceed SSD_SCRATCH_BYTES raise SsdError (SSD_ERR_SCRATCH).  Calls that
    overlap on one GPU race on its scratch."""
    torch = _torch()
    lib = load()
    b, l, h, p = x.shape
    g, n = B.shape[2], B.shape[3]
    dev = x.device
    io = x.dtype
    _check("x", x, io)
    _check("dt", dt, io, (b, l, h), dev)
    _check("B", B, io, (b, l, g, n), dev)
    _check("C", C, io, (b, l, g, n), dev)
    _check("y", y, io, (b, l, h, p), dev)
    _check("A", A, torch.float32, (h,), dev)
    _check("D", D, torch.float32, (h,), dev)
    _check("dt_bias", dt_bias, torch.float32, (h,), dev)
    _check("initial_state", initial_state, torch.float32, (b, h, n, p), dev)
    _check("final_state", final_state, torch.float32, (b, h, n, p), dev)
    _check("seq_idx", seq_idx, torch.int32, (b, l), dev)
    nck = -(-l // int(chunk_size)) if chunk_size > 0 else 0
    _check("chunk_states", chunk_states, torch.float32, (b, nck, h, n, p), dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    rc = lib.ssd_chunk_scan_noalloc(
        _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(dt_bias),
        int(bool(dt_softplus)), float(dt_limit[0]), float(dt_limit[1]),
        _ptr(initial_state), _ptr(seq_idx), _ptr(y), _ptr(final_state), _ptr(chunk_states),
        b, l, h, p, n, g, int(chunk_size), _io_code(io), stream, None)
    if rc != 0:
        raise SsdError("ssd_chunk_scan_noalloc", rc)
    return y


def chunk_scan_bwd(x, dt, A, B, C, dy, D=None, chunk_size: int = 256, dt_bias=None,
                   initial_state=None, d_final=None, dt_softplus: bool = True,
                   dt_limit: Tuple[float, float] = (0.0, math.inf), seq_idx=None,
                   workspace=None):
    """Gradients of chunk_scan's y (cotangent dy) and final state (d_final)
    with respect to every input (ssd_chunk_scan_bwd), deterministic.
    Returns a dict: dx, ddt, dB, dC (io dtype), dA, and dD, d_dt_bias,
    d_init (fp32) for the inputs that were given."""
    torch = _torch()
    lib = load()
    b, l, h, p = x.shape
    g, n = B.shape[2], B.shape[3]
    dev = x.device
    if dev.type != "cuda":
        raise ValueError("x must be a GPU tensor")
    io = x.dtype
    _io_code(io)
    _check("x", x, io)
    _check("dt", dt, io, (b, l, h), dev)
    _check("B", B, io, (b, l, g, n), dev)
    _check("C", C, io, (b, l, g, n), dev)
    _check("dy", dy, io, (b, l, h, p), dev)
    _check("A", A, torch.float32, (h,), dev)
    _check("D", D, torch.float32, (h,), dev)
    _check("dt_bias", dt_bias, torch.float32, (h,), dev)
    _check("initial_state", initial_state, torch.float32, (b, h, n, p), dev)
    _check("d_final", d_final, torch.float32, (b, h, n, p), dev)
    _check("seq_idx", seq_idx, torch.int32, (b, l), dev)
    out = dict(dx=torch.empty_like(x), ddt=torch.empty_like(dt),
               dA=torch.empty((h,), dtype=torch.float32, device=dev),
               dB=torch.empty_like(B), dC=torch.empty_like(C))
    if D is not None:
        out["dD"] = torch.empty((h,), dtype=torch.float32, device=dev)
    if dt_bias is not None:
        out["d_dt_bias"] = torch.empty((h,), dtype=torch.float32, device=dev)
    if initial_state is not None:
        out["d_init"] = torch.empty((b, h, n, p), dtype=torch.float32, device=dev)
    wsb = int(lib.ssd_chunk_scan_bwd_workspace_bytes(b, l, h, p, n, g, int(chunk_size),
                                                     _io_code(io)))
    ws = workspace if workspace is not None else torch.empty(max(wsb, 1), dtype=torch.uint8,
                                                             device=dev)
    _check("workspace", ws, torch.uint8, None, dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    rc = lib.ssd_chunk_scan_bwd(
        _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(dt_bias),
        int(bool(dt_softplus)), float(dt_limit[0]), float(dt_limit[1]), _ptr(initial_state),
        _ptr(seq_idx), _ptr(dy), _ptr(d_final), _ptr(out["dx"]), _ptr(out["ddt"]),
        _ptr(out["dA"]), _ptr(out["dB"]), _ptr(out["dC"]), _ptr(out.get("dD")),
        _ptr(out.get("d_dt_bias")), _ptr(out.get("d_init")), b, l, h, p, n, g,
        int(chunk_size), _io_code(io), _ptr(ws), ws.numel() * ws.element_size(), stream)
    if rc != 0:
        raise SsdError("ssd_chunk_scan_bwd", rc)
    return out


def segment_log_decay(dt, A, dt_bias=None, dt_softplus: bool = True,
                      dt_limit: Tuple[float, float] = (0.0, math.inf), seq_idx=None):
    """Total log decay [b, h] of a segment (ssd_segment_log_decay)."""
    torch = _torch()
    lib = load()
    b, l, h = dt.shape
    dev = dt.device
    _check("dt", dt, dt.dtype)
    _check("A", A, torch.float32, (h,), dev)
    _check("dt_bias", dt_bias, torch.float32, (h,), dev)
    _check("seq_idx", seq_idx, torch.int32, (b, l), dev)
    out = torch.empty((b, h), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    rc = lib.ssd_segment_log_decay(_ptr(dt), _ptr(A), _ptr(dt_bias), int(bool(dt_softplus)),
                                   float(dt_limit[0]), float(dt_limit[1]), _ptr(seq_idx),
                                   _ptr(out), b, l, h, _io_code(dt.dtype), stream)
    if rc != 0:
        raise SsdError("ssd_segment_log_decay", rc)
    return out


def combine_segments(log_decay, seg_states, initial_state=None, starts_document=None):
    """Entry states [K, b, h, n, p] of K segments and the final state
    [b, h, n, p] from their log decays [K, b, h] and zero-start final
    states [K, b, h, n, p] (ssd_combine_segments)."""
    torch = _torch()
    lib = load()
    K, b, h, n, p = seg_states.shape
    dev = seg_states.device
    _check("log_decay", log_decay, torch.float32, (K, b, h), dev)
    _check("seg_states", seg_states, torch.float32)
    _check("initial_state", initial_state, torch.float32, (b, h, n, p), dev)
    _check("starts_document", starts_document, torch.int32, (K, b), dev)
    entry = torch.empty_like(seg_states)
    fin = torch.empty((b, h, n, p), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    rc = lib.ssd_combine_segments(_ptr(log_decay), _ptr(seg_states), _ptr(initial_state),
                                  _ptr(starts_document), _ptr(entry), _ptr(fin), K, b, h, p, n,
                                  stream)
    if rc != 0:
        raise SsdError("ssd_combine_segments", rc)
    return entry, fin


def step(state, x, dt, A, B, C, D=None, dt_bias=None, dt_softplus: bool = True,
         dt_limit: Tuple[float, float] = (0.0, math.inf), out=None):
    """One decode step (ssd_step): updates `state` [b,h,n,p] in place, returns y."""
    torch = _torch()
    lib = load()
    if x.dim() != 3:
        raise ValueError("x must be [batch, heads, head_dim]")
    b, h, p = x.shape
    g, n = B.shape[1], B.shape[2]
    dev = x.device
    if dev.type != "cuda":
        raise ValueError("x must be a GPU tensor")
    io = x.dtype
    _io_code(io)
    _check("state", state, torch.float32, (b, h, n, p), dev)
    _check("x", x, io)
    _check("dt", dt, io, (b, h), dev)
    _check("B", B, io, (b, g, n), dev)
    _check("C", C, io, (b, g, n), dev)
    _check("A", A, torch.float32, (h,), dev)
    _check("D", D, torch.float32, (h,), dev)
    _check("dt_bias", dt_bias, torch.float32, (h,), dev)
    y = torch.empty_like(x) if out is None else out
    _check("out", y, io, (b, h, p), dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    rc = lib.ssd_step(_ptr(state), _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D),
                      _ptr(dt_bias), int(bool(dt_softplus)), float(dt_limit[0]),
                      float(dt_limit[1]), _ptr(y), b, h, p, n, g, _io_code(io), stream)
    if rc != 0:
        raise SsdError("ssd_step", rc)
    return y


def conv1d_silu(xbc, weight, heads, head_dim, state_dim, groups, bias=None, conv_init=None,
                seq_idx=None, apply_silu: bool = True, return_conv_state: bool = False, out=None):
    """Causal depthwise conv1d + bias + SiLU over the packed x | B | C
    channels xbc [b, l, ch], split into the scan's inputs (ssd_conv1d_silu).
    weight [ch, width] fp32; conv_init [b, width-1, ch] fp32.  Returns
    (x, B, C), plus the final conv state [b, width-1, ch] when asked for.
    `out` may pass preallocated (x, B, C)."""
    torch = _torch()
    lib = load()
    if xbc.dim() != 3:
        raise ValueError("xbc must be [batch, seqlen, channels]")
    b, l, ch = xbc.shape
    dev = xbc.device
    if dev.type != "cuda":
        raise ValueError("xbc must be a GPU tensor")
    io = xbc.dtype
    h, p, n, g = int(heads), int(head_dim), int(state_dim), int(groups)
    if ch != h * p + 2 * g * n:
        raise ValueError("xbc has %d channels, expected heads*head_dim + 2*groups*state_dim = %d"
                         % (ch, h * p + 2 * g * n))
    K = int(weight.shape[1]) if weight.dim() == 2 else -1
    _check("xbc", xbc, io)
    _check("weight", weight, torch.float32, (ch, K), dev)
    _check("bias", bias, torch.float32, (ch,), dev)
    _check("conv_init", conv_init, torch.float32, (b, K - 1, ch), dev)
    _check("seq_idx", seq_idx, torch.int32, (b, l), dev)
    if out is None:
        x = torch.empty((b, l, h, p), dtype=io, device=dev)
        B = torch.empty((b, l, g, n), dtype=io, device=dev)
        C = torch.empty((b, l, g, n), dtype=io, device=dev)
    else:
        x, B, C = out
    _check("x", x, io, (b, l, h, p), dev)
    _check("B", B, io, (b, l, g, n), dev)
    _check("C", C, io, (b, l, g, n), dev)
    fin = None
    if return_conv_state:
        fin = torch.empty((b, K - 1, ch), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    rc = lib.ssd_conv1d_silu(_ptr(xbc), _ptr(weight), _ptr(bias), _ptr(conv_init), _ptr(seq_idx),
                             _ptr(x), _ptr(B), _ptr(C), _ptr(fin), b, l, h, p, n, g, K,
                             int(bool(apply_silu)), _io_code(io), stream)
    if rc != 0:
        raise SsdError("ssd_conv1d_silu", rc)
    return (x, B, C, fin) if return_conv_state else (x, B, C)


def gated_norm(y, z=None, weight=None, group_size: Optional[int] = None, eps: float = 1e-5,
               normalize: bool = True, out=None):
    """y * silu(z), then an RMS norm over groups of `group_size` channels of
    the last axis times `weight` (ssd_gated_norm).  y [..., dim] in the io
    dtype; z like y or None; weight [dim] fp32 or None.  `out` may be y."""
    torch = _torch()
    lib = load()
    dev = y.device
    if dev.type != "cuda":
        raise ValueError("y must be a GPU tensor")
    io = y.dtype
    dim = int(y.shape[-1])
    rows = y.numel() // dim if dim else 0
    G = dim if group_size is None else int(group_size)
    _check("y", y, io)
    _check("z", z, io, tuple(y.shape), dev)
    _check("weight", weight, torch.float32, (dim,), dev)
    o = torch.empty_like(y) if out is None else out
    _check("out", o, io, tuple(y.shape), dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    rc = lib.ssd_gated_norm(_ptr(y), _ptr(z), _ptr(weight), _ptr(o), rows, dim, G, float(eps),
                            int(bool(normalize)), _io_code(io), stream)
    if rc != 0:
        raise SsdError("ssd_gated_norm", rc)
    return o


def mixer_workspace_bytes(batch, seqlen, heads, head_dim, state_dim, groups, chunk,
                          io="bf16") -> int:
    """Workspace bytes of one mixer_forward call (ssd_mixer_workspace_bytes)."""
    code = _lib.SSD_BF16 if io == "bf16" else _lib.SSD_F32
    return int(load().ssd_mixer_workspace_bytes(batch, seqlen, heads, head_dim, state_dim,
                                                groups, chunk, code))


def mixer_forward(xbc, dt, A, conv_weight, heads, head_dim, state_dim, groups, z=None,
                  conv_bias=None, conv_init=None, D=None, dt_bias=None,
                  dt_softplus: bool = True, dt_limit: Tuple[float, float] = (0.0, math.inf),
                  initial_state=None, seq_idx=None, norm_weight=None,
                  norm_group: Optional[int] = None, eps: float = 1e-5, normalize: bool = True,
                  chunk_size: int = 256, return_final_state: bool = False,
                  return_conv_state: bool = False, out=None, workspace=None):
    """The mixer between its projections in one call (ssd_mixer_forward):
    conv1d + SiLU + split of xbc [b, l, h*p + 2*g*n], the chunk scan, and
    the silu(z)-gated RMS norm over groups of norm_group channels (default:
    all h*p).  Returns out [b, l, h, p], followed by the final state and/or
    the final conv state [b, width-1, ch] when asked for."""
    torch = _torch()
    lib = load()
    if xbc.dim() != 3:
        raise ValueError("xbc must be [batch, seqlen, channels]")
    b, l, ch = xbc.shape
    dev = xbc.device
    if dev.type != "cuda":
        raise ValueError("xbc must be a GPU tensor")
    io = xbc.dtype
    code = _io_code(io)
    h, p, n, g = int(heads), int(head_dim), int(state_dim), int(groups)
    if ch != h * p + 2 * g * n:
        raise ValueError("xbc has %d channels, expected heads*head_dim + 2*groups*state_dim = %d"
                         % (ch, h * p + 2 * g * n))
    K = int(conv_weight.shape[1]) if conv_weight.dim() == 2 else -1
    _check("xbc", xbc, io)
    _check("dt", dt, io, (b, l, h), dev)
    _check("z", z, io, (b, l, h * p), dev)
    _check("conv_weight", conv_weight, torch.float32, (ch, K), dev)
    _check("conv_bias", conv_bias, torch.float32, (ch,), dev)
    _check("conv_init", conv_init, torch.float32, (b, K - 1, ch), dev)
    _check("A", A, torch.float32, (h,), dev)
    _check("D", D, torch.float32, (h,), dev)
    _check("dt_bias", dt_bias, torch.float32, (h,), dev)
    _check("initial_state", initial_state, torch.float32, (b, h, n, p), dev)
    _check("seq_idx", seq_idx, torch.int32, (b, l), dev)
    _check("norm_weight", norm_weight, torch.float32, (h * p,), dev)
    y = torch.empty((b, l, h, p), dtype=io, device=dev) if out is None else out
    _check("out", y, io, (b, l, h, p), dev)
    fin = torch.empty((b, h, n, p), dtype=torch.float32, device=dev) \
        if return_final_state else None
    cfin = torch.empty((b, K - 1, ch), dtype=torch.float32, device=dev) \
        if return_conv_state else None
    wsb = int(lib.ssd_mixer_workspace_bytes(b, l, h, p, n, g, int(chunk_size), code))
    ws = workspace
    if ws is None:
        ws = torch.empty(max(wsb, 256), dtype=torch.uint8, device=dev)
    _check("workspace", ws, torch.uint8, None, dev)
    G = h * p if norm_group is None else int(norm_group)
    stream = torch.cuda.current_stream(dev).cuda_stream
    rc = lib.ssd_mixer_forward(
        _ptr(xbc), _ptr(z), _ptr(dt), _ptr(conv_weight), _ptr(conv_bias), K, _ptr(conv_init),
        _ptr(cfin), _ptr(A), _ptr(D), _ptr(dt_bias), int(bool(dt_softplus)),
        float(dt_limit[0]), float(dt_limit[1]), _ptr(initial_state), _ptr(fin), _ptr(seq_idx),
        _ptr(norm_weight), G, float(eps), int(bool(normalize)), _ptr(y), b, l, h, p, n, g,
        int(chunk_size), code, _ptr(ws), ws.numel() * ws.element_size(), stream)
    if rc != 0:
        raise SsdError("ssd_mixer_forward", rc)
    if not return_final_state and not return_conv_state:
        return y
    return (y,) + ((fin,) if return_final_state else ()) + \
        ((cfin,) if return_conv_state else ())
