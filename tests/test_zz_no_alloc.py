"""ssd_chunk_scan_noalloc (the scan on the library's static device scratch)
against ssd_chunk_scan_ex with a caller workspace: the same kernels on the
same inputs, so every output must be the same bits.  Two calls in a row,
the second smaller, so the second runs on the scratch the first left
behind; then a call whose sizes exceed the scratch is rejected with
nothing written.  Calls go through the C ABI (ctypes)."""
import numpy as np
import pytest

import ssd_synth as syn
from gpu_util import gpu_inputs, log, torch_mod

pytestmark = pytest.mark.gpu


def _both(inp, Q, seq=None, states=False):
    import mamba_ssd_chunked_chunk_amd as ssd
    torch = torch_mod()
    g = gpu_inputs(inp)
    b, l, h, p = g["x"].shape
    n = g["B"].shape[3]
    nck = -(-l // Q)
    sq = None if seq is None else torch.from_numpy(seq).to("cuda")
    ref = ssd.chunk_scan(g["x"], g["dt"], g["A"], g["B"], g["C"], g["D"], chunk_size=Q,
                         dt_bias=g["dt_bias"], initial_state=g["init"],
                         return_final_state=True, seq_idx=sq, return_chunk_states=states)
    y = torch.full_like(g["x"], float("nan"))
    fin = torch.full((b, h, n, p), float("nan"), dtype=torch.float32, device="cuda")
    cs = torch.full((b, nck, h, n, p), float("nan"), dtype=torch.float32, device="cuda") \
        if states else None
    ssd.chunk_scan_noalloc(g["x"], g["dt"], g["A"], g["B"], g["C"], y, g["D"], chunk_size=Q,
                           dt_bias=g["dt_bias"], initial_state=g["init"], final_state=fin,
                           seq_idx=sq, chunk_states=cs)
    torch.cuda.synchronize()
    got = (y, fin) + ((cs,) if states else ())
    for name, a, r in zip(("y", "final_state", "chunk_states"), got, ref):
        assert torch.equal(a, r), "%s differs from ssd_chunk_scan_ex" % name


@pytest.mark.parametrize("io", ["bf16", "f32"])
def test_noalloc_matches_workspace_entry_twice(io):
    # first call: larger sizes, initial state, chunk states
    inp = syn.random_case(5100, 2, 1000, 8, 64, 128, 2, io=io, init_std=0.1)
    log("noalloc call 1", io)
    _both(inp, 256, states=True)
    # second call: smaller sizes, packed documents, on the scratch the first
    # call left behind
    inp = syn.random_case(5101, 1, 300, 4, 32, 64, 1, io=io, init_std=0.0)
    seq = syn.doc_index(5101, 1, 300, lo=16, hi=128)
    log("noalloc call 2", io)
    _both(inp, 100, seq=seq)


def test_noalloc_rejects_sizes_beyond_scratch():
    import mamba_ssd_chunked_chunk_amd as ssd
    from mamba_ssd_chunked_chunk_amd import _lib
    torch = torch_mod()
    b, l, h, p, n, g, Q = 4, 4096, 80, 64, 128, 1, 256
    assert ssd.workspace_bytes(b, l, h, p, n, g, Q) > _lib.SSD_SCRATCH_BYTES
    x = torch.zeros((b, l, h, p), dtype=torch.bfloat16, device="cuda")
    dt = torch.zeros((b, l, h), dtype=torch.bfloat16, device="cuda")
    B = torch.zeros((b, l, g, n), dtype=torch.bfloat16, device="cuda")
    A = -torch.ones(h, dtype=torch.float32, device="cuda")
    y = torch.full_like(x, 3.0)
    with pytest.raises(ssd.SsdError) as e:
        ssd.chunk_scan_noalloc(x, dt, A, B, B, y, chunk_size=Q)
    assert e.value.code == _lib.SSD_ERR_SCRATCH
    torch.cuda.synchronize()
    assert bool((y == 3.0).all()), "a rejected call wrote its output"
