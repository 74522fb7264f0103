"""A sequence split into segments on one GPU (the sequence-sharded scan,
through the C ABI): pass 1 from zero states, ssd_segment_log_decay and
ssd_combine_segments, pass 2 from the entry states; against one pass and
the oracle."""
import numpy as np
import pytest

import ssd_synth as syn
from gpu_util import STATE_AXES, Y_AXES, check_close, gpu_inputs, oracle_kw, to_f64, torch_mod

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("init", [0.0, 0.3])
@pytest.mark.parametrize("packed", [False, True])
def test_segments_match_one_pass(io, init, packed):
    import mamba_ssd_chunked_chunk_amd as ssd
    import oracle
    torch = torch_mod()
    b, l, h, p, n, g, Q = 2, 600, 4, 64, 64, 2, 64
    inp = syn.random_case(6000 + int(10 * init) + packed, b, l, h, p, n, g, io=io, init_std=init)
    gi = gpu_inputs(inp)
    seq = None
    if packed:
        seq = np.zeros((b, l), np.int32)
        seq[0, 100:] = 1
        seq[0, 256:] = 2    # starts exactly at a segment start
        seq[1, 300:] = 7    # crosses a segment boundary
    sqd = None if seq is None else torch.from_numpy(seq).to("cuda")
    cuts = [0, 256, 450, 600]   # ragged segments
    K = len(cuts) - 1
    segs = []
    for k in range(K):
        lo, hi = cuts[k], cuts[k + 1]
        segs.append({key: gi[key][:, lo:hi].contiguous() for key in ("x", "dt", "B", "C")})
        segs[-1]["seq"] = None if sqd is None else sqd[:, lo:hi].contiguous()
    # pass 1: every segment from a zero state
    S = torch.empty((K, b, h, n, p), dtype=torch.float32, device="cuda")
    L = torch.empty((K, b, h), dtype=torch.float32, device="cuda")
    for k, sg in enumerate(segs):
        _, S[k] = ssd.chunk_scan(sg["x"], sg["dt"], gi["A"], sg["B"], sg["C"], gi["D"],
                                 chunk_size=Q, dt_bias=gi["dt_bias"], return_final_state=True,
                                 seq_idx=sg["seq"])
        L[k] = ssd.segment_log_decay(sg["dt"], gi["A"], dt_bias=gi["dt_bias"], seq_idx=sg["seq"])
    starts = None
    if seq is not None:
        st = np.zeros((K, b), np.int32)
        for k in range(1, K):
            st[k] = seq[:, cuts[k]] != seq[:, cuts[k] - 1]
        starts = torch.from_numpy(st).to("cuda")
    entry, fin = ssd.combine_segments(L, S, initial_state=gi["init"], starts_document=starts)
    # pass 2: every segment from its entry state
    ys = []
    for k, sg in enumerate(segs):
        ys.append(ssd.chunk_scan(sg["x"], sg["dt"], gi["A"], sg["B"], sg["C"], gi["D"],
                                 chunk_size=Q, dt_bias=gi["dt_bias"],
                                 initial_state=None if (k == 0 and gi["init"] is None) else entry[k],
                                 seq_idx=sg["seq"]))
    y = torch.cat(ys, 1)
    torch.cuda.synchronize()
    yo, fo = oracle.scan(**oracle_kw(inp), seq_idx=seq)
    check_close(to_f64(y), yo, io, "y from segments", Y_AXES)
    check_close(to_f64(fin), fo, io, "final state from segments", STATE_AXES)
