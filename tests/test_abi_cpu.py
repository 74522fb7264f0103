"""Host-side checks of libssd.so that need no GPU.

The library loads, exports every function include/ssd.h declares, and
rejects invalid arguments with the documented status before touching the
HIP runtime (so these calls are safe on a machine without a GPU: only
argument checking runs).
"""
import ctypes
import math
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ssd.h")


def _lib():
    from mamba_ssd_chunked_chunk_amd import _lib
    try:
        return _lib.load()
    except _lib.LibraryMissing:
        from mamba_ssd_chunked_chunk_amd import build
        build.build(verbose=False)
        return _lib.load()


@pytest.fixture(scope="module")
def lib():
    return _lib()


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ssd_\w+)\s*\(", text)))


def test_exports_every_declared_symbol(lib):
    from mamba_ssd_chunked_chunk_amd import _lib as L
    declared = _declared_functions()
    assert set(declared) == set(L.EXPORTS)
    for name in declared:
        assert hasattr(lib, name), name


def test_abi_version_matches_header(lib):
    m = re.search(r"#define\s+SSD_ABI_VERSION\s+(\d+)", open(HEADER).read())
    assert lib.ssd_abi_version() == int(m.group(1))


def test_status_strings(lib):
    for code in range(0, -8, -1):
        s = lib.ssd_status_string(code)
        assert s and s != b"unknown status"
    assert lib.ssd_status_string(12345) == b"unknown status"


def test_workspace_query_is_pure_and_validating(lib):
    ws = lib.ssd_chunk_scan_workspace_bytes
    a = ws(8, 2048, 24, 64, 128, 1, 256)
    assert a == ws(8, 2048, 24, 64, 128, 1, 256) and a > 0
    # boundary states alone: b * chunks * h * n * p * 4 bytes
    assert a >= 8 * 8 * 24 * 128 * 64 * 4
    assert ws(8, 2048, 24, 64, 128, 5, 256) == 0      # heads % groups
    assert ws(8, 2048, 24, 64, 128, 1, 0) == 0        # chunk
    assert ws(-1, 2048, 24, 64, 128, 1, 256) == 0
    assert ws(0, 2048, 24, 64, 128, 1, 256) >= 0
    assert ws(8, 4096, 24, 64, 128, 1, 256) > a       # grows with length


FAKE = 0x10000  # 256-byte aligned, never dereferenced: every call below fails validation


def _scan(lib, **over):
    kw = dict(x=FAKE, dt=FAKE, A=FAKE, B=FAKE, C=FAKE, D=None, dt_bias=None, sp=1,
              lo=0.0, hi=math.inf, init=None, y=FAKE, fin=None, b=2, l=64, h=4, p=64, n=128,
              g=1, Q=64, io=1, ws=FAKE, wsb=1 << 30, stream=None)
    kw.update(over)
    return lib.ssd_chunk_scan(kw["x"], kw["dt"], kw["A"], kw["B"], kw["C"], kw["D"],
                              kw["dt_bias"], kw["sp"], kw["lo"], kw["hi"], kw["init"], kw["y"],
                              kw["fin"], kw["b"], kw["l"], kw["h"], kw["p"], kw["n"], kw["g"],
                              kw["Q"], kw["io"], kw["ws"], kw["wsb"], kw["stream"])


def test_chunk_scan_rejects_bad_arguments(lib):
    from mamba_ssd_chunked_chunk_amd import _lib as L
    assert _scan(lib, io=7) == L.SSD_ERR_UNSUPPORTED
    assert _scan(lib, b=-1) == L.SSD_ERR_SHAPE
    assert _scan(lib, l=-3) == L.SSD_ERR_SHAPE
    assert _scan(lib, h=0) == L.SSD_ERR_SHAPE
    assert _scan(lib, Q=0) == L.SSD_ERR_SHAPE
    assert _scan(lib, h=6, g=4) == L.SSD_ERR_SHAPE
    assert _scan(lib, p=48) == L.SSD_ERR_UNSUPPORTED
    assert _scan(lib, n=256) == L.SSD_ERR_UNSUPPORTED
    assert _scan(lib, x=None) == L.SSD_ERR_NULL
    assert _scan(lib, A=None) == L.SSD_ERR_NULL
    assert _scan(lib, y=None) == L.SSD_ERR_NULL
    assert _scan(lib, x=FAKE + 8) == L.SSD_ERR_ALIGN
    assert _scan(lib, dt=FAKE + 1) == L.SSD_ERR_ALIGN
    assert _scan(lib, init=FAKE + 4) == L.SSD_ERR_ALIGN
    assert _scan(lib, ws=FAKE + 16) == L.SSD_ERR_ALIGN
    assert _scan(lib, ws=None) == L.SSD_ERR_WORKSPACE
    assert _scan(lib, wsb=1024) == L.SSD_ERR_WORKSPACE


def test_step_rejects_bad_arguments(lib):
    from mamba_ssd_chunked_chunk_amd import _lib as L

    def step(**over):
        kw = dict(state=FAKE, x=FAKE, dt=FAKE, A=FAKE, B=FAKE, C=FAKE, D=None, bias=None,
                  sp=1, lo=0.0, hi=math.inf, y=FAKE, b=4, h=8, p=64, n=128, g=2, io=1,
                  stream=None)
        kw.update(over)
        return lib.ssd_step(kw["state"], kw["x"], kw["dt"], kw["A"], kw["B"], kw["C"], kw["D"],
                            kw["bias"], kw["sp"], kw["lo"], kw["hi"], kw["y"], kw["b"], kw["h"],
                            kw["p"], kw["n"], kw["g"], kw["io"], kw["stream"])
    assert step(io=2) == L.SSD_ERR_UNSUPPORTED
    assert step(h=8, g=3) == L.SSD_ERR_SHAPE
    assert step(b=-1) == L.SSD_ERR_SHAPE
    assert step(p=24) == L.SSD_ERR_UNSUPPORTED
    assert step(state=None) == L.SSD_ERR_NULL
    assert step(C=None) == L.SSD_ERR_NULL
    assert step(state=FAKE + 4) == L.SSD_ERR_ALIGN
    assert step(b=0) == L.SSD_OK     # nothing to do, nothing launched


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    from mamba_ssd_chunked_chunk_amd import _lib as L
    monkeypatch.setattr(L, "_lib", None)
    monkeypatch.setattr(L, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(L.LibraryMissing):
        L.load()


def test_oracle_is_not_on_the_product_path():
    """The package never imports, loads or names the oracle."""
    pkg = os.path.join(ROOT, "mamba_ssd_chunked_chunk_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".hpp", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f)).read()
                assert "oracle" not in text.lower(), os.path.join(dirpath, f)


def test_scan_ex_rejects_bad_arguments(lib):
    from mamba_ssd_chunked_chunk_amd import _lib as L

    def ex(**over):
        kw = dict(seq=None, states=None, b=2, l=64, io=1, wsb=1 << 30)
        kw.update(over)
        return lib.ssd_chunk_scan_ex(FAKE, FAKE, FAKE, FAKE, FAKE, None, None, 1, 0.0, math.inf,
                                     None, kw["seq"], FAKE, None, kw["states"], kw["b"], kw["l"],
                                     4, 64, 128, 1, 64, kw["io"], FAKE, kw["wsb"], None, None)
    assert ex(seq=FAKE + 2) == L.SSD_ERR_ALIGN
    assert ex(states=FAKE + 8) == L.SSD_ERR_ALIGN
    assert ex(io=5) == L.SSD_ERR_UNSUPPORTED
    assert ex(wsb=16) == L.SSD_ERR_WORKSPACE


def test_conv_and_norm_reject_bad_arguments(lib):
    from mamba_ssd_chunked_chunk_amd import _lib as L

    def conv(**over):
        kw = dict(xbc=FAKE, w=FAKE, x=FAKE, B=FAKE, C=FAKE, fin=None, b=2, l=64, h=4, p=64, n=64,
                  g=1, K=4, io=1)
        kw.update(over)
        return lib.ssd_conv1d_silu(kw["xbc"], kw["w"], None, None, None, kw["x"], kw["B"],
                                   kw["C"], kw["fin"], kw["b"], kw["l"], kw["h"], kw["p"],
                                   kw["n"], kw["g"], kw["K"], 1, kw["io"], None)
    assert conv(K=5) == L.SSD_ERR_UNSUPPORTED
    assert conv(K=0) == L.SSD_ERR_SHAPE
    assert conv(p=18) == L.SSD_ERR_UNSUPPORTED
    assert conv(io=3) == L.SSD_ERR_UNSUPPORTED
    assert conv(xbc=None) == L.SSD_ERR_NULL
    assert conv(x=FAKE + 4) == L.SSD_ERR_ALIGN
    assert conv(b=0) == L.SSD_OK

    def norm(**over):
        kw = dict(y=FAKE, out=FAKE, rows=8, dim=64, G=16, eps=1e-5, io=1)
        kw.update(over)
        return lib.ssd_gated_norm(kw["y"], None, None, kw["out"], kw["rows"], kw["dim"], kw["G"],
                                  kw["eps"], 1, kw["io"], None)
    assert norm(G=24) == L.SSD_ERR_SHAPE          # does not divide dim
    assert norm(G=6, dim=60) == L.SSD_ERR_UNSUPPORTED
    assert norm(eps=-1.0) == L.SSD_ERR_SHAPE
    assert norm(y=None) == L.SSD_ERR_NULL
    assert norm(out=FAKE + 2) == L.SSD_ERR_ALIGN
    assert norm(rows=0) == L.SSD_OK


def test_backward_and_segments_reject_bad_arguments(lib):
    from mamba_ssd_chunked_chunk_amd import _lib as L

    def bwd(**over):
        kw = dict(p=64, n=128, b=2, l=64, dy=FAKE, dx=FAKE, wsb=1 << 34, io=1)
        kw.update(over)
        return lib.ssd_chunk_scan_bwd(FAKE, FAKE, FAKE, FAKE, FAKE, None, None, 1, 0.0, math.inf,
                                      None, None, kw["dy"], None, kw["dx"], FAKE, FAKE, FAKE,
                                      FAKE, None, None, None, kw["b"], kw["l"], 4, kw["p"],
                                      kw["n"], 1, 64, kw["io"], FAKE, kw["wsb"], None)
    assert bwd(p=16) == L.SSD_ERR_UNSUPPORTED      # head_dim becomes a state size
    assert bwd(b=0) == L.SSD_ERR_SHAPE
    assert bwd(dy=None) == L.SSD_ERR_NULL
    assert bwd(dx=FAKE + 8) == L.SSD_ERR_ALIGN
    assert bwd(wsb=1024) == L.SSD_ERR_WORKSPACE
    for io in (L.SSD_F32, L.SSD_BF16):
        assert lib.ssd_chunk_scan_bwd_workspace_bytes(2, 64, 4, 64, 128, 1, 64, io) > 0
        assert lib.ssd_chunk_scan_bwd_workspace_bytes(2, 64, 4, 64, 128, 3, 64, io) == 0
    assert lib.ssd_chunk_scan_bwd_workspace_bytes(2, 64, 4, 64, 128, 1, 64, 7) == 0
    assert lib.ssd_combine_segments(FAKE, FAKE, None, None, None, None, 0, 2, 4, 64, 64,
                                    None) == L.SSD_ERR_SHAPE
    assert lib.ssd_combine_segments(None, FAKE, None, None, None, None, 2, 2, 4, 64, 64,
                                    None) == L.SSD_ERR_NULL
    assert lib.ssd_segment_log_decay(FAKE, None, None, 1, 0.0, math.inf, None, FAKE, 2, 64, 4, 1,
                                     None) == L.SSD_ERR_NULL
    assert lib.ssd_segment_log_decay(FAKE, FAKE, None, 1, 0.0, math.inf, None, FAKE, 2, 64, 4, 9,
                                     None) == L.SSD_ERR_UNSUPPORTED


def test_noalloc_scratch_size_matches_header_and_rejects_beyond_it(lib):
    """ssd_chunk_scan_noalloc rejects sizes whose workspace exceeds the
    static scratch before any HIP call (the pointers below are never
    dereferenced), and the binding's size is the header's."""
    from mamba_ssd_chunked_chunk_amd import _lib as L
    m = re.search(r"#define\s+SSD_SCRATCH_BYTES\s+\((\d+)u\s*<<\s*(\d+)\)",
                  open(HEADER).read())
    assert m and int(m.group(1)) << int(m.group(2)) == L.SSD_SCRATCH_BYTES
    b, l, h, p, n, g, Q = 4, 4096, 80, 64, 128, 1, 256
    need = lib.ssd_chunk_scan_workspace_bytes(b, l, h, p, n, g, Q)
    assert need > L.SSD_SCRATCH_BYTES
    fake = ctypes.c_void_p(1 << 20)
    rc = lib.ssd_chunk_scan_noalloc(fake, fake, fake, fake, fake, None, None, 1, 0.0,
                                    math.inf, None, None, fake, None, None, b, l, h, p, n, g,
                                    Q, L.SSD_BF16, None, None)
    assert rc == L.SSD_ERR_SCRATCH
    assert b"SSD_SCRATCH_BYTES" in lib.ssd_status_string(rc)


def test_mixer_checks_every_pass_before_launching(lib):
    """ssd_mixer_forward returns the status of whichever of its three passes
    rejects an argument, before its first launch (on this machine a launch
    would report SSD_ERR_HIP instead)."""
    from mamba_ssd_chunked_chunk_amd import _lib as L
    b, l, h, p, n, g, Q = 2, 64, 4, 64, 64, 1, 64
    wsb = lib.ssd_mixer_workspace_bytes(b, l, h, p, n, g, Q, 1)
    assert wsb > lib.ssd_chunk_scan_workspace_bytes(b, l, h, p, n, g, Q) + b * l * h * p * 2
    assert lib.ssd_mixer_workspace_bytes(b, l, h, p, n, g, 0, 1) == 0
    assert lib.ssd_mixer_workspace_bytes(b, l, h, p, n, g, Q, 7) == 0

    def mix(**over):
        kw = dict(xbc=FAKE, z=None, dt=FAKE, K=4, G=h * p, eps=1e-5, out=FAKE, b=b, l=l, p=p,
                  io=1, ws=FAKE, wsb=wsb, init=None, seq=None)
        kw.update(over)
        return lib.ssd_mixer_forward(kw["xbc"], kw["z"], kw["dt"], FAKE, None, kw["K"], None,
                                     None, FAKE, None, None, 1, 0.0, math.inf, kw["init"], None,
                                     kw["seq"], None, kw["G"], kw["eps"], 1, kw["out"], kw["b"],
                                     kw["l"], h, kw["p"], n, g, Q, kw["io"], kw["ws"], kw["wsb"],
                                     None)
    assert mix(wsb=wsb - 1) == L.SSD_ERR_WORKSPACE
    assert mix(ws=None) == L.SSD_ERR_WORKSPACE
    assert mix(ws=FAKE + 16) == L.SSD_ERR_ALIGN
    assert mix(K=5) == L.SSD_ERR_UNSUPPORTED           # the conv's check
    assert mix(xbc=FAKE + 4) == L.SSD_ERR_ALIGN        # the conv's check
    assert mix(dt=FAKE + 1) == L.SSD_ERR_ALIGN         # the scan's check
    assert mix(init=FAKE + 8) == L.SSD_ERR_ALIGN       # the scan's check
    assert mix(seq=FAKE + 2) == L.SSD_ERR_ALIGN
    assert mix(G=24) == L.SSD_ERR_SHAPE                # the norm's check
    assert mix(eps=-1.0) == L.SSD_ERR_SHAPE            # the norm's check
    assert mix(z=FAKE + 2) == L.SSD_ERR_ALIGN          # the norm's check
    assert mix(out=None) == L.SSD_ERR_NULL
    assert mix(io=4) == L.SSD_ERR_UNSUPPORTED
    assert mix(p=18) == L.SSD_ERR_UNSUPPORTED
    assert mix(b=0, wsb=lib.ssd_mixer_workspace_bytes(0, l, h, p, n, g, Q, 1)) == L.SSD_OK
