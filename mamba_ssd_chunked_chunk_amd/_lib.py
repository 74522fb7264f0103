"""ctypes view of libssd.so (the C ABI declared in include/ssd.h)."""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libssd.so")

SSD_F32 = 0
SSD_BF16 = 1
SSD_OK = 0
SSD_ERR_NULL = -1
SSD_ERR_SHAPE = -2
SSD_ERR_UNSUPPORTED = -3
SSD_ERR_WORKSPACE = -4
SSD_ERR_ALIGN = -5
SSD_ERR_HIP = -6
SSD_ERR_SCRATCH = -7
# bytes of the static device scratch of ssd_chunk_scan_noalloc
SSD_SCRATCH_BYTES = 128 << 20

# kernel_events slots of ssd_chunk_scan_ex
EVENT_SLOTS = ("chunk_state", "state_scan", "chunk_out", "token_states")

# every symbol include/ssd.h declares
EXPORTS = ("ssd_chunk_scan", "ssd_chunk_scan_ex", "ssd_chunk_scan_noalloc",
           "ssd_chunk_scan_workspace_bytes", "ssd_chunk_scan_state_chunks", "ssd_step",
           "ssd_conv1d_silu", "ssd_gated_norm", "ssd_mixer_forward",
           "ssd_mixer_workspace_bytes", "ssd_chunk_scan_bwd",
           "ssd_segment_log_decay", "ssd_combine_segments",
           "ssd_chunk_scan_bwd_workspace_bytes", "ssd_status_string", "ssd_abi_version")

_lib = None


class LibraryMissing(RuntimeError):
    pass


def load() -> ctypes.CDLL:
    """Load libssd.so from the package directory (never a fallback)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise LibraryMissing(
            "libssd.so is not built (%s); run `python -m mamba_ssd_chunked_chunk_amd.build`"
            % LIB_PATH)
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, I64, F = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float
    lib.ssd_chunk_scan.restype = I32
    lib.ssd_chunk_scan.argtypes = [P, P, P, P, P, P, P, I32, F, F, P, P, P,
                                   I64, I64, I64, I64, I64, I64, I64, I32,
                                   P, ctypes.c_size_t, P]
    lib.ssd_chunk_scan_ex.restype = I32
    lib.ssd_chunk_scan_ex.argtypes = [P, P, P, P, P, P, P, I32, F, F, P, P, P, P, P,
                                      I64, I64, I64, I64, I64, I64, I64, I32,
                                      P, ctypes.c_size_t, P, P]
    lib.ssd_chunk_scan_noalloc.restype = I32
    lib.ssd_chunk_scan_noalloc.argtypes = [P, P, P, P, P, P, P, I32, F, F, P, P, P, P, P,
                                           I64, I64, I64, I64, I64, I64, I64, I32, P, P]
    lib.ssd_chunk_scan_workspace_bytes.restype = ctypes.c_size_t
    lib.ssd_chunk_scan_workspace_bytes.argtypes = [I64] * 7
    lib.ssd_chunk_scan_state_chunks.restype = I64
    lib.ssd_chunk_scan_state_chunks.argtypes = [I64] * 7 + [I32, I32]
    lib.ssd_step.restype = I32
    lib.ssd_step.argtypes = [P, P, P, P, P, P, P, P, I32, F, F, P,
                             I64, I64, I64, I64, I64, I32, P]
    lib.ssd_conv1d_silu.restype = I32
    lib.ssd_conv1d_silu.argtypes = [P, P, P, P, P, P, P, P, P, I64, I64, I64, I64, I64, I64,
                                    I64, I32, I32, P]
    lib.ssd_gated_norm.restype = I32
    lib.ssd_gated_norm.argtypes = [P, P, P, P, I64, I64, I64, F, I32, I32, P]
    lib.ssd_mixer_forward.restype = I32
    lib.ssd_mixer_forward.argtypes = [P, P, P, P, P, I64, P, P, P, P, P, I32, F, F, P, P, P, P,
                                      I64, F, I32, P, I64, I64, I64, I64, I64, I64, I64, I32,
                                      P, ctypes.c_size_t, P]
    lib.ssd_mixer_workspace_bytes.restype = ctypes.c_size_t
    lib.ssd_mixer_workspace_bytes.argtypes = [I64] * 7 + [I32]
    lib.ssd_chunk_scan_bwd.restype = I32
    lib.ssd_chunk_scan_bwd.argtypes = [P, P, P, P, P, P, P, I32, F, F, P, P, P, P,
                                       P, P, P, P, P, P, P, P,
                                       I64, I64, I64, I64, I64, I64, I64, I32,
                                       P, ctypes.c_size_t, P]
    lib.ssd_chunk_scan_bwd_workspace_bytes.restype = ctypes.c_size_t
    lib.ssd_chunk_scan_bwd_workspace_bytes.argtypes = [I64] * 7 + [I32]
    lib.ssd_segment_log_decay.restype = I32
    lib.ssd_segment_log_decay.argtypes = [P, P, P, I32, F, F, P, P, I64, I64, I64, I32, P]
    lib.ssd_combine_segments.restype = I32
    lib.ssd_combine_segments.argtypes = [P, P, P, P, P, P, I64, I64, I64, I64, I64, P]
    lib.ssd_status_string.restype = ctypes.c_char_p
    lib.ssd_status_string.argtypes = [I32]
    lib.ssd_abi_version.restype = I32
    lib.ssd_abi_version.argtypes = []
    _lib = lib
    return lib


def status_string(code: int) -> str:
    return load().ssd_status_string(int(code)).decode()
