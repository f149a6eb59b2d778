"""ctypes loader for libfa.so.  No compute happens here.

The library is loaded from this package directory only.  If it is missing the
import of any compute entry point raises immediately: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfa.so")

FA_F32, FA_F16, FA_BF16 = 0, 1, 2
STATUS = {
    0: "FA_OK",
    1: "FA_ERR_NULL",
    2: "FA_ERR_SHAPE",
    3: "FA_ERR_HEADDIM",
    4: "FA_ERR_DTYPE",
    5: "FA_ERR_SCALE",
    6: "FA_ERR_ALIGN",
    7: "FA_ERR_WORKSPACE",
    8: "FA_ERR_HIP",
    9: "FA_ERR_SCRATCH",
}
FA_SCRATCH_BYTES = 64 << 20
# every symbol include/fa.h declares
EXPORTS = ("fa_fwd", "fa_fwd_stats", "fa_fwd_stats_bytes", "fa_fwd_split",
           "fa_fwd_split_noalloc", "fa_fwd_split_suggest", "fa_fwd_split_workspace_bytes", "fa_naive_fwd", "fa_naive_workspace_bytes", "fa_bwd", "fa_bwd_workspace_bytes",
           "fa_bwd_split", "fa_bwd_split_workspace_bytes", "fa_bwd_split_suggest",
           "fa_status_string", "fa_version", "fa_last_hip_error")

_lib = None


class FAError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str = ""):
        self.status = status
        super().__init__(f"{where}: {STATUS.get(status, status)} ({detail})")


def load():
    """Load libfa.so and declare its C signatures.  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} not found: build it with `python -m exact_attention_90_amd.build` "
            "(the HIP library is required; there is no CPU fallback)")
    lib = ctypes.CDLL(LIB_PATH)
    P, I, F = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    lib.fa_fwd.argtypes = [P, P, P, P, P, I, I, I, I, F, I, P]
    lib.fa_fwd.restype = I
    lib.fa_fwd_split.argtypes = [P, P, P, P, P, P, I, I, I, I, I, F, I, P]
    lib.fa_fwd_split.restype = I
    lib.fa_fwd_stats.argtypes = [P, P, P, P, P, P, I, I, I, I, F, I, P]
    lib.fa_fwd_stats.restype = I
    lib.fa_fwd_stats_bytes.argtypes = [I, I, I]
    lib.fa_fwd_stats_bytes.restype = ctypes.c_size_t
    lib.fa_fwd_split_noalloc.argtypes = [P, P, P, P, P, I, I, I, I, I, F, I, P]
    lib.fa_fwd_split_noalloc.restype = I
    lib.fa_fwd_split_suggest.argtypes = [I, I, I, I, I]
    lib.fa_fwd_split_suggest.restype = I
    lib.fa_fwd_split_workspace_bytes.argtypes = [I, I, I, I, I]
    lib.fa_fwd_split_workspace_bytes.restype = ctypes.c_size_t
    lib.fa_naive_fwd.argtypes = [P, P, P, P, P, P, P, I, I, I, I, F, I, P]
    lib.fa_naive_fwd.restype = I
    lib.fa_naive_workspace_bytes.argtypes = [I, I, I, I]
    lib.fa_naive_workspace_bytes.restype = ctypes.c_size_t
    lib.fa_bwd.argtypes = [P, P, P, P, P, P, P, P, P, P, I, I, I, I, F, I, P]
    lib.fa_bwd.restype = I
    lib.fa_bwd_workspace_bytes.argtypes = [I, I, I, I, I]
    lib.fa_bwd_workspace_bytes.restype = ctypes.c_size_t
    lib.fa_bwd_split.argtypes = [P, P, P, P, P, P, P, P, P, P, I, I, I, I, I, F, I, P]
    lib.fa_bwd_split.restype = I
    lib.fa_bwd_split_workspace_bytes.argtypes = [I, I, I, I, I, I]
    lib.fa_bwd_split_workspace_bytes.restype = ctypes.c_size_t
    lib.fa_bwd_split_suggest.argtypes = [I, I, I, I, I]
    lib.fa_bwd_split_suggest.restype = I
    lib.fa_status_string.argtypes = [I]
    lib.fa_status_string.restype = ctypes.c_char_p
    lib.fa_version.argtypes = []
    lib.fa_version.restype = ctypes.c_char_p
    lib.fa_last_hip_error.argtypes = []
    lib.fa_last_hip_error.restype = I
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().fa_status_string(status).decode()


def check(status: int, where: str):
    if status != 0:
        lib = load()
        detail = lib.fa_status_string(status).decode()
        if status == 8:
            detail += f"; hipError {lib.fa_last_hip_error()}"
        raise FAError(status, where, detail)
