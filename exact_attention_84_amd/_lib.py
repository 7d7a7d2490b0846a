"""ctypes loader of libfa.so (the C ABI declared in include/fa.h).

The library must have been built in-tree (``python -m exact_attention_84_amd.build``
or ``__graft_entry__.build()``).  There is no fallback: a missing or stale
library raises immediately.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("FA_LIB_PATH", os.path.join(_HERE, "libfa.so"))

FA_OK = 0
FA_DTYPE_BF16 = 0
FA_DTYPE_F32 = 1
NOALLOC_SCRATCH_BYTES = 64 << 20  # FA_NOALLOC_SCRATCH_BYTES of fa.h
STATUS_NAMES = {0: "FA_OK", 1: "FA_ERR_NULL", 2: "FA_ERR_SHAPE", 3: "FA_ERR_HEADDIM",
                4: "FA_ERR_GQA", 5: "FA_ERR_DTYPE", 6: "FA_ERR_ARCH", 7: "FA_ERR_WORKSPACE",
                8: "FA_ERR_HIP", 9: "FA_ERR_ARG"}
EXPORTS = ("fa_fwd", "fa_fwd_ext", "fa_fwd_fp8", "fa_decode_workspace_size",
           "fa_fwd_decode_splitkv",
           "fa_decode_kvcache_workspace_size", "fa_fwd_decode_kvcache",
           "fa_fwd_decode_kvcache_noalloc", "fa_combine",
           "fa_bwd_workspace_size", "fa_bwd", "fa_status_string", "fa_last_error")

_lib = None

P = ctypes.c_void_p
I = ctypes.c_int
F = ctypes.c_float


class FaError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        self.status = status
        super().__init__(f"{where}: {STATUS_NAMES.get(status, status)}: {detail}")


def load() -> ctypes.CDLL:
    """Load libfa.so once and declare every exported signature."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python -m exact_attention_84_amd.build` "
            "(the attention path has no fallback)")
    lib = ctypes.CDLL(LIB_PATH)
    lib.fa_fwd.argtypes = [P, P, P, P, P, I, I, I, I, I, I, F, I, P, P, I, I, I, P]
    lib.fa_fwd.restype = I
    lib.fa_decode_workspace_size.argtypes = [I, I, I, I, I]
    lib.fa_decode_workspace_size.restype = ctypes.c_size_t
    lib.fa_fwd_decode_splitkv.argtypes = [P, P, P, P, P, P, I, I, I, I, I, F, I, P,
                                          ctypes.c_size_t, I, P]
    lib.fa_fwd_decode_splitkv.restype = I
    lib.fa_combine.argtypes = [P, P, I, I, I, P, P, I, P]
    lib.fa_combine.restype = I
    lib.fa_fwd_ext.argtypes = [P, P, P, P, P, I, I, I, I, I, I, F, I, P, P, I, I, I, I, F, P, I,
                               I, P]
    lib.fa_fwd_ext.restype = I
    lib.fa_fwd_fp8.argtypes = [P, P, P, P, P, I, I, I, I, I, I, F, F, F, F, I, P, P, I, I, I, P]
    lib.fa_fwd_fp8.restype = I
    lib.fa_decode_kvcache_workspace_size.argtypes = [I, I, I, I, I]
    lib.fa_decode_kvcache_workspace_size.restype = ctypes.c_size_t
    lib.fa_fwd_decode_kvcache.argtypes = [P, P, P, P, P, P, P, I, I, I, P, P, I, I, I, P, P, I, I,
                                          I, I, I, F, I, P, ctypes.c_size_t, I, P]
    lib.fa_fwd_decode_kvcache.restype = I
    lib.fa_fwd_decode_kvcache_noalloc.argtypes = [P, P, P, P, P, P, P, I, I, I, P, P, I, I, I, P,
                                                  P, I, I, I, I, I, F, I, I, P]
    lib.fa_fwd_decode_kvcache_noalloc.restype = I
    lib.fa_bwd_workspace_size.argtypes = [I, I, I]
    lib.fa_bwd_workspace_size.restype = ctypes.c_size_t
    lib.fa_bwd.argtypes = [P, P, P, P, P, P, P, P, P, I, I, I, I, I, I, F, I, P, P, I, I, I, P,
                           ctypes.c_size_t, P]
    lib.fa_bwd.restype = I
    lib.fa_status_string.argtypes = [I]
    lib.fa_status_string.restype = ctypes.c_char_p
    lib.fa_last_error.argtypes = []
    lib.fa_last_error.restype = ctypes.c_char_p
    _lib = lib
    return lib


def check(status: int, where: str) -> None:
    if status != FA_OK:
        detail = load().fa_last_error().decode(errors="replace")
        raise FaError(status, where, detail)
