"""ctypes loader for libfa.so: declares the C ABI of include/fa.h.

There is no fallback: if the library is missing the calls raise, so nothing
silently runs anywhere but the HIP kernels.
"""
from __future__ import annotations

import ctypes
import operator
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libfa.so")
# The race-check build of the same sources (every LDS phase closed by a full
# wait and a barrier); only the tests load it, to compare with libfa.so.
SYNC_LIB_PATH = os.path.join(_PKG, "libfa_sync.so")

FA_OK = 0
STATUS_NAMES = {
    0: "FA_OK", -1: "FA_ERR_NULL", -2: "FA_ERR_SHAPE", -3: "FA_ERR_HEAD_DIM", -4: "FA_ERR_GQA",
    -5: "FA_ERR_ALIGN", -6: "FA_ERR_WORKSPACE", -7: "FA_ERR_LAUNCH", -8: "FA_ERR_ARG", -9: "FA_ERR_SCRATCH",
}

_lib = None


class FaError(RuntimeError):
    """A libfa call returned a non-zero status."""

    def __init__(self, status: int, where: str):
        self.status = status
        msg = _load().fa_status_string(status).decode()
        super().__init__(f"{where}: {msg} (status {status})")


class _Int32(ctypes.c_int):
    """int argument that raises instead of wrapping (plain c_int keeps the low 32 bits)."""

    @classmethod
    def from_param(cls, value):
        value = operator.index(value)
        if not -(1 << 31) <= value < (1 << 31):
            raise OverflowError(f"{value} does not fit a C int")
        return ctypes.c_int(value)


class _Size(ctypes.c_size_t):
    """size_t argument that rejects negative and oversized values instead of wrapping."""

    @classmethod
    def from_param(cls, value):
        value = operator.index(value)
        if not 0 <= value < (1 << (8 * ctypes.sizeof(ctypes.c_size_t))):
            raise OverflowError(f"{value} does not fit a C size_t")
        return ctypes.c_size_t(value)


def _declare(lib):
    vp, i, f, sz = ctypes.c_void_p, _Int32, ctypes.c_float, _Size
    lib.fa_fwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, vp]
    lib.fa_fwd.restype = ctypes.c_int
    lib.fa_fwd_workspace_bytes.argtypes = [i, i, i, i]
    lib.fa_fwd_workspace_bytes.restype = ctypes.c_size_t
    lib.fa_fwd_ws.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, vp, sz, vp]
    lib.fa_fwd_ws.restype = ctypes.c_int
    lib.fa_fwd_ws_timed.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, vp, sz, vp, vp]
    lib.fa_fwd_ws_timed.restype = ctypes.c_int
    lib.fa_fwd_noalloc.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, vp]
    lib.fa_fwd_noalloc.restype = ctypes.c_int
    lib.fa_fwd_noalloc_max_scratch_bytes.argtypes = []
    lib.fa_fwd_noalloc_max_scratch_bytes.restype = ctypes.c_size_t
    lib.fa_fwd_fp8.argtypes = [vp, vp, vp, f, f, f, vp, vp, i, i, i, i, i, i, f, vp]
    lib.fa_fwd_fp8.restype = ctypes.c_int
    lib.fa_fwd_fp8_ws.argtypes = [vp, vp, vp, f, f, f, vp, vp, i, i, i, i, i, i, f, vp, sz, vp]
    lib.fa_fwd_fp8_ws.restype = ctypes.c_int
    lib.fa_decode_workspace_bytes.argtypes = [i, i, i, i, i]
    lib.fa_decode_workspace_bytes.restype = ctypes.c_size_t
    lib.fa_decode.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, vp, sz, vp]
    lib.fa_decode.restype = ctypes.c_int
    lib.fa_decode_varlen.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, f, vp, sz, vp]
    lib.fa_decode_varlen.restype = ctypes.c_int
    lib.fa_bwd_workspace_bytes.argtypes = [i, i, i, i]
    lib.fa_bwd_workspace_bytes.restype = ctypes.c_size_t
    lib.fa_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, f, vp, sz, vp]
    lib.fa_bwd.restype = ctypes.c_int
    lib.fa_status_string.argtypes = [i]
    lib.fa_status_string.restype = ctypes.c_char_p
    return lib


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is not built; run `python -c 'import __graft_entry__ as g; g.build()'` "
                "or `python exact_tiled_attention_fa_amd/build.py`")
        _lib = _declare(ctypes.CDLL(LIB_PATH))
    return _lib


def lib():
    return _load()


def open_library(path: str):
    """Load another build of the same C ABI (e.g. SYNC_LIB_PATH) with its
    argument types declared; the package's own calls keep using libfa.so."""
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run exact_tiled_attention_fa_amd/build.py")
    return _declare(ctypes.CDLL(path))


def check(status: int, where: str) -> None:
    if status != FA_OK:
        raise FaError(status, where)
