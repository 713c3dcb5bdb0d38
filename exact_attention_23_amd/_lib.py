"""ctypes view of libfa.so: the declarations of include/fa.h, nothing more."""
from __future__ import annotations

import ctypes
import os

from .build import LIB_PATH

FA_OK = 0
FA_ERR_NULLPTR = 1
FA_ERR_SHAPE = 2
FA_ERR_HEADDIM = 3
FA_ERR_DTYPE = 4
FA_ERR_SCALE = 5
FA_ERR_CAUSAL = 6
FA_ERR_ALIGN = 7
FA_ERR_ALIAS = 8
FA_ERR_LAUNCH = 9
FA_ERR_PATH = 10
FA_ERR_WORKSPACE = 11
FA_ERR_STRIDE = 12
FA_ERR_SCRATCH = 13
FA_BWD_NOALLOC_SCRATCH_BYTES = 16 << 20

FA_PATH_AUTO = 0
FA_PATH_TILED = 1
FA_PATH_SHORT = 2

FA_BWD_PRE = 1
FA_BWD_DKDV = 2
FA_BWD_DQ = 4
FA_BWD_ALL = 7

FA_DTYPE_FP16 = 0
FA_DTYPE_BF16 = 1

_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libfa.so (built in-tree by exact_attention_23_amd.build).

    Raises RuntimeError when it has not been built: there is no other path.
    """
    global _lib
    if _lib is not None:
        return _lib
    # PyTorch ships its own HIP runtime under the same soname. Loading torch
    # first makes libfa.so bind to that copy, so the process has one HIP
    # runtime; loaded the other way round, torch would bring a second one
    # that shares no device state with ours.
    try:
        import torch  # noqa: F401
    except ImportError:  # the C ABI checks still work without torch
        pass
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it with `python -m exact_attention_23_amd.build` "
            "(there is no fallback implementation)")
    lib = ctypes.CDLL(path)
    i64, vp = ctypes.c_int64, ctypes.c_void_p
    lib.fa_fwd.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64,
                           ctypes.c_float, ctypes.c_int, ctypes.c_int, vp]
    lib.fa_fwd.restype = ctypes.c_int
    lib.fa_fwd_ex.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64,
                              ctypes.c_float, ctypes.c_int, ctypes.c_int, ctypes.c_int, vp]
    lib.fa_fwd_ex.restype = ctypes.c_int
    lib.fa_fwd_strided.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, vp,
                                   ctypes.c_float, ctypes.c_int, ctypes.c_int, vp]
    lib.fa_fwd_strided.restype = ctypes.c_int
    lib.fa_fwd_stream_workspace_bytes.argtypes = [i64, i64, i64, i64, i64, ctypes.c_int]
    lib.fa_fwd_stream_workspace_bytes.restype = i64
    lib.fa_fwd_stream_advised.argtypes = [i64, i64, i64, i64, i64, ctypes.c_int, ctypes.c_int]
    lib.fa_fwd_stream_advised.restype = ctypes.c_int
    lib.fa_fwd_stream.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, ctypes.c_float,
                                  ctypes.c_int, ctypes.c_int, vp, i64, vp]
    lib.fa_fwd_stream.restype = ctypes.c_int
    lib.fa_fwd_fp8.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, ctypes.c_float,
                               ctypes.c_float, ctypes.c_float, ctypes.c_float, ctypes.c_int,
                               ctypes.c_int, vp]
    lib.fa_fwd_fp8.restype = ctypes.c_int
    lib.fa_bwd_workspace_bytes.argtypes = [i64, i64, i64]
    lib.fa_bwd_workspace_bytes.restype = i64
    lib.fa_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64,
                           ctypes.c_float, ctypes.c_int, ctypes.c_int, vp]
    lib.fa_bwd.restype = ctypes.c_int
    lib.fa_bwd_ex.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64,
                              ctypes.c_float, ctypes.c_int, ctypes.c_int, ctypes.c_int, vp]
    lib.fa_bwd_ex.restype = ctypes.c_int
    lib.fa_bwd_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64,
                                   ctypes.c_float, ctypes.c_int, ctypes.c_int, vp]
    lib.fa_bwd_noalloc.restype = ctypes.c_int
    lib.fa_std_row_stride.argtypes = [i64]
    lib.fa_std_row_stride.restype = i64
    lib.fa_std_fwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, ctypes.c_float,
                               ctypes.c_int, ctypes.c_int, vp]
    lib.fa_std_fwd.restype = ctypes.c_int
    lib.fa_status_str.argtypes = [ctypes.c_int]
    lib.fa_status_str.restype = ctypes.c_char_p
    lib.fa_last_launch_error.argtypes = []
    lib.fa_last_launch_error.restype = ctypes.c_char_p
    lib.fa_version.argtypes = []
    lib.fa_version.restype = ctypes.c_int
    _lib = lib
    return lib
