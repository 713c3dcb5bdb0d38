"""MI355X (gfx950) exact-attention forward: Python binding of libfa.so.

The binding only marshals arguments; every step of the computation runs in
the HIP kernels behind the C ABI declared in include/fa.h. PyTorch supplies
device memory and the current stream. There is no CPU or PyTorch fallback: a
missing library or an unsupported argument raises.
"""
from __future__ import annotations

import math
from typing import Optional, Tuple

from . import _lib
from ._lib import (FA_DTYPE_BF16, FA_DTYPE_FP16, FA_OK, FA_PATH_AUTO,  # noqa: F401
                   FA_PATH_SHORT, FA_PATH_TILED)

__all__ = ["FaError", "fa_fwd", "fa_fwd_ex", "attention", "version"]

_PATHS = {"auto": FA_PATH_AUTO, "tiled": FA_PATH_TILED, "short": FA_PATH_SHORT}


class FaError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"fa_fwd failed with status {status}: {msg}")
        self.status = status


def version() -> int:
    return _lib.load().fa_version()


def status_str(status: int) -> str:
    return _lib.load().fa_status_str(status).decode()


def fa_fwd(q: int, k: int, v: int, o: int, lse: Optional[int], B: int, H: int, Nq: int,
           Nk: int, d: int, scale: float, causal: int, dtype: int, stream: int) -> int:
    """Direct call of the C entry point with raw device addresses; returns the status."""
    return _lib.load().fa_fwd(q, k, v, o, lse or None, B, H, Nq, Nk, d, float(scale),
                              int(causal), int(dtype), stream or None)


def fa_fwd_ex(q: int, k: int, v: int, o: int, lse: Optional[int], B: int, H: int, Nq: int,
              Nk: int, d: int, scale: float, causal: int, dtype: int, path: int,
              stream: int) -> int:
    """fa_fwd with an explicit kernel choice (FA_PATH_*); returns the status."""
    return _lib.load().fa_fwd_ex(q, k, v, o, lse or None, B, H, Nq, Nk, d, float(scale),
                                 int(causal), int(dtype), int(path), stream or None)


def _current_stream(device_index: int):
    """Raw handle of the current stream of a device (None: the null stream).

    torch's private raw getter costs ~0.1 µs against ~3 µs for building a
    Stream object through the public API, which dominates short calls; the
    public API is the fallback."""
    import torch

    raw = getattr(torch._C, "_cuda_getCurrentRawStream", None)
    h = raw(device_index) if raw is not None else torch.cuda.current_stream(device_index).cuda_stream
    return h or None


def _dtype_code(t) -> int:
    import torch

    if t.dtype == torch.float16:
        return FA_DTYPE_FP16
    if t.dtype == torch.bfloat16:
        return FA_DTYPE_BF16
    raise TypeError(f"unsupported dtype {t.dtype}: fp16 or bf16 expected")


def attention(q, k, v, *, causal: bool = False, scale: Optional[float] = None,
              out=None, lse=None, return_lse: bool = True, path: str = "auto"):
    """O = softmax(scale * Q K^T [causal mask]) V on the GPU, plus LSE.

    q: [B, H, Nq, d], k and v: [B, H, Nk, d], contiguous fp16/bf16 CUDA (HIP)
    tensors on one device. scale=None means 1/sqrt(d). Returns (out, lse) with
    lse [B, H, Nq] float32, or (out, None) when return_lse is False. The work
    is enqueued on the current stream of q's device. path selects the kernel
    ("auto", "tiled" or "short"; see fa_path in include/fa.h).
    """
    import torch

    for name, t in (("q", q), ("k", k), ("v", v)):
        if not isinstance(t, torch.Tensor) or not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor")
        if t.dim() != 4 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous [B, H, N, d] tensor")
    if not (q.device == k.device == v.device):
        raise ValueError("q, k, v must be on one device")
    if not (q.dtype == k.dtype == v.dtype):
        raise ValueError("q, k, v must share a dtype")
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    if tuple(k.shape) != (B, H, Nk, d) or tuple(v.shape) != (B, H, Nk, d):
        raise ValueError("k and v must be [B, H, Nk, d] matching q")
    code = _dtype_code(q)
    if path not in _PATHS:
        raise ValueError(f"path must be one of {sorted(_PATHS)}")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    elif (out.shape != q.shape or out.dtype != q.dtype or out.device != q.device
          or not out.is_contiguous()):
        raise ValueError("out must be a contiguous tensor like q")
    if lse is None and return_lse:
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    elif lse is not None and (tuple(lse.shape) != (B, H, Nq) or lse.dtype != torch.float32
                              or lse.device != q.device or not lse.is_contiguous()):
        raise ValueError("lse must be a contiguous float32 [B, H, Nq] tensor")
    lib = _lib.load()
    call = (q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
            lse.data_ptr() if lse is not None else None,
            B, H, Nq, Nk, d, float(scale), 1 if causal else 0, code, _PATHS[path])
    # The launch goes to the current device; switch only when q lives elsewhere
    # (the device guard costs several microseconds per call).
    idx = q.device.index
    if idx == torch.cuda.current_device():
        st = lib.fa_fwd_ex(*call, _current_stream(idx))
    else:
        with torch.cuda.device(q.device):
            st = lib.fa_fwd_ex(*call, _current_stream(idx))
    if st != FA_OK:
        msg = status_str(st)
        if st == _lib.FA_ERR_LAUNCH:
            msg += ": " + _lib.load().fa_last_launch_error().decode()
        raise FaError(st, msg)
    return out, lse
