"""MI355X (gfx950) exact attention, forward and backward: Python binding of libfa.so.

The binding only marshals arguments; every step of the computation runs in
the HIP kernels behind the C ABI declared in include/fa.h. PyTorch supplies
device memory and the current stream. There is no CPU or PyTorch fallback: a
missing library or an unsupported argument raises.
"""
from __future__ import annotations

import collections
import ctypes
import math
from typing import Optional, Tuple

from . import _lib
from ._lib import (FA_DTYPE_BF16, FA_DTYPE_FP16, FA_OK, FA_PATH_AUTO,  # noqa: F401
                   FA_PATH_SHORT, FA_PATH_TILED)

__all__ = ["FaError", "fa_fwd", "fa_fwd_ex", "fa_fwd_strided", "attention_fp8", "fa_bwd",
           "fa_bwd_ex", "fa_bwd_noalloc", "fa_bwd_workspace_bytes", "attention", "attention_backward",
           "flash_attention", "release_workspaces", "standard_attention", "fa_std_fwd", "version"]

_PATHS = {"auto": FA_PATH_AUTO, "tiled": FA_PATH_TILED, "short": FA_PATH_SHORT, "stream": -1}

# Workspaces of the stream form, one per (device, stream): calls on one stream
# run in order, so they can share it. At most _STREAM_WS_MAX are kept (the
# least recently used goes first); release_workspaces() drops them all.
_STREAM_WS = collections.OrderedDict()
_STREAM_WS_MAX = 4


_ADVISED = {}


def _stream_advised(lib, device_index, *shape) -> bool:
    """fa_fwd_stream_advised for one device and call shape, asked once (a
    ctypes call costs about a microsecond on every attention() call)."""
    key = (device_index,) + shape
    r = _ADVISED.get(key)
    if r is None:
        r = bool(lib.fa_fwd_stream_advised(*shape))
        if len(_ADVISED) < 4096:
            _ADVISED[key] = r
    return r


def _stream_workspace(device, stream, nbytes):
    """The stream form's workspace for (device, stream), or None when none
    large enough exists and the current stream is being captured into a
    graph (memory allocated there would belong to the graph's private pool
    and outlive nothing but the graph)."""
    import torch

    key = (device.index, stream)
    ws = _STREAM_WS.get(key)
    if ws is not None and ws.numel() >= nbytes:
        _STREAM_WS.move_to_end(key)
        return ws
    if torch.cuda.is_current_stream_capturing():
        return None
    # Freed memory goes back to torch's caching allocator on the stream it was
    # allocated on, which is the stream that used it, so reuse stays ordered
    # after the kernels that read it.
    _STREAM_WS.pop(key, None)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=device)
    _STREAM_WS[key] = ws
    while len(_STREAM_WS) > _STREAM_WS_MAX:
        _STREAM_WS.popitem(last=False)
    return ws


def release_workspaces() -> None:
    """Drop every cached workspace of the stream form (they are re-created,
    outside graph capture, on the next call that needs one)."""
    _STREAM_WS.clear()


class FaError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"libfa call failed with status {status}: {msg}")
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


def fa_fwd_strided(q: int, k: int, v: int, o: int, lse: Optional[int], B: int, H: int, Nq: int,
                   Nk: int, d: int, strides, scale: float, causal: int, dtype: int,
                   stream: int) -> int:
    """fa_fwd on tensors in any layout with contiguous d: `strides` is 12 element
    strides (q, k, v, o; each batch, head, row); returns the status."""
    arr = None if strides is None else (ctypes.c_int64 * 12)(*strides)
    return _lib.load().fa_fwd_strided(q, k, v, o, lse or None, B, H, Nq, Nk, d,
                                      None if arr is None else ctypes.cast(arr, ctypes.c_void_p),
                                      float(scale), int(causal), int(dtype), stream or None)


def fa_bwd_workspace_bytes(B: int, H: int, Nq: int) -> int:
    """Workspace bytes fa_bwd needs (-1 for invalid sizes)."""
    return _lib.load().fa_bwd_workspace_bytes(B, H, Nq)


def fa_bwd(q: int, k: int, v: int, o: int, dout: int, lse: int, dq: int, dk: int, dv: int,
           workspace: int, workspace_bytes: int, B: int, H: int, Nq: int, Nk: int, d: int,
           scale: float, causal: int, dtype: int, stream: int) -> int:
    """Direct call of the backward C entry point with raw device addresses;
    returns the status."""
    return _lib.load().fa_bwd(q or None, k or None, v or None, o or None, dout or None,
                              lse or None, dq or None, dk or None, dv or None,
                              workspace or None, workspace_bytes, B, H, Nq, Nk, d,
                              float(scale), int(causal), int(dtype), stream or None)


def fa_bwd_ex(q: int, k: int, v: int, o: int, dout: int, lse: int, dq: int, dk: int, dv: int,
              workspace: int, workspace_bytes: int, B: int, H: int, Nq: int, Nk: int, d: int,
              scale: float, causal: int, dtype: int, kernels: int, stream: int) -> int:
    """fa_bwd enqueuing only the kernels in the FA_BWD_* mask; returns the status."""
    return _lib.load().fa_bwd_ex(q or None, k or None, v or None, o or None, dout or None,
                                 lse or None, dq or None, dk or None, dv or None,
                                 workspace or None, workspace_bytes, B, H, Nq, Nk, d,
                                 float(scale), int(causal), int(dtype), int(kernels), stream or None)


def fa_bwd_noalloc(q: int, k: int, v: int, o: int, dout: int, lse: int, dq: int, dk: int,
                   dv: int, B: int, H: int, Nq: int, Nk: int, d: int, scale: float, causal: int,
                   dtype: int, stream: int) -> int:
    """Direct call of the backward entry point that allocates nothing (its
    D/LSE records live in the library's static scratch); returns the status."""
    return _lib.load().fa_bwd_noalloc(q or None, k or None, v or None, o or None, dout or None,
                                      lse or None, dq or None, dk or None, dv or None, B, H, Nq,
                                      Nk, d, float(scale), int(causal), int(dtype), stream or None)


def _current_stream(device_index: int):
    """Raw handle of the current stream of a device (None: the null stream).

    torch's private raw getter costs ~0.1 µs against ~3 µs for building a
    Stream object through the public API, which dominates short calls; the
    public API is the fallback."""
    import torch

    raw = getattr(torch._C, "_cuda_getCurrentRawStream", None)
    h = raw(device_index) if raw is not None else torch.cuda.current_stream(device_index).cuda_stream
    return h or None


def _current_device() -> int:
    """Index of the current device (torch's raw getter; the public
    torch.cuda.current_device adds a lazy-initialisation check per call)."""
    import torch

    raw = getattr(torch._C, "_cuda_getDevice", None)
    return raw() if raw is not None else torch.cuda.current_device()


def _dtype_code(t) -> int:
    import torch

    if t.dtype == torch.float16:
        return FA_DTYPE_FP16
    if t.dtype == torch.bfloat16:
        return FA_DTYPE_BF16
    raise TypeError(f"unsupported dtype {t.dtype}: fp16 or bf16 expected")


def _layout_strides(t, name):
    """(batch, head, row) element strides of a [B, H, N, d] GPU tensor whose
    last dimension is contiguous."""
    if t.dim() != 4 or t.stride(3) != 1:
        raise ValueError(f"{name} must be a [B, H, N, d] tensor with contiguous d")
    return [t.stride(0), t.stride(1), t.stride(2)]


def attention(q, k, v, *, causal: bool = False, scale: Optional[float] = None,
              out=None, lse=None, return_lse: bool = True, path: str = "auto"):
    """O = softmax(scale * Q K^T [causal mask]) V on the GPU, plus LSE.

    q: [B, H, Nq, d], k and v: [B, H, Nk, d], fp16/bf16 CUDA (HIP) tensors
    on one device. Contiguous tensors go through fa_fwd_ex; any other layout
    with a contiguous last dimension (e.g. [B, N, H, d] transposed to
    [B, H, N, d], or views of a fused [B, N, 3, H, d] projection) through
    fa_fwd_strided, read in place. scale=None means 1/sqrt(d). Returns (out,
    lse) with lse [B, H, Nq] float32, or (out, None) when return_lse is
    False; out gets q's layout when q is dense, else is contiguous. The work
    is enqueued on the current stream of q's device. path selects the kernel
    ("auto", "tiled" or "short"; see fa_path in include/fa.h) and is only
    available for contiguous tensors.
    """
    import torch

    # Device indices (get_device) rather than torch.device objects, and one
    # pass over the inputs: at N = 400 the host cost of this wrapper is
    # comparable to the kernel's.
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not isinstance(t, torch.Tensor) or not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor")
        if t.dim() != 4:
            raise ValueError(f"{name} must be a [B, H, N, d] tensor")
    dev = q.get_device()
    if k.get_device() != dev or v.get_device() != dev:
        raise ValueError("q, k, v must be on one device")
    dt = q.dtype
    if k.dtype != dt or v.dtype != dt:
        raise ValueError("q, k, v must share a dtype")
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    if k.shape != (B, H, Nk, d) or v.shape != (B, H, Nk, d):
        raise ValueError("k and v must be [B, H, Nk, d] matching q")
    code = _dtype_code(q)
    if path not in _PATHS:
        raise ValueError(f"path must be one of {sorted(_PATHS)}")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)  # q's strides when q is dense, else contiguous
    elif out.shape != q.shape or out.dtype != dt or out.get_device() != dev:
        raise ValueError("out must be a tensor like q")
    if lse is None and return_lse:
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    elif lse is not None and (lse.shape != (B, H, Nq) or lse.dtype != torch.float32
                              or lse.get_device() != dev or not lse.is_contiguous()):
        raise ValueError("lse must be a contiguous float32 [B, H, Nq] tensor")
    lib = _lib.load()
    contiguous = q.is_contiguous() and k.is_contiguous() and v.is_contiguous() and out.is_contiguous()
    ptrs = (q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
            lse.data_ptr() if lse is not None else None, B, H, Nq, Nk, d)
    c = 1 if causal else 0
    use_stream = contiguous and (path == "stream" or (
        path == "auto" and _stream_advised(lib, dev, B, H, Nq, Nk, d, code, c)))
    if use_stream:
        st_handle = _current_stream(dev)
        nbytes = lib.fa_fwd_stream_workspace_bytes(B, H, Nq, Nk, d, code)
        if nbytes < 0:
            raise FaError(_lib.FA_ERR_LAUNCH, "stream form unavailable on this device")
        ws = _stream_workspace(q.device, st_handle, nbytes)
        if ws is None:
            if path == "stream":
                raise FaError(_lib.FA_ERR_WORKSPACE,
                              "the stream form's workspace is not allocated during graph capture: "
                              "call attention(..., path='stream') once on this stream before capturing")
            use_stream = False  # the automatic choice takes the tiled kernel instead
        else:
            fn, call = lib.fa_fwd_stream, ptrs + (float(scale), c, code, ws.data_ptr(), ws.numel())
    if not use_stream and contiguous:
        fn, call = lib.fa_fwd_ex, ptrs + (float(scale), c, code, _PATHS[path])
    elif not use_stream:
        if path != "auto":
            raise ValueError("path applies to contiguous tensors only")
        strides = (_layout_strides(q, "q") + _layout_strides(k, "k") + _layout_strides(v, "v")
                   + _layout_strides(out, "out"))
        arr = (ctypes.c_int64 * 12)(*strides)
        fn, call = lib.fa_fwd_strided, ptrs + (ctypes.cast(arr, ctypes.c_void_p), float(scale), c,
                                               code)
    # The launch goes to the current device; switch only when q lives elsewhere
    # (the device guard costs several microseconds per call).
    if dev == _current_device():
        st = fn(*call, _current_stream(dev))
    else:
        with torch.cuda.device(dev):
            st = fn(*call, _current_stream(dev))
    _check(st)
    return out, lse


def attention_fp8(q, k, v, q_descale: float, k_descale: float, v_descale: float, *,
                  causal: bool = False, scale: Optional[float] = None, out_dtype=None,
                  out=None, lse=None, return_lse: bool = True):
    """Attention on FP8 (e4m3) q, k, v with per-tensor dequantisation factors.

    q: [B, H, Nq, d], k and v: [B, H, Nk, d], contiguous torch.float8_e4m3fn
    GPU tensors, d = 32, 64 or 128; element x of q means q_descale * x (likewise
    k, v). Returns (out, lse): out [B, H, Nq, d] in out_dtype (torch.bfloat16
    by default, or torch.float16), lse [B, H, Nq] float32 (None when
    return_lse is False). scale=None means 1/sqrt(d).
    """
    import torch

    for name, t in (("q", q), ("k", k), ("v", v)):
        if not isinstance(t, torch.Tensor) or not t.is_cuda or t.dtype != torch.float8_e4m3fn:
            raise ValueError(f"{name} must be a float8_e4m3fn GPU tensor")
        if t.dim() != 4 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous [B, H, N, d] tensor")
    if not (q.device == k.device == v.device):
        raise ValueError("q, k, v must be on one device")
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    if tuple(k.shape) != (B, H, Nk, d) or tuple(v.shape) != (B, H, Nk, d):
        raise ValueError("k and v must be [B, H, Nk, d] matching q")
    if out_dtype is None:
        out_dtype = out.dtype if out is not None else torch.bfloat16
    code = {torch.float16: FA_DTYPE_FP16, torch.bfloat16: FA_DTYPE_BF16}.get(out_dtype)
    if code is None:
        raise TypeError("out_dtype must be torch.float16 or torch.bfloat16")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty((B, H, Nq, d), dtype=out_dtype, device=q.device)
    elif (tuple(out.shape) != (B, H, Nq, d) or out.dtype != out_dtype or out.device != q.device
          or not out.is_contiguous()):
        raise ValueError("out must be a contiguous [B, H, Nq, d] tensor of out_dtype")
    if lse is None and return_lse:
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    elif lse is not None and (tuple(lse.shape) != (B, H, Nq) or lse.dtype != torch.float32
                              or lse.device != q.device or not lse.is_contiguous()):
        raise ValueError("lse must be a contiguous float32 [B, H, Nq] tensor")
    lib = _lib.load()
    call = (q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
            lse.data_ptr() if lse is not None else None, B, H, Nq, Nk, d, float(scale),
            float(q_descale), float(k_descale), float(v_descale), 1 if causal else 0, code)
    idx = q.device.index
    if idx == torch.cuda.current_device():
        st = lib.fa_fwd_fp8(*call, _current_stream(idx))
    else:
        with torch.cuda.device(q.device):
            st = lib.fa_fwd_fp8(*call, _current_stream(idx))
    _check(st)
    return out, lse


def fa_std_fwd(q: int, k: int, v: int, o: int, lse: Optional[int], s: int, p: int, B: int, H: int,
               Nq: int, Nk: int, d: int, scale: float, causal: int, dtype: int, stream: int) -> int:
    """Direct call of the standard-attention entry point; returns the status."""
    return _lib.load().fa_std_fwd(q or None, k or None, v or None, o or None, lse or None, s or None,
                                  p or None, B, H, Nq, Nk, d, float(scale), int(causal), int(dtype),
                                  stream or None)


def standard_attention(q, k, v, *, causal: bool = False, scale: Optional[float] = None,
                       return_intermediates: bool = False):
    """Attention computed the standard way (the baseline of the fused forward):
    S = scale Q K^T and P = softmax(S) are materialised in device memory
    between three kernels. q, k, v as in attention() (contiguous). Returns
    (out, lse), or (out, lse, s, p) with return_intermediates: s [B, H, Nq,
    NkP] float32 and p [B, H, Nq, NkP] in q's dtype, NkP = Nk rounded up to
    a multiple of 64 (columns past Nk: s unwritten, p zero)."""
    import torch

    _check_gpu_4d(q=q, k=k, v=v)
    if not (q.device == k.device == v.device) or not (q.dtype == k.dtype == v.dtype):
        raise ValueError("q, k, v must share a device and a dtype")
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    if tuple(k.shape) != (B, H, Nk, d) or tuple(v.shape) != (B, H, Nk, d):
        raise ValueError("k and v must be [B, H, Nk, d] matching q")
    code = _dtype_code(q)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    lib = _lib.load()
    nkp = lib.fa_std_row_stride(Nk)
    if nkp < 0:
        raise ValueError("Nk out of range")
    out = torch.empty_like(q)
    lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    s = torch.empty((B, H, Nq, nkp), dtype=torch.float32, device=q.device)
    p = torch.empty((B, H, Nq, nkp), dtype=q.dtype, device=q.device)
    idx = q.device.index
    call = (q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(), s.data_ptr(),
            p.data_ptr(), B, H, Nq, Nk, d, float(scale), 1 if causal else 0, code)
    if idx == torch.cuda.current_device():
        st = lib.fa_std_fwd(*call, _current_stream(idx))
    else:
        with torch.cuda.device(q.device):
            st = lib.fa_std_fwd(*call, _current_stream(idx))
    _check(st)
    return (out, lse, s, p) if return_intermediates else (out, lse)


def _check(st: int):
    if st != FA_OK:
        msg = status_str(st)
        if st == _lib.FA_ERR_LAUNCH:
            msg += ": " + _lib.load().fa_last_launch_error().decode()
        raise FaError(st, msg)


def _check_gpu_4d(**tensors):
    import torch

    for name, t in tensors.items():
        if not isinstance(t, torch.Tensor) or not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor")
        if t.dim() != 4 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous [B, H, N, d] tensor")


def attention_backward(q, k, v, out, dout, lse, *, causal: bool = False,
                       scale: Optional[float] = None, dq=None, dk=None, dv=None):
    """Gradients (dq, dk, dv) of attention for upstream gradient dout.

    q, k, v, causal and scale are those of the forward call; out and lse are
    its results (lse [B, H, Nq] float32). dout is shaped like q. All tensors
    are contiguous GPU tensors on one device, q/k/v/out/dout in one fp16 or
    bf16 dtype. Gradients come back in that dtype; dq/dk/dv may be passed to
    write into existing tensors. The workspace is allocated here (torch's
    caching allocator) and released when the call returns; the kernels run on
    the current stream, which keeps it alive until they finish.
    """
    import torch

    _check_gpu_4d(q=q, k=k, v=v, out=out, dout=dout)
    if not (q.device == k.device == v.device == out.device == dout.device == lse.device):
        raise ValueError("all tensors must be on one device")
    if not (q.dtype == k.dtype == v.dtype == out.dtype == dout.dtype):
        raise ValueError("q, k, v, out, dout must share a dtype")
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    if tuple(k.shape) != (B, H, Nk, d) or tuple(v.shape) != (B, H, Nk, d):
        raise ValueError("k and v must be [B, H, Nk, d] matching q")
    if out.shape != q.shape or dout.shape != q.shape:
        raise ValueError("out and dout must be shaped like q")
    if (tuple(lse.shape) != (B, H, Nq) or lse.dtype != torch.float32 or not lse.is_contiguous()):
        raise ValueError("lse must be a contiguous float32 [B, H, Nq] tensor")
    code = _dtype_code(q)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    grads = []
    for name, g, like in (("dq", dq, q), ("dk", dk, k), ("dv", dv, v)):
        if g is None:
            g = torch.empty_like(like)
        elif (g.shape != like.shape or g.dtype != like.dtype or g.device != like.device
              or not g.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous tensor like {'q' if name == 'dq' else name[1]}")
        grads.append(g)
    dq, dk, dv = grads
    lib = _lib.load()
    ws_bytes = lib.fa_bwd_workspace_bytes(B, H, Nq)
    if ws_bytes < 0:
        raise ValueError("sizes out of range for the backward pass")
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device)
    call = (q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), dout.data_ptr(),
            lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), ws.data_ptr(), ws_bytes,
            B, H, Nq, Nk, d, float(scale), 1 if causal else 0, code)
    idx = q.device.index
    if idx == torch.cuda.current_device():
        st = lib.fa_bwd(*call, _current_stream(idx))
    else:
        with torch.cuda.device(q.device):
            st = lib.fa_bwd(*call, _current_stream(idx))
    _check(st)
    return dq, dk, dv


def _autograd_function():
    import torch

    class FlashAttention(torch.autograd.Function):
        """Forward through fa_fwd (keeping O and LSE), backward through fa_bwd."""

        @staticmethod
        def forward(ctx, q, k, v, causal, scale):
            q, k, v = q.contiguous(), k.contiguous(), v.contiguous()
            o, lse = attention(q, k, v, causal=causal, scale=scale)
            ctx.save_for_backward(q, k, v, o, lse)
            ctx.causal, ctx.scale = causal, scale
            return o

        @staticmethod
        def backward(ctx, do):
            q, k, v, o, lse = ctx.saved_tensors
            dq, dk, dv = attention_backward(q, k, v, o, do.contiguous(), lse,
                                            causal=ctx.causal, scale=ctx.scale)
            return dq, dk, dv, None, None

    return FlashAttention


_FLASH_FN = None


def flash_attention(q, k, v, *, causal: bool = False, scale: Optional[float] = None):
    """Differentiable attention: O = softmax(scale * Q K^T [causal]) V, with
    the gradients of Q, K and V computed by the backward kernels."""
    global _FLASH_FN
    if _FLASH_FN is None:
        _FLASH_FN = _autograd_function()
    return _FLASH_FN.apply(q, k, v, causal, scale)
