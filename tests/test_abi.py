"""The C ABI of libfa.so, checked without a GPU.

Every argument check in fa_fwd and fa_bwd runs before any HIP call, so
invalid calls can be made here; no valid (launching) call is made.
"""
import ctypes
import os
import re

import pytest

import exact_attention_23_amd as fa
from exact_attention_23_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")


def _header_text():
    with open(HEADER, encoding="utf-8") as f:
        return f.read()


def _declared_functions():
    src = re.sub(r"/\*.*?\*/", "", _header_text(), flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(fa_\w+)\s*\(", src, flags=re.M)))


def test_library_exports_every_declared_symbol():
    lib = _lib.load()
    names = _declared_functions()
    assert "fa_fwd" in names and "fa_status_str" in names and "fa_version" in names
    for n in names:
        assert hasattr(lib, n), f"libfa.so does not export {n}"


def test_header_enums_match_binding():
    src = _header_text()
    for name in ["FA_OK", "FA_ERR_NULLPTR", "FA_ERR_SHAPE", "FA_ERR_HEADDIM", "FA_ERR_DTYPE",
                 "FA_ERR_SCALE", "FA_ERR_CAUSAL", "FA_ERR_ALIGN", "FA_ERR_ALIAS", "FA_ERR_LAUNCH",
                 "FA_ERR_PATH", "FA_DTYPE_FP16", "FA_DTYPE_BF16", "FA_PATH_AUTO", "FA_PATH_TILED",
                 "FA_PATH_SHORT", "FA_ERR_WORKSPACE", "FA_BWD_PRE", "FA_BWD_DKDV", "FA_BWD_DQ",
                 "FA_BWD_ALL"]:
        m = re.search(rf"\b{name}\s*=\s*(\d+)", src)
        assert m, name
        assert int(m.group(1)) == getattr(_lib, name), name


def test_status_strings():
    lib = _lib.load()
    for s in range(0, 12):
        txt = lib.fa_status_str(s)
        assert txt and txt.decode() != "unknown status"
    assert lib.fa_status_str(99).decode() == "unknown status"
    assert fa.version() >= 100


# Fake device addresses: never dereferenced, because each call below fails a
# check that precedes every HIP call.
Q, K, V, O, L = 0x10000000, 0x20000000, 0x30000000, 0x40000000, 0x50000000
GOOD = dict(q=Q, k=K, v=V, o=O, lse=L, B=2, H=3, Nq=100, Nk=77, d=64, scale=0.125,
            causal=0, dtype=0, stream=None)


def call(**kw):
    a = dict(GOOD)
    a.update(kw)
    return fa.fa_fwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["Nq"], a["Nk"],
                     a["d"], a["scale"], a["causal"], a["dtype"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(q=0), _lib.FA_ERR_NULLPTR),
    (dict(k=0), _lib.FA_ERR_NULLPTR),
    (dict(v=0), _lib.FA_ERR_NULLPTR),
    (dict(o=0), _lib.FA_ERR_NULLPTR),
    (dict(dtype=2), _lib.FA_ERR_DTYPE),
    (dict(dtype=-1), _lib.FA_ERR_DTYPE),
    (dict(d=16), _lib.FA_ERR_HEADDIM),
    (dict(d=96), _lib.FA_ERR_HEADDIM),
    (dict(d=256), _lib.FA_ERR_HEADDIM),
    (dict(B=0), _lib.FA_ERR_SHAPE),
    (dict(H=0), _lib.FA_ERR_SHAPE),
    (dict(Nq=0), _lib.FA_ERR_SHAPE),
    (dict(Nk=0), _lib.FA_ERR_SHAPE),
    (dict(Nq=-5), _lib.FA_ERR_SHAPE),
    (dict(Nk=(1 << 29) // 64), _lib.FA_ERR_SHAPE),
    (dict(Nq=(1 << 29) // 32, d=32), _lib.FA_ERR_SHAPE),
    (dict(B=1 << 20, H=1 << 12), _lib.FA_ERR_SHAPE),
    (dict(causal=2), _lib.FA_ERR_CAUSAL),
    (dict(causal=-1), _lib.FA_ERR_CAUSAL),
    (dict(scale=float("nan")), _lib.FA_ERR_SCALE),
    (dict(scale=float("inf")), _lib.FA_ERR_SCALE),
    (dict(scale=float("-inf")), _lib.FA_ERR_SCALE),
    (dict(q=Q + 8), _lib.FA_ERR_ALIGN),
    (dict(o=O + 2), _lib.FA_ERR_ALIGN),
    (dict(lse=L + 2), _lib.FA_ERR_ALIGN),
    (dict(o=Q), _lib.FA_ERR_ALIAS),
    (dict(o=K + 256), _lib.FA_ERR_ALIAS),
    (dict(lse=V + 64), _lib.FA_ERR_ALIAS),
    (dict(lse=O + 1024), _lib.FA_ERR_ALIAS),
])
def test_invalid_arguments_rejected_before_launch(kw, status):
    assert call(**kw) == status


def test_check_order_is_stable():
    # several faults at once: the first check in the documented order wins
    assert call(q=0, d=3, B=0) == _lib.FA_ERR_NULLPTR
    assert call(dtype=7, d=3) == _lib.FA_ERR_DTYPE
    assert call(d=3, B=0) == _lib.FA_ERR_HEADDIM


def call_ex(path, **kw):
    a = dict(GOOD)
    a.update(kw)
    return fa.fa_fwd_ex(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["Nq"],
                        a["Nk"], a["d"], a["scale"], a["causal"], a["dtype"], path, a["stream"])


@pytest.mark.parametrize("path,kw", [
    (3, {}),
    (-1, {}),
    (_lib.FA_PATH_SHORT, dict(Nk=1025, d=64)),      # 17 key tiles
    (_lib.FA_PATH_SHORT, dict(Nk=1025, d=32)),
    (_lib.FA_PATH_SHORT, dict(Nk=577, d=128)),      # 10 key tiles
])
def test_path_rejected_before_launch(path, kw):
    assert call_ex(path, **kw) == _lib.FA_ERR_PATH


def test_path_checked_after_the_other_arguments():
    assert call_ex(7, q=0) == _lib.FA_ERR_NULLPTR
    assert call_ex(7, d=48) == _lib.FA_ERR_HEADDIM
    assert call_ex(7, o=Q) == _lib.FA_ERR_ALIAS
    # the short path's key limit is reached exactly at 16 (d <= 64) and 9 (d = 128) tiles:
    # those sizes pass the path check and fail only on the fake pointers' later checks
    for path in (_lib.FA_PATH_AUTO, _lib.FA_PATH_TILED, _lib.FA_PATH_SHORT):
        assert call_ex(path, Nk=1024, d=64, q=0) == _lib.FA_ERR_NULLPTR
        assert call_ex(path, Nk=576, d=128, causal=5) == _lib.FA_ERR_CAUSAL


def test_python_wrapper_rejects_cpu_tensors():
    torch = pytest.importorskip("torch")
    q = torch.zeros(1, 1, 4, 64, dtype=torch.float16)
    with pytest.raises(ValueError):
        fa.attention(q, q, q)


def test_ctypes_signature():
    lib = _lib.load()
    assert lib.fa_fwd.restype is ctypes.c_int
    assert len(lib.fa_fwd.argtypes) == 14
    assert lib.fa_fwd_ex.restype is ctypes.c_int
    assert len(lib.fa_fwd_ex.argtypes) == 15


# ---- backward entry points
DO, DQ, DK, DV, WS = 0x60000000, 0x70000000, 0x80000000, 0x90000000, 0xA0000000
BGOOD = dict(q=Q, k=K, v=V, o=O, dout=DO, lse=L, dq=DQ, dk=DK, dv=DV, ws=WS, ws_bytes=1 << 20,
             B=2, H=3, Nq=100, Nk=77, d=64, scale=0.125, causal=0, dtype=0, stream=None)


def bcall(**kw):
    a = dict(BGOOD)
    a.update(kw)
    return fa.fa_bwd(a["q"], a["k"], a["v"], a["o"], a["dout"], a["lse"], a["dq"], a["dk"],
                     a["dv"], a["ws"], a["ws_bytes"], a["B"], a["H"], a["Nq"], a["Nk"], a["d"],
                     a["scale"], a["causal"], a["dtype"], a["stream"])


def test_workspace_size():
    # two fp32 values per query row, rows padded to 32
    assert fa.fa_bwd_workspace_bytes(2, 3, 100) == 2 * 3 * 4 * 256
    assert fa.fa_bwd_workspace_bytes(1, 1, 1) == 256
    assert fa.fa_bwd_workspace_bytes(1, 1, 32) == 256
    assert fa.fa_bwd_workspace_bytes(1, 1, 33) == 512
    assert fa.fa_bwd_workspace_bytes(0, 1, 1) == -1
    assert fa.fa_bwd_workspace_bytes(1, 0, 1) == -1
    assert fa.fa_bwd_workspace_bytes(1, 1, 0) == -1
    assert fa.fa_bwd_workspace_bytes(1 << 20, 1 << 12, 1) == -1
    assert fa.fa_bwd_workspace_bytes(1, 1, (1 << 29) + 1) == -1


@pytest.mark.parametrize("kw,status", [
    (dict(q=0), _lib.FA_ERR_NULLPTR),
    (dict(o=0), _lib.FA_ERR_NULLPTR),
    (dict(dout=0), _lib.FA_ERR_NULLPTR),
    (dict(lse=0), _lib.FA_ERR_NULLPTR),
    (dict(dq=0), _lib.FA_ERR_NULLPTR),
    (dict(dk=0), _lib.FA_ERR_NULLPTR),
    (dict(dv=0), _lib.FA_ERR_NULLPTR),
    (dict(dtype=2), _lib.FA_ERR_DTYPE),
    (dict(d=96), _lib.FA_ERR_HEADDIM),
    (dict(Nk=0), _lib.FA_ERR_SHAPE),
    (dict(Nq=(1 << 29) // 32, d=32), _lib.FA_ERR_SHAPE),
    (dict(causal=3), _lib.FA_ERR_CAUSAL),
    (dict(scale=float("nan")), _lib.FA_ERR_SCALE),
    (dict(dout=DO + 8), _lib.FA_ERR_ALIGN),
    (dict(dk=DK + 4), _lib.FA_ERR_ALIGN),
    (dict(lse=L + 1), _lib.FA_ERR_ALIGN),
    (dict(ws=0), _lib.FA_ERR_WORKSPACE),
    (dict(ws=WS + 8), _lib.FA_ERR_WORKSPACE),
    (dict(ws_bytes=2 * 3 * 4 * 256 - 1), _lib.FA_ERR_WORKSPACE),
    (dict(dq=Q), _lib.FA_ERR_ALIAS),
    (dict(dk=V + 512), _lib.FA_ERR_ALIAS),
    (dict(dv=DO), _lib.FA_ERR_ALIAS),
    (dict(dv=DK + 256), _lib.FA_ERR_ALIAS),
    (dict(ws=DQ + 1024), _lib.FA_ERR_ALIAS),
    (dict(ws=L), _lib.FA_ERR_ALIAS),
    (dict(dq=WS), _lib.FA_ERR_ALIAS),
])
def test_bwd_invalid_arguments_rejected_before_launch(kw, status):
    assert bcall(**kw) == status


def test_bwd_exact_workspace_is_enough_for_the_checks():
    # a workspace of exactly fa_bwd_workspace_bytes passes its check; the call
    # then fails a later check (an alias), so nothing is launched
    need = fa.fa_bwd_workspace_bytes(2, 3, 100)
    assert bcall(ws_bytes=need, dv=K) == _lib.FA_ERR_ALIAS


@pytest.mark.parametrize("mask", [0, -1, 8, 15])
def test_bwd_kernel_mask_rejected_before_launch(mask):
    a = dict(BGOOD)
    assert fa.fa_bwd_ex(a["q"], a["k"], a["v"], a["o"], a["dout"], a["lse"], a["dq"], a["dk"],
                        a["dv"], a["ws"], a["ws_bytes"], a["B"], a["H"], a["Nq"], a["Nk"], a["d"],
                        a["scale"], a["causal"], a["dtype"], mask, None) == _lib.FA_ERR_PATH
    # the other checks come first
    assert fa.fa_bwd_ex(0, a["k"], a["v"], a["o"], a["dout"], a["lse"], a["dq"], a["dk"],
                        a["dv"], a["ws"], a["ws_bytes"], a["B"], a["H"], a["Nq"], a["Nk"], a["d"],
                        a["scale"], a["causal"], a["dtype"], mask, None) == _lib.FA_ERR_NULLPTR


# ---- strided forward
def contiguous_strides(B, H, Nq, Nk, d):
    return [H * Nq * d, Nq * d, d, H * Nk * d, Nk * d, d, H * Nk * d, Nk * d, d, H * Nq * d, Nq * d, d]


def scall(strides, **kw):
    a = dict(GOOD)
    a.update(kw)
    return fa.fa_fwd_strided(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["Nq"],
                             a["Nk"], a["d"], strides, a["scale"], a["causal"], a["dtype"], a["stream"])


def _with(i, val):
    s = contiguous_strides(2, 3, 100, 77, 64)
    s[i] = val
    return s


@pytest.mark.parametrize("strides", [
    None,
    _with(2, 32),            # q rows closer than d
    _with(5, 68),            # k row stride not a multiple of 8
    _with(0, -64),           # negative batch stride
    _with(7, 4),             # v head stride not a multiple of 8
    _with(11, 1 << 30),      # o rows span too far for one head
    _with(10, 64),           # o heads overlap rows of another head
    _with(9, 0),             # o batches share memory
])
def test_strided_layouts_rejected(strides):
    assert scall(strides) == _lib.FA_ERR_STRIDE


def test_strided_checks_keep_their_order():
    assert scall(None, q=0) == _lib.FA_ERR_NULLPTR
    assert scall(_with(2, 32), d=96) == _lib.FA_ERR_HEADDIM
    assert scall(_with(2, 32), scale=float("nan")) == _lib.FA_ERR_SCALE


def test_strided_alias_uses_spans():
    # [B, N, H, d] o placed inside q's span, and q interleaved with o
    s = contiguous_strides(2, 3, 100, 77, 64)
    assert scall(s, o=Q + 4096) == _lib.FA_ERR_ALIAS
    # inputs may share memory (a fused QKV buffer): k and v inside q's span
    # pass the checks up to the alias test of o, which fails here on purpose
    fused = [100 * 3 * 3 * 64, 64, 3 * 3 * 64] * 3 + [100 * 3 * 64, 64, 3 * 64]
    assert scall(fused, B=2, H=3, Nq=100, Nk=100, k=Q + 3 * 64 * 2, v=Q + 6 * 64 * 2,
                 o=Q + 64) == _lib.FA_ERR_ALIAS


# ---- FP8 forward
FGOOD = dict(q=Q, k=K, v=V, o=O, lse=L, B=2, H=3, Nq=100, Nk=77, d=64, scale=0.125,
             qd=0.01, kd=0.02, vd=0.03, causal=0, out_dtype=1, stream=None)


def fcall(**kw):
    a = dict(FGOOD)
    a.update(kw)
    return _lib.load().fa_fwd_fp8(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["Nq"],
                                  a["Nk"], a["d"], a["scale"], a["qd"], a["kd"], a["vd"], a["causal"],
                                  a["out_dtype"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), _lib.FA_ERR_NULLPTR),
    (dict(o=None), _lib.FA_ERR_NULLPTR),
    (dict(out_dtype=2), _lib.FA_ERR_DTYPE),
    (dict(d=16), _lib.FA_ERR_HEADDIM),
    (dict(d=96), _lib.FA_ERR_HEADDIM),
    (dict(Nq=0), _lib.FA_ERR_SHAPE),
    (dict(causal=2), _lib.FA_ERR_CAUSAL),
    (dict(qd=0.0), _lib.FA_ERR_SCALE),
    (dict(kd=-1.0), _lib.FA_ERR_SCALE),
    (dict(vd=float("nan")), _lib.FA_ERR_SCALE),
    (dict(scale=float("inf")), _lib.FA_ERR_SCALE),
    (dict(scale=1e30, qd=1e30), _lib.FA_ERR_SCALE),
    (dict(k=K + 8), _lib.FA_ERR_ALIGN),
    (dict(lse=L + 1), _lib.FA_ERR_ALIGN),
    (dict(o=Q + 1024), _lib.FA_ERR_ALIAS),
    (dict(lse=O + 64), _lib.FA_ERR_ALIAS),
])
def test_fp8_invalid_arguments_rejected_before_launch(kw, status):
    assert fcall(**kw) == status


# ---- stream forward
def stcall(**kw):
    a = dict(GOOD)
    a.update(kw)
    ws = a.get("ws", WS)
    return _lib.load().fa_fwd_stream(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"],
                                     a["Nq"], a["Nk"], a["d"], a["scale"], a["causal"], a["dtype"],
                                     ws, a.get("ws_bytes", 1 << 30), a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(q=0), _lib.FA_ERR_NULLPTR),
    (dict(d=96), _lib.FA_ERR_HEADDIM),
    (dict(causal=1), _lib.FA_ERR_PATH),
    (dict(ws=0), _lib.FA_ERR_WORKSPACE),
    (dict(ws=WS + 4), _lib.FA_ERR_WORKSPACE),
    (dict(o=Q), _lib.FA_ERR_ALIAS),
])
def test_stream_invalid_arguments_rejected_before_launch(kw, status):
    assert stcall(**kw) == status


def test_stream_size_queries_reject_bad_sizes():
    lib = _lib.load()
    assert lib.fa_fwd_stream_workspace_bytes(0, 1, 1, 1, 64, 0) == -1
    assert lib.fa_fwd_stream_workspace_bytes(1, 1, 1, 1, 96, 0) == -1
    assert lib.fa_fwd_stream_workspace_bytes(1, 1, 1, 1, 64, 3) == -1
    assert lib.fa_fwd_stream_advised(16, 4, 6400, 6400, 32, 0, 1) == 0  # causal
    assert lib.fa_fwd_stream_advised(0, 4, 6400, 6400, 32, 0, 0) == 0


def ncall(**kw):
    """fa_bwd_noalloc with BGOOD's arguments (no workspace) overridden by kw."""
    a = dict(BGOOD)
    a.update(kw)
    return fa.fa_bwd_noalloc(a["q"], a["k"], a["v"], a["o"], a["dout"], a["lse"], a["dq"], a["dk"],
                             a["dv"], a["B"], a["H"], a["Nq"], a["Nk"], a["d"], a["scale"],
                             a["causal"], a["dtype"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(q=0), _lib.FA_ERR_NULLPTR),
    (dict(dv=0), _lib.FA_ERR_NULLPTR),
    (dict(lse=0), _lib.FA_ERR_NULLPTR),
    (dict(dtype=2), _lib.FA_ERR_DTYPE),
    (dict(d=96), _lib.FA_ERR_HEADDIM),
    (dict(Nq=0), _lib.FA_ERR_SHAPE),
    (dict(causal=2), _lib.FA_ERR_CAUSAL),
    (dict(scale=float("inf")), _lib.FA_ERR_SCALE),
    (dict(dq=DQ + 8), _lib.FA_ERR_ALIGN),
    # the static scratch holds 65536 records of 32 rows: one more is refused
    (dict(B=1, H=65537, Nq=32), _lib.FA_ERR_SCRATCH),
    (dict(B=2, H=1, Nq=32 * 32768 + 1), _lib.FA_ERR_SCRATCH),
    (dict(dq=Q), _lib.FA_ERR_ALIAS),
    (dict(dv=DK + 256), _lib.FA_ERR_ALIAS),
])
def test_noalloc_invalid_arguments_rejected_before_launch(kw, status):
    assert ncall(**kw) == status


def test_noalloc_scratch_limit_matches_header():
    assert _lib.FA_BWD_NOALLOC_SCRATCH_BYTES == 16 << 20
    assert re.search(r"#define FA_BWD_NOALLOC_SCRATCH_BYTES \(16LL << 20\)", _header_text())
    # the largest accepted size fits exactly; checked before any alias test
    assert fa.fa_bwd_workspace_bytes(1, 65536, 32) == _lib.FA_BWD_NOALLOC_SCRATCH_BYTES
    assert ncall(B=1, H=65536, Nq=32, dv=DK + 256) == _lib.FA_ERR_ALIAS


SS, PP = 0x7000000, 0x8000000  # stand-in device addresses of S and P


def stdcall(**kw):
    a = dict(q=Q, k=K, v=V, o=O, lse=L, s=SS, p=PP, B=2, H=3, Nq=100, Nk=77, d=64, scale=0.125,
             causal=0, dtype=0, stream=None)
    a.update(kw)
    return fa.fa_std_fwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["s"], a["p"], a["B"], a["H"],
                         a["Nq"], a["Nk"], a["d"], a["scale"], a["causal"], a["dtype"], a["stream"])


def test_std_row_stride():
    assert fa._lib.load().fa_std_row_stride(1) == 64
    assert fa._lib.load().fa_std_row_stride(64) == 64
    assert fa._lib.load().fa_std_row_stride(65) == 128
    assert fa._lib.load().fa_std_row_stride(0) == -1


@pytest.mark.parametrize("kw,status", [
    (dict(q=0), _lib.FA_ERR_NULLPTR),
    (dict(s=0), _lib.FA_ERR_NULLPTR),
    (dict(p=0), _lib.FA_ERR_NULLPTR),
    (dict(dtype=3), _lib.FA_ERR_DTYPE),
    (dict(d=16), _lib.FA_ERR_HEADDIM),
    (dict(Nk=0), _lib.FA_ERR_SHAPE),
    (dict(Nq=1 << 16, Nk=1 << 13), _lib.FA_ERR_SHAPE),  # Nq * NkP reaches 2^29
    (dict(causal=5), _lib.FA_ERR_CAUSAL),
    (dict(scale=float("nan")), _lib.FA_ERR_SCALE),
    (dict(s=SS + 4), _lib.FA_ERR_ALIGN),
    (dict(p=PP + 8), _lib.FA_ERR_ALIGN),
    (dict(s=Q), _lib.FA_ERR_ALIAS),
    (dict(p=O), _lib.FA_ERR_ALIAS),
    (dict(p=SS + 1024), _lib.FA_ERR_ALIAS),
    (dict(lse=PP), _lib.FA_ERR_ALIAS),
])
def test_std_invalid_arguments_rejected_before_launch(kw, status):
    assert stdcall(**kw) == status
