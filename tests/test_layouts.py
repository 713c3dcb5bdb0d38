"""Parity of the strided forward (fa_fwd_strided) with the fp64 oracle.

Inputs are drawn contiguous [B, H, N, d], copied into the layout under test
(sequence-major [B, N, H, d], a fused [B, N, 3, H, d] projection output, or
padded rows), and passed as [B, H, N, d] views; the oracle sees the original
contiguous tensors. Outputs are compared element by element, and padding
around strided outputs must be left untouched.
"""
import pytest
import torch

import exact_attention_23_amd as fa
import oracle
from tests.gpu_util import compare, default_scale, note, rand_inputs, require_gpu

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def bnhd_view(t):
    """[B, H, N, d] -> a [B, H, N, d] view of a sequence-major [B, N, H, d] copy."""
    return t.transpose(1, 2).contiguous().to(DEV).transpose(1, 2)


def fused_views(q, k, v):
    """q, k, v as views of one [B, N, 3, H, d] buffer."""
    qkv = torch.stack([t.transpose(1, 2) for t in (q, k, v)], dim=2).contiguous().to(DEV)
    return tuple(qkv[:, :, i].transpose(1, 2) for i in range(3)), qkv


def padded_rows(t, pad):
    """[B, H, N, d] view whose rows are d + pad elements apart (pad filled with a sentinel)."""
    B, H, N, d = t.shape
    buf = torch.full((B, H, N, d + pad), -7.0, dtype=t.dtype).to(DEV)
    buf[..., :d] = t.to(DEV)
    return buf[..., :d], buf


CASES = [
    # (B, H, Nq, Nk, d, dtype, causal)
    (1, 2, 361, 361, 64, "fp16", False),     # short path (few workgroups)
    (2, 3, 400, 400, 32, "bf16", True),
    (4, 8, 1000, 1000, 64, "fp16", True),    # tiled path
    (2, 4, 515, 515, 128, "bf16", False),
    (3, 4, 700, 700, 32, "fp16", False),
]


def _ids(c):
    return "B%dH%d_q%dk%d_d%d_%s_%s" % (c[0], c[1], c[2], c[3], c[4], c[5], "causal" if c[6] else "full")


@pytest.mark.parametrize("case", CASES, ids=_ids)
def test_sequence_major_inputs_and_output(case):
    require_gpu()
    B, H, Nq, Nk, d, dt, causal = case
    note(f"layout [B,N,H,d] {case}")
    q, k, v = rand_inputs(B, H, Nq, Nk, d, dt, seed=Nq + 17 * d)
    qv, kv, vv = bnhd_view(q), bnhd_view(k), bnhd_view(v)
    assert not qv.is_contiguous()
    o, lse = fa.attention(qv, kv, vv, causal=causal)
    assert o.stride() == qv.stride()  # the output takes q's sequence-major layout
    torch.cuda.synchronize()
    O, L = oracle.attention(q, k, v, scale=default_scale(d), causal=causal)
    compare(o.cpu(), lse.cpu(), O, L, what=f"[B,N,H,d] {case}")


@pytest.mark.parametrize("case", [c for c in CASES if c[2] == c[3]], ids=_ids)
def test_fused_qkv_views(case):
    require_gpu()
    B, H, N, _, d, dt, causal = case
    note(f"layout fused qkv {case}")
    q, k, v = rand_inputs(B, H, N, N, d, dt, seed=N + 31 * d)
    (qv, kv, vv), qkv = fused_views(q, k, v)
    before = qkv.clone()
    o_bnhd = torch.empty((B, N, H, d), dtype=q.dtype, device=DEV)
    o, lse = fa.attention(qv, kv, vv, causal=causal, out=o_bnhd.transpose(1, 2))
    torch.cuda.synchronize()
    assert torch.equal(qkv, before), "the fused input buffer was written"
    O, L = oracle.attention(q, k, v, scale=default_scale(d), causal=causal)
    compare(o_bnhd.transpose(1, 2).cpu(), lse.cpu(), O, L, what=f"fused qkv {case}")


def test_padded_rows_and_mixed_layouts():
    """q contiguous, k sequence-major, v with padded rows, o with padded rows;
    Nq != Nk, causal; the padding of o keeps its sentinel."""
    require_gpu()
    note("layout mixed")
    for d, dt in ((64, "fp16"), (128, "bf16"), (32, "fp16")):
        q, k, v = rand_inputs(2, 3, 300, 520, d, dt, seed=d + 5)
        vv, _ = padded_rows(v, 24)
        ov, obuf = padded_rows(torch.zeros_like(q), 8)
        for causal in (False, True):
            o, lse = fa.attention(q.to(DEV), bnhd_view(k), vv, causal=causal, out=ov)
            torch.cuda.synchronize()
            assert bool((obuf[..., d:] == -7.0).all()), "padding of o was written"
            O, L = oracle.attention(q, k, v, scale=default_scale(d), causal=causal)
            compare(o.cpu(), lse.cpu(), O, L, what=f"mixed d={d} causal={causal}")


def test_strided_equals_contiguous_bitwise():
    """The same values in another layout give bit-identical results (the
    kernels read the same numbers in the same order)."""
    require_gpu()
    note("layout bitwise")
    q, k, v = rand_inputs(2, 4, 1000, 1000, 64, "fp16", seed=3)
    o1, l1 = fa.attention(q.to(DEV), k.to(DEV), v.to(DEV), causal=True)
    o2, l2 = fa.attention(bnhd_view(q), bnhd_view(k), bnhd_view(v), causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2.contiguous()) and torch.equal(l1, l2)
