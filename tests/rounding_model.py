"""A CPU model of the forward kernels' rounding, for reasoning about tolerances.

This is not the oracle and not the product: it replays, in numpy, the order
in which the HIP forward rounds its intermediate values, so that a test can
say how far from the exact result a kernel with that arithmetic must land.
It shares no code with the HIP path (it reads none of its sources) and no
arithmetic with the oracle (it computes its own scores in float64 and rounds
them the kernel's way).

Modelled steps, per query row (the method of the kwkr.cn YOLO11
FlashAttention-2 article, section 1.2, and "FlashAttention 深度解读",
原理 2, with the kernel's own precision choices):
  * scores s_j = sum_c q_c k_c, rounded to fp32 (the matrix instruction
    accumulates in fp32; its internal order is not modelled);
  * the reference maximum m (exp2 domain, fp32): the largest visible score
    of the row's first 32 keys (head width 32, whose loop takes its
    reference from the first 32-key unit) or first 64 keys (64 and 128),
    times c = |scale| log2(e), as the tiled kernel takes it; the short-range
    kernel instead takes the exact maximum of every 64-key tile and merges the
    tiles at the end with weights 2^(m_w - M);
  * p_j = 2^(s_j c - m) in fp32 (one fused multiply-add, then exp2);
  * P rounded to the input type by round-to-nearest-even (the P operand of
    the P V product);
  * O_acc = sum_j round(p_j) v_j, rounded to fp32;
  * the normaliser l: either the fp32 sum of the unrounded p ("fp32") or the
    sum of the rounded P the product actually used ("rounded");
  * O = round_type(O_acc / l); LSE = ln2 (m + log2(sum of unrounded p)).
The reference maximum is never raised after the first tile: true for inputs
whose later scores stay within ~15 log2 units of the first tile's, which
holds for every case this model is applied to here.
"""
from __future__ import annotations

import math

import numpy as np
import torch

LOG2E = 1.4426950408889634


def _f32(x):
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def _round_type(x, dtype):
    t = torch.from_numpy(np.ascontiguousarray(np.asarray(x, dtype=np.float32)))
    return t.to(dtype).to(torch.float64).numpy()


def head_forward(q, k, v, scale, causal, dtype, norm="rounded", kernel="tiled"):
    """Modelled kernel output (O, LSE) of one head: q [Nq, d], k/v [Nk, d]
    float64 arrays holding values of `dtype` (torch.float16/bfloat16)."""
    Nq, d = q.shape
    Nk = k.shape[0]
    s = _f32(q @ k.T) * (1.0 if scale >= 0 else -1.0)  # a negative scale flips Q's sign bits
    if scale == 0.0:
        s = np.zeros_like(s)
    c = float(np.float32(abs(scale) * LOG2E)) if scale != 0.0 else 1.0
    vis = np.ones((Nq, Nk), dtype=bool)
    if causal:
        vis = np.arange(Nk)[None, :] <= np.arange(Nq)[:, None]
    s_m = np.where(vis, s, -np.inf)
    if kernel == "tiled":
        first = 32 if d == 32 else 64
        m = _f32(s_m[:, :first].max(axis=1) * np.float32(c))  # fp32 product
        tiles = [(0, Nk, m)]
    else:
        tiles = []
        for k0 in range(0, Nk, 64):
            mw = _f32(s_m[:, k0:k0 + 64].max(axis=1) * np.float32(c))
            tiles.append((k0, min(Nk, k0 + 64), mw))
    M = np.max(np.stack([t[2] for t in tiles]), axis=0)
    M0 = np.where(np.isfinite(M), M, 0.0)
    o_acc = np.zeros((Nq, d))
    l32 = np.zeros(Nq)
    lr = np.zeros(Nq)
    for k0, k1, mw in tiles:
        ok = np.isfinite(mw)
        ref = np.where(ok, mw, 0.0)
        t = _f32(s[:, k0:k1] * c - ref[:, None])
        p = np.where(vis[:, k0:k1], _f32(np.exp2(t)), 0.0)
        pr = _round_type(p, dtype)
        # merge weight of a tile (short-range kernel); 1 for the single range
        f = np.where(ok, _f32(np.exp2(ref - M0)), 0.0)
        o_acc += f[:, None] * _f32(pr @ v[k0:k1])
        l32 += f * _f32(p.sum(axis=1))
        lr += f * _f32(pr.sum(axis=1))
    ref_all = M0
    l = l32 if norm == "fp32" else lr
    O = _round_type(_f32(_f32(o_acc) * _f32(1.0 / _f32(l))[:, None]), dtype)
    lse = math.log(2.0) * (ref_all + np.log2(l32))
    return O, lse


def forward(q, k, v, scale, causal, norm="rounded", kernel="tiled"):
    """head_forward over [B, H, N, d] torch tensors; returns float64 arrays."""
    dtype = q.dtype
    qd, kd, vd = (t.to(torch.float64).numpy() for t in (q, k, v))
    B, H, Nq, d = q.shape
    O = np.empty((B, H, Nq, d))
    L = np.empty((B, H, Nq))
    for b in range(B):
        for h in range(H):
            O[b, h], L[b, h] = head_forward(qd[b, h], kd[b, h], vd[b, h], scale, causal, dtype,
                                            norm=norm, kernel=kernel)
    return O, L
