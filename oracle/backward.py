"""Gradients of exact attention, written out from the definition, in float64
on the CPU.

TEST INFRASTRUCTURE ONLY (see the package docstring): no product code may
import this module.

What is computed, and where the cited articles state it:
  * Training runs a backward pass through the attention, for which the
    forward keeps its softmax statistics (kwkr.cn YOLO11 FlashAttention-2
    article, section 2.3), and that backward recomputes the softmax instead of
    storing it ("YOLOv12推理速度翻倍秘诀：Flash Attention加持", section 1, on
    numerically stable recomputation). The articles give no formulas for it; the
    plainest reading is the gradient of the forward definition (see
    definition.py) with respect to Q, K and V, for a given upstream gradient
    dO of the output, i.e. the vector-Jacobian product of
    O = softmax(scale * Q K^T [causal mask]) V.
  * Written out by the chain rule for one head, with P the row softmax:
        dV = P^T dO
        dP = dO V^T
        D_i = sum_j P_ij dP_ij           (the row-wise Jacobian of softmax)
        dS = P * (dP - D[:, None])       (masked entries have P = 0, so dS = 0)
        dQ = scale * dS K
        dK = scale * dS^T Q
    Nothing is tiled, recomputed or taken from saved statistics here: S and P
    are materialised in full rows from Q, K and V.
"""
from __future__ import annotations

import math
from typing import Optional, Tuple

import numpy as np

from .definition import apply_causal_mask, scores, softmax_stats, to_f64, _check_head_shapes


def attention_backward_head(q_h, k_h, v_h, do_h, scale: float, causal: bool = False,
                            row_ids: Optional[np.ndarray] = None
                            ) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """dQ [Nq, d], dK [Nk, d], dV [Nk, d] of one head for upstream gradient
    do_h [Nq, d]. row_ids: absolute query index of each row (causal mask)."""
    q_h, k_h, v_h, do_h = to_f64(q_h), to_f64(k_h), to_f64(v_h), to_f64(do_h)
    _check_head_shapes(q_h, k_h, v_h)
    if do_h.shape != q_h.shape:
        raise ValueError("dO must have the shape of Q")
    S = scores(q_h, k_h, scale)
    if causal:
        if row_ids is None:
            row_ids = np.arange(q_h.shape[0])
        S = apply_causal_mask(S, np.asarray(row_ids))
    E, _, l = softmax_stats(S)
    P = E / l[:, None]
    dV = P.T @ do_h
    dP = do_h @ v_h.T
    D = (P * dP).sum(axis=1)
    dS = P * (dP - D[:, None])
    dQ = scale * (dS @ k_h)
    dK = scale * (dS.T @ q_h)
    return dQ, dK, dV


def attention_backward(q, k, v, do, scale: Optional[float] = None, causal: bool = False
                       ) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """dQ, dK, dV over [B, H, N, d] tensors (float64), for upstream gradient do
    of the output of definition.attention with the same arguments."""
    q, k, v, do = to_f64(q), to_f64(k), to_f64(v), to_f64(do)
    if q.ndim != 4 or k.ndim != 4 or v.ndim != 4 or do.shape != q.shape:
        raise ValueError("expected [B, H, N, d] inputs with dO shaped like Q")
    B, H, Nq, d = q.shape
    if k.shape[:2] != (B, H) or v.shape != k.shape or k.shape[3] != d:
        raise ValueError("shape mismatch between q, k, v")
    if min(B, H, Nq, k.shape[2], d) < 1:
        raise ValueError("empty input")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dQ = np.empty_like(q)
    dK = np.empty_like(k)
    dV = np.empty_like(v)
    for b in range(B):
        for h in range(H):
            dQ[b, h], dK[b, h], dV[b, h] = attention_backward_head(
                q[b, h], k[b, h], v[b, h], do[b, h], scale, causal)
    return dQ, dK, dV


def row_delta(o, do) -> np.ndarray:
    """D_i = sum_d dO_id O_id per query row ([B, H, Nq] float64). Equal to
    sum_j P_ij dP_ij of attention_backward_head, since O_i = sum_j P_ij V_j."""
    return (to_f64(o) * to_f64(do)).sum(axis=-1)


def attention_backward_sampled(q_h, k_h, v_h, do_h, scale: float, causal: bool = False,
                               rows=(), keys=(), row_block: int = 1024):
    """dQ for selected query rows and dK, dV for selected keys of one head,
    for heads too long to hold S whole.

    The same chain rule as attention_backward_head, with the query rows taken
    row_block at a time: each row's P, dP and D depend on that row alone, so
    dQ of a row comes from its own block, and dK_j, dV_j (sums over all rows
    i) are accumulated block by block. Returns (dQ [len(rows), d],
    dK [len(keys), d], dV [len(keys), d])."""
    q_h, k_h, v_h, do_h = to_f64(q_h), to_f64(k_h), to_f64(v_h), to_f64(do_h)
    _check_head_shapes(q_h, k_h, v_h)
    rows = np.asarray(rows, dtype=np.int64)
    keys = np.asarray(keys, dtype=np.int64)
    Nq, d = q_h.shape
    dQ = np.zeros((len(rows), d))
    dK = np.zeros((len(keys), d))
    dV = np.zeros((len(keys), d))
    for r0 in range(0, Nq, row_block):
        r1 = min(Nq, r0 + row_block)
        S = scores(q_h[r0:r1], k_h, scale)
        if causal:
            S = apply_causal_mask(S, np.arange(r0, r1))
        E, _, l = softmax_stats(S)
        P = E / l[:, None]
        dP = do_h[r0:r1] @ v_h.T
        D = (P * dP).sum(axis=1)
        dS = P * (dP - D[:, None])
        dV += P[:, keys].T @ do_h[r0:r1]
        dK += scale * (dS[:, keys].T @ q_h[r0:r1])
        sel = (rows >= r0) & (rows < r1)
        if sel.any():
            dQ[sel] = scale * (dS[rows[sel] - r0] @ k_h)
    return dQ, dK, dV
