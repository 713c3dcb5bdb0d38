"""Exact attention written out as its definition, in float64 on the CPU.

TEST INFRASTRUCTURE ONLY (see the package docstring): no product code may
import this module.

What is computed, and where the cited articles state it:
  * O = softmax(Q K^T * scale) V, the three steps being the Q-K product, a row
    softmax, and the product with V ("FlashAttention 深度解读", section 背景,
    its attention formula; kwkr.cn YOLO11 FlashAttention-2 article, section
    1.1; ai2ai.xin flash-attention-principle page, section on the
    self-attention bottleneck, its five-step list).
  * scale defaults to 1/sqrt(head_dim) (kwkr.cn article, section 2.2, on the
    scale argument of scaled_dot_product_attention).
  * the tiled, online-softmax method equals this plain definition up to the
    order of floating-point rounding (kwkr.cn article, sections 1.2 and 1.3),
    so the oracle is the definition itself: S is materialised in full rows,
    the softmax is an explicit row softmax, nothing is tiled along keys.
  * causal=True masks key j for query i when j > i (the causal flag of the
    flash_attention call in "FlashAttention 深度解读", usage section; read as
    the top-left alignment of PyTorch's is_causal, which the kwkr.cn article
    calls in section 2.2). A masked score is exactly -inf, i.e. weight 0.
  * LSE_i = ln sum_j exp(S_ij) over unmasked keys, S already scaled: the
    softmax statistics (running max and running sum) that the kwkr.cn article,
    section 2.3, says training keeps for the backward pass, folded into one
    number per row.

Subtracting the row maximum before exp (the precision-handling paragraph of
"FlashAttention 深度解读") changes nothing in exact arithmetic; it is done here
only so float64 exp never overflows on large logits.
"""
from __future__ import annotations

import math
from typing import Optional, Sequence, Tuple

import numpy as np


def to_f64(x) -> np.ndarray:
    """Exact conversion of a torch tensor (fp16/bf16/fp8/fp32/...) or array to
    float64. (torch is imported only for torch tensors, so the oracle runs on
    numpy arrays with numpy alone.)"""
    if type(x).__module__.split(".")[0] == "torch":
        import torch

        return x.detach().to("cpu", torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def scores(q_h: np.ndarray, k_h: np.ndarray, scale: float) -> np.ndarray:
    """S = scale * Q K^T for one head: q_h [Nq, d], k_h [Nk, d] -> [Nq, Nk]."""
    return scale * (q_h @ k_h.T)


def apply_causal_mask(S: np.ndarray, row_ids: np.ndarray) -> np.ndarray:
    """Set S[r, j] = -inf where key j lies after query row_ids[r] (j > i)."""
    cols = np.arange(S.shape[1])
    masked = cols[None, :] > row_ids[:, None]
    out = S.copy()
    out[masked] = -np.inf
    return out


def softmax_stats(S: np.ndarray):
    """Explicit full-row softmax pieces: m_i = max_j S_ij, P_ij = exp(S_ij - m_i),
    l_i = sum_j P_ij. Returns (P, m, l); P/l[:, None] is the softmax."""
    m = S.max(axis=1)
    P = np.exp(S - m[:, None])
    l = P.sum(axis=1)
    return P, m, l


def _check_head_shapes(q_h, k_h, v_h):
    if q_h.ndim != 2 or k_h.ndim != 2 or v_h.ndim != 2:
        raise ValueError("per-head inputs must be 2-D")
    if q_h.shape[1] != k_h.shape[1] or k_h.shape[0] != v_h.shape[0]:
        raise ValueError("shape mismatch between q, k, v")
    if q_h.shape[0] < 1 or k_h.shape[0] < 1:
        raise ValueError("empty sequence")


def probabilities(q_h, k_h, scale: float, causal: bool = False,
                  row_ids: Optional[np.ndarray] = None) -> np.ndarray:
    """The normalised attention weights softmax(S) for one head, [Nq, Nk]."""
    q_h, k_h = to_f64(q_h), to_f64(k_h)
    S = scores(q_h, k_h, scale)
    if causal:
        if row_ids is None:
            row_ids = np.arange(q_h.shape[0])
        S = apply_causal_mask(S, np.asarray(row_ids))
    P, _, l = softmax_stats(S)
    return P / l[:, None]


def attention_head(q_h, k_h, v_h, scale: float, causal: bool = False,
                   row_ids: Optional[np.ndarray] = None) -> Tuple[np.ndarray, np.ndarray]:
    """Attention for one head.

    q_h: [Nq, d] query rows; k_h, v_h: [Nk, d]; row_ids: the absolute query
    index of each row of q_h (defaults to 0..Nq-1), used only by the causal
    mask. Returns O [Nq, d] and LSE [Nq], both float64.
    """
    q_h, k_h, v_h = to_f64(q_h), to_f64(k_h), to_f64(v_h)
    _check_head_shapes(q_h, k_h, v_h)
    S = scores(q_h, k_h, scale)
    if causal:
        if row_ids is None:
            row_ids = np.arange(q_h.shape[0])
        S = apply_causal_mask(S, np.asarray(row_ids))
    P, m, l = softmax_stats(S)
    O = (P @ v_h) / l[:, None]
    lse = m + np.log(l)
    return O, lse


def attention(q, k, v, scale: Optional[float] = None, causal: bool = False,
              row_block: int = 1024) -> Tuple[np.ndarray, np.ndarray]:
    """Attention over [B, H, Nq, d] queries and [B, H, Nk, d] keys/values.

    Returns O [B, H, Nq, d] and LSE [B, H, Nq] in float64. For memory, the
    query rows of a head are taken `row_block` at a time; each block still
    holds complete rows of S and does a complete row softmax.
    """
    q, k, v = to_f64(q), to_f64(k), to_f64(v)
    if q.ndim != 4 or k.ndim != 4 or v.ndim != 4:
        raise ValueError("expected [B, H, N, d] inputs")
    B, H, Nq, d = q.shape
    if k.shape[:2] != (B, H) or v.shape != k.shape or k.shape[3] != d:
        raise ValueError("shape mismatch between q, k, v")
    if min(B, H, Nq, k.shape[2], d) < 1:
        raise ValueError("empty input")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    O = np.empty((B, H, Nq, d), dtype=np.float64)
    L = np.empty((B, H, Nq), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            for r0 in range(0, Nq, row_block):
                r1 = min(Nq, r0 + row_block)
                O[b, h, r0:r1], L[b, h, r0:r1] = attention_head(
                    q[b, h, r0:r1], k[b, h], v[b, h], scale, causal,
                    row_ids=np.arange(r0, r1))
    return O, L


def attention_rows(q, k, v, b: int, h: int, rows: Sequence[int],
                   scale: Optional[float] = None,
                   causal: bool = False) -> Tuple[np.ndarray, np.ndarray]:
    """Attention output for selected query rows of head (b, h) only.

    Lets a full-size problem be checked on sampled rows: each row's result is
    a function of that query row and the head's keys/values alone.
    """
    rows = np.asarray(rows, dtype=np.int64)
    qh = to_f64(q[b, h])[rows]
    d = qh.shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    return attention_head(qh, k[b, h], v[b, h], scale, causal, row_ids=rows)
