"""Checks that pin the gradient oracle (oracle/backward.py) to facts outside it.

Each check takes a module exposing attention_backward_head, attention_backward
and row_delta, and raises when it disagrees with:
  * central finite differences of the forward oracle (oracle.definition) on
    tiny inputs: the gradient of sum(O * dO) with respect to Q, K and V;
  * float64 autograd of a plain PyTorch attention (matmul, masked_fill,
    softmax, matmul) on the CPU;
  * closed forms: one key (P = 1, so dQ = dK = 0 and dV = sum of dO), scale 0
    (uniform weights: dQ = dK = 0, every dV row the mean of dO);
  * invariants: dK sums to zero over the keys and dV sums to the sum of dO
    (rows of P sum to 1); identical K rows give dQ = 0; adding one vector to
    every K row changes nothing; the gradients are linear in dO; row_delta
    equals sum_j P_ij (dO V^T)_ij;
  * the default scale 1/sqrt(d): float64 autograd of PyTorch's CPU
    scaled_dot_product_attention called without a scale.
tests/test_oracle_backward.py runs them on the oracle and on planted mistakes.
"""
from __future__ import annotations

import numpy as np

from oracle import definition as fwd

TOL = 1e-10


def _close(a, b, tol=TOL, what=""):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} != {b.shape}"
    err = np.max(np.abs(a - b)) if a.size else 0.0
    assert err <= tol, f"{what}: max abs err {err} > {tol}"


def _inputs(rng, B, H, Nq, Nk, d, sigma=1.0):
    q = rng.standard_normal((B, H, Nq, d)) * sigma
    k = rng.standard_normal((B, H, Nk, d)) * sigma
    v = rng.standard_normal((B, H, Nk, d))
    do = rng.standard_normal((B, H, Nq, d))
    return q, k, v, do


def check_finite_differences(ora):
    rng = np.random.default_rng(11)
    for causal, (Nq, Nk, d) in ((False, (3, 4, 3)), (True, (4, 4, 2)), (False, (2, 5, 4))):
        q, k, v, do = _inputs(rng, 1, 1, Nq, Nk, d)
        scale = 0.7
        dQ, dK, dV = ora.attention_backward_head(q[0, 0], k[0, 0], v[0, 0], do[0, 0], scale, causal)

        def loss(qh, kh, vh):
            O, _ = fwd.attention_head(qh, kh, vh, scale, causal)
            return float((O * do[0, 0]).sum())

        h = 1e-6
        for which, grad in (("q", dQ), ("k", dK), ("v", dV)):
            base = {"q": q[0, 0], "k": k[0, 0], "v": v[0, 0]}
            num = np.zeros_like(base[which])
            for idx in np.ndindex(*num.shape):
                plus = {n: a.copy() for n, a in base.items()}
                minus = {n: a.copy() for n, a in base.items()}
                plus[which][idx] += h
                minus[which][idx] -= h
                num[idx] = (loss(plus["q"], plus["k"], plus["v"])
                            - loss(minus["q"], minus["k"], minus["v"])) / (2 * h)
            _close(grad, num, 1e-7, f"finite differences d{which} causal={causal}")


def check_torch_autograd(ora):
    import torch

    rng = np.random.default_rng(12)
    for causal, (B, H, Nq, Nk, d) in ((False, (2, 2, 7, 9, 5)), (True, (1, 3, 9, 9, 4)),
                                      (True, (1, 1, 6, 11, 3))):
        q, k, v, do = _inputs(rng, B, H, Nq, Nk, d, sigma=1.5)
        scale = 0.4
        tq, tk, tv = (torch.tensor(a, dtype=torch.float64, requires_grad=True) for a in (q, k, v))
        S = (tq @ tk.transpose(-1, -2)) * scale
        if causal:
            mask = torch.ones(Nq, Nk, dtype=torch.bool).triu(1)
            S = S.masked_fill(mask, float("-inf"))
        O = torch.softmax(S, dim=-1) @ tv
        O.backward(torch.tensor(do, dtype=torch.float64))
        dQ, dK, dV = ora.attention_backward(q, k, v, do, scale=scale, causal=causal)
        _close(dQ, tq.grad.numpy(), 1e-11, f"autograd dQ causal={causal}")
        _close(dK, tk.grad.numpy(), 1e-11, f"autograd dK causal={causal}")
        _close(dV, tv.grad.numpy(), 1e-11, f"autograd dV causal={causal}")


def check_one_key(ora):
    rng = np.random.default_rng(13)
    q, k, v, do = _inputs(rng, 1, 2, 5, 1, 4)
    for causal in (False, True):
        dQ, dK, dV = ora.attention_backward(q, k, v, do, scale=0.9, causal=causal)
        _close(dQ, np.zeros_like(dQ), what="one key dQ")
        _close(dK, np.zeros_like(dK), what="one key dK")
        _close(dV[:, :, 0], do.sum(axis=2), what="one key dV")


def check_scale_zero(ora):
    rng = np.random.default_rng(14)
    q, k, v, do = _inputs(rng, 1, 2, 6, 8, 3)
    dQ, dK, dV = ora.attention_backward(q, k, v, do, scale=0.0, causal=False)
    _close(dQ, np.zeros_like(dQ), what="scale 0 dQ")
    _close(dK, np.zeros_like(dK), what="scale 0 dK")
    _close(dV, np.broadcast_to(do.sum(axis=2, keepdims=True) / 8, dV.shape), what="scale 0 dV")


def check_sums(ora):
    rng = np.random.default_rng(15)
    q, k, v, do = _inputs(rng, 2, 2, 7, 10, 4, sigma=2.0)
    for causal in (False, True):
        _, dK, dV = ora.attention_backward(q, k, v, do, scale=0.6, causal=causal)
        _close(dK.sum(axis=2), np.zeros(dK.shape[:2] + (4,)), 1e-10, f"sum dK causal={causal}")
        _close(dV.sum(axis=2), do.sum(axis=2), 1e-10, f"sum dV causal={causal}")


def check_identical_keys(ora):
    rng = np.random.default_rng(16)
    q, k, v, do = _inputs(rng, 1, 2, 6, 6, 5)
    k[:] = k[:, :, :1]
    for causal in (False, True):
        dQ, _, _ = ora.attention_backward(q, k, v, do, scale=0.8, causal=causal)
        _close(dQ, np.zeros_like(dQ), 1e-12, f"identical keys dQ causal={causal}")


def check_key_shift(ora):
    rng = np.random.default_rng(17)
    q, k, v, do = _inputs(rng, 1, 2, 7, 9, 4)
    shift = rng.standard_normal(4)
    for causal in (False, True):
        a = ora.attention_backward(q, k, v, do, scale=0.5, causal=causal)
        b = ora.attention_backward(q, k + shift, v, do, scale=0.5, causal=causal)
        for x, y, n in zip(a, b, ("dQ", "dK", "dV")):
            _close(x, y, 1e-10, f"key shift {n} causal={causal}")


def check_linear_in_do(ora):
    rng = np.random.default_rng(18)
    q, k, v, do1 = _inputs(rng, 1, 2, 5, 7, 3)
    do2 = rng.standard_normal(do1.shape)
    for causal in (False, True):
        g1 = ora.attention_backward(q, k, v, do1, scale=0.7, causal=causal)
        g2 = ora.attention_backward(q, k, v, do2, scale=0.7, causal=causal)
        g3 = ora.attention_backward(q, k, v, do1 + 2.0 * do2, scale=0.7, causal=causal)
        for x, y, z, n in zip(g1, g2, g3, ("dQ", "dK", "dV")):
            _close(z, x + 2.0 * y, 1e-10, f"linear in dO {n} causal={causal}")


def check_row_delta(ora):
    rng = np.random.default_rng(19)
    q, k, v, do = _inputs(rng, 2, 1, 6, 8, 4)
    for causal in (False, True):
        O, _ = fwd.attention(q, k, v, scale=0.9, causal=causal)
        D = ora.row_delta(O, do)
        for b in range(2):
            P = fwd.probabilities(q[b, 0], k[b, 0], 0.9, causal)
            ref = (P * (do[b, 0] @ v[b, 0].T)).sum(axis=1)
            _close(D[b, 0], ref, 1e-12, f"row delta causal={causal}")


def check_default_scale(ora):
    import torch
    import torch.nn.functional as F

    rng = np.random.default_rng(20)
    q, k, v, do = _inputs(rng, 1, 2, 5, 6, 7)
    for causal in (False, True):
        tq, tk, tv = (torch.tensor(a, dtype=torch.float64, requires_grad=True) for a in (q, k, v))
        O = F.scaled_dot_product_attention(tq, tk, tv, is_causal=causal)
        O.backward(torch.tensor(do, dtype=torch.float64))
        dQ, dK, dV = ora.attention_backward(q, k, v, do, causal=causal)
        _close(dQ, tq.grad.numpy(), 1e-11, f"default scale dQ causal={causal}")
        _close(dK, tk.grad.numpy(), 1e-11, f"default scale dK causal={causal}")
        _close(dV, tv.grad.numpy(), 1e-11, f"default scale dV causal={causal}")


def check_sampled_matches_full(ora):
    """The row-blocked sampled form against the whole-head gradients."""
    rng = np.random.default_rng(21)
    for causal, (Nq, Nk, d, blk) in ((False, (37, 29, 8, 10)), (True, (40, 40, 6, 7)),
                                     (True, (25, 60, 4, 100))):
        q, k, v, do = _inputs(rng, 1, 1, Nq, Nk, d, sigma=1.3)
        full = ora.attention_backward_head(q[0, 0], k[0, 0], v[0, 0], do[0, 0], 0.45, causal)
        rows = [0, 3, Nq // 2, Nq - 1]
        keys = [0, 1, Nk // 3, Nk - 1]
        dq, dk, dv = ora.attention_backward_sampled(q[0, 0], k[0, 0], v[0, 0], do[0, 0], 0.45,
                                                    causal, rows, keys, row_block=blk)
        _close(dq, full[0][rows], 1e-12, f"sampled dQ causal={causal}")
        _close(dk, full[1][keys], 1e-12, f"sampled dK causal={causal}")
        _close(dv, full[2][keys], 1e-12, f"sampled dV causal={causal}")


ALL_CHECKS = [
    check_finite_differences,
    check_torch_autograd,
    check_one_key,
    check_scale_zero,
    check_sums,
    check_identical_keys,
    check_key_shift,
    check_linear_in_do,
    check_row_delta,
    check_default_scale,
    check_sampled_matches_full,
]
