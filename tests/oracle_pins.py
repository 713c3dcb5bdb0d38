"""Checks that pin the oracle to facts outside itself.

Each check takes the oracle module (normally `oracle.definition`) and raises
AssertionError (or any exception) when the module disagrees with:
  * brute force: a naive pure-Python loop over tiny inputs (no numpy, no max
    subtraction), written independently of the oracle's code;
  * closed forms (one key; two keys as a logistic mix);
  * the hand-derived examples in tests/golden/hand_examples.json;
  * invariants of the definition (rows of the softmax sum to 1, identical V
    rows, identical K rows, key/value permutation, scale 0, the causal first
    row and prefixes, a constant logit shift, affine V, independence of
    batches and heads, row-blocking);
  * PyTorch's CPU float64 scaled_dot_product_attention (the library call that
    the kwkr.cn YOLO11 article, section 2.2, and the ai2ai.xin principle page,
    usage section, make) and torch.logsumexp.
tests/test_oracle.py runs them on the oracle; tests/test_oracle_mutants.py
plants mistakes in a copy of the oracle and requires some check to fail.
"""
from __future__ import annotations

import json
import math
import os
import random

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "hand_examples.json")
TOL = 1e-12


def _close(a, b, tol=TOL, what=""):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} != {b.shape}"
    err = np.max(np.abs(a - b)) if a.size else 0.0
    assert err <= tol, f"{what}: max abs err {err} > {tol}"


def _rand(shape, rng, sigma=1.0):
    return rng.standard_normal(shape) * sigma


def brute_force(q, k, v, scale, causal):
    """Naive attention with Python floats: weight_j = exp(scale * <q_i, k_j>)
    for every allowed key j (j <= i when causal), O_i = sum_j w_j v_j / sum_j w_j,
    LSE_i = ln sum_j w_j. Inputs are nested lists [B][H][N][d]."""
    B, H = len(q), len(q[0])
    O, L = [], []
    for b in range(B):
        Ob, Lb = [], []
        for h in range(H):
            Q, K, V = q[b][h], k[b][h], v[b][h]
            Oh, Lh = [], []
            for i, qi in enumerate(Q):
                ws = []
                for j, kj in enumerate(K):
                    if causal and j > i:
                        continue
                    dot = 0.0
                    for c in range(len(qi)):
                        dot += qi[c] * kj[c]
                    ws.append((j, math.exp(scale * dot)))
                Z = sum(w for _, w in ws)
                row = []
                for c in range(len(V[0])):
                    acc = 0.0
                    for j, w in ws:
                        acc += w * V[j][c]
                    row.append(acc / Z)
                Oh.append(row)
                Lh.append(math.log(Z))
            Ob.append(Oh)
            Lb.append(Lh)
        O.append(Ob)
        L.append(Lb)
    return np.array(O), np.array(L)


# ---------------------------------------------------------------- checks
def check_brute_force(ora):
    rng = np.random.default_rng(7)
    shapes = [(1, 1, 1, 1, 1), (1, 1, 2, 2, 2), (2, 2, 3, 3, 4), (1, 2, 5, 3, 2),
              (2, 1, 3, 6, 4), (1, 1, 7, 7, 3)]
    for (B, H, Nq, Nk, d) in shapes:
        for causal in (False, True):
            q = _rand((B, H, Nq, d), rng)
            k = _rand((B, H, Nk, d), rng)
            v = _rand((B, H, Nk, d), rng)
            scale = 0.37 + rng.random()
            O, L = ora.attention(q, k, v, scale=scale, causal=causal)
            Ob, Lb = brute_force(q.tolist(), k.tolist(), v.tolist(), scale, causal)
            _close(O, Ob, what=f"brute O {B,H,Nq,Nk,d,causal}")
            _close(L, Lb, what=f"brute LSE {B,H,Nq,Nk,d,causal}")


def check_brute_force_row_blocks(ora):
    """Row-blocked evaluation (several blocks, causal) against brute force."""
    rng = np.random.default_rng(11)
    B, H, N, d = 1, 2, 9, 3
    q, k, v = (_rand((B, H, N, d), rng) for _ in range(3))
    Ob, Lb = brute_force(q.tolist(), k.tolist(), v.tolist(), 0.8, True)
    for rb in (1, 2, 4, 9):
        O, L = ora.attention(q, k, v, scale=0.8, causal=True, row_block=rb)
        _close(O, Ob, what=f"row_block={rb} O")
        _close(L, Lb, what=f"row_block={rb} LSE")


def check_attention_rows(ora):
    """Sampled rows of a head (any order, causal or not) against brute force."""
    rng = np.random.default_rng(12)
    B, H, N, d = 2, 2, 8, 3
    q, k, v = (_rand((B, H, N, d), rng) for _ in range(3))
    for causal in (False, True):
        Ob, Lb = brute_force(q.tolist(), k.tolist(), v.tolist(), 0.6, causal)
        rows = [7, 2, 5, 0]
        O, L = ora.attention_rows(q, k, v, 1, 0, rows, scale=0.6, causal=causal)
        _close(O, Ob[1, 0][rows], what=f"rows O causal={causal}")
        _close(L, Lb[1, 0][rows], what=f"rows LSE causal={causal}")


def check_closed_forms(ora):
    rng = np.random.default_rng(3)
    for d in (1, 2, 4):
        # one key: O = v_0, LSE = S_00
        q = _rand((1, 1, 1, d), rng)
        k = _rand((1, 1, 1, d), rng)
        v = _rand((1, 1, 1, d), rng)
        s = 0.9
        O, L = ora.attention(q, k, v, scale=s)
        _close(O[0, 0, 0], v[0, 0, 0], what="N=1 O")
        _close(L[0, 0, 0], s * float(q[0, 0, 0] @ k[0, 0, 0]), what="N=1 LSE")
        # two keys: O = sig(S0-S1) v0 + (1-sig) v1, LSE = logaddexp(S0, S1)
        q = _rand((1, 1, 1, d), rng)
        k = _rand((1, 1, 2, d), rng)
        v = _rand((1, 1, 2, d), rng)
        O, L = ora.attention(q, k, v, scale=s)
        S0 = s * float(q[0, 0, 0] @ k[0, 0, 0])
        S1 = s * float(q[0, 0, 0] @ k[0, 0, 1])
        sig = 1.0 / (1.0 + math.exp(-(S0 - S1)))
        _close(O[0, 0, 0], sig * v[0, 0, 0] + (1 - sig) * v[0, 0, 1], what="N=2 O")
        _close(L[0, 0, 0], np.logaddexp(S0, S1), what="N=2 LSE")


def check_golden(ora):
    with open(GOLDEN, encoding="utf-8") as f:
        cases = json.load(f)["cases"]
    for c in cases:
        q = np.array(c["q"])[None, None]
        k = np.array(c["k"])[None, None]
        v = np.array(c["v"])[None, None]
        O, L = ora.attention(q, k, v, scale=c["scale"], causal=c["causal"])
        _close(O[0, 0], c["o"], tol=1e-12, what=c["name"] + " O")
        _close(L[0, 0], c["lse"], tol=1e-12, what=c["name"] + " LSE")


def check_rows_sum_to_one(ora):
    rng = np.random.default_rng(4)
    for causal in (False, True):
        q = _rand((6, 5), rng, 3.0)
        k = _rand((6, 5), rng, 3.0)
        P = ora.probabilities(q, k, 0.5, causal=causal)
        _close(P.sum(axis=1), np.ones(6), what="row sums")
        assert np.all(P >= 0)
        if causal:
            assert np.all(P[np.triu_indices(6, 1)] == 0.0), "causal weights above diagonal"


def check_identical_v_rows(ora):
    rng = np.random.default_rng(5)
    u = _rand((4,), rng)
    q = _rand((1, 1, 5, 4), rng, 2.0)
    k = _rand((1, 1, 7, 4), rng, 2.0)
    v = np.broadcast_to(u, (1, 1, 7, 4)).copy()
    for causal in (False, True):
        O, _ = ora.attention(q, k, v, scale=0.7, causal=causal)
        _close(O, np.broadcast_to(u, O.shape), what="identical V rows")


def check_identical_k_rows(ora):
    rng = np.random.default_rng(6)
    q = _rand((1, 1, 6, 3), rng, 2.0)
    k = np.broadcast_to(_rand((3,), rng), (1, 1, 6, 3)).copy()
    v = _rand((1, 1, 6, 3), rng)
    O, L = ora.attention(q, k, v, scale=1.3)
    _close(O[0, 0], np.broadcast_to(v[0, 0].mean(axis=0), (6, 3)), what="identical K -> mean V")
    O, L = ora.attention(q, k, v, scale=1.3, causal=True)
    prefix = np.cumsum(v[0, 0], axis=0) / np.arange(1, 7)[:, None]
    _close(O[0, 0], prefix, what="identical K causal -> prefix mean")


def check_permutation(ora):
    rng = np.random.default_rng(8)
    q = _rand((2, 3, 5, 4), rng)
    k = _rand((2, 3, 9, 4), rng)
    v = _rand((2, 3, 9, 4), rng)
    O, L = ora.attention(q, k, v, scale=0.5)
    perm = rng.permutation(9)
    Op, Lp = ora.attention(q, k[:, :, perm], v[:, :, perm], scale=0.5)
    _close(O, Op, tol=1e-12, what="perm O")
    _close(L, Lp, tol=1e-12, what="perm LSE")


def check_scale_zero(ora):
    rng = np.random.default_rng(9)
    q = _rand((1, 2, 4, 3), rng)
    k = _rand((1, 2, 6, 3), rng)
    v = _rand((1, 2, 6, 3), rng)
    O, L = ora.attention(q, k, v, scale=0.0)
    _close(O, np.broadcast_to(v.mean(axis=2, keepdims=True), O.shape), what="scale 0 O")
    _close(L, np.full(L.shape, math.log(6)), what="scale 0 LSE")


def check_causal_rows(ora):
    rng = np.random.default_rng(10)
    q = _rand((1, 1, 6, 4), rng)
    k = _rand((1, 1, 6, 4), rng)
    v = _rand((1, 1, 6, 4), rng)
    O, L = ora.attention(q, k, v, scale=0.9, causal=True)
    _close(O[0, 0, 0], v[0, 0, 0], what="causal row 0 O")
    _close(L[0, 0, 0], 0.9 * float(q[0, 0, 0] @ k[0, 0, 0]), what="causal row 0 LSE")
    for i in range(6):
        Oi, Li = ora.attention(q[:, :, i:i + 1], k[:, :, :i + 1], v[:, :, :i + 1], scale=0.9)
        _close(O[0, 0, i], Oi[0, 0, 0], what=f"causal prefix row {i}")
        _close(L[0, 0, i], Li[0, 0, 0], what=f"causal prefix LSE {i}")


def check_logit_shift(ora):
    rng = np.random.default_rng(13)
    q = _rand((1, 1, 4, 3), rng)
    k = _rand((1, 1, 5, 3), rng)
    v = _rand((1, 1, 5, 3), rng)
    s, c = 0.8, 2.5
    O, L = ora.attention(q, k, v, scale=s)
    q2 = np.concatenate([q, np.ones((1, 1, 4, 1))], axis=3)
    k2 = np.concatenate([k, np.full((1, 1, 5, 1), c / s)], axis=3)
    v2 = v  # value width may differ from the query width? keep equal widths:
    O2, L2 = ora.attention(q2, k2, np.concatenate([v2, np.zeros((1, 1, 5, 1))], axis=3), scale=s)
    _close(O2[..., :3], O, tol=1e-12, what="logit shift O")
    _close(L2, L + c, tol=1e-12, what="logit shift LSE")


def check_affine_v(ora):
    rng = np.random.default_rng(14)
    q = _rand((1, 1, 4, 3), rng)
    k = _rand((1, 1, 5, 3), rng)
    v = _rand((1, 1, 5, 3), rng)
    u = _rand((3,), rng)
    a = -1.7
    for causal in (False, True):
        O, _ = ora.attention(q, k, v, scale=0.6, causal=causal)
        O2, _ = ora.attention(q, k, a * v + u, scale=0.6, causal=causal)
        _close(O2, a * O + u, tol=1e-12, what="affine V")


def check_batch_head_independence(ora):
    rng = np.random.default_rng(15)
    q = _rand((2, 3, 4, 2), rng)
    k = _rand((2, 3, 5, 2), rng)
    v = _rand((2, 3, 5, 2), rng)
    O, L = ora.attention(q, k, v, scale=0.5)
    for b in range(2):
        for h in range(3):
            Oh, Lh = ora.attention(q[b:b + 1, h:h + 1], k[b:b + 1, h:h + 1],
                                   v[b:b + 1, h:h + 1], scale=0.5)
            _close(O[b, h], Oh[0, 0], what="independence O")
            _close(L[b, h], Lh[0, 0], what="independence LSE")
    # changing another head's inputs leaves this head unchanged
    k2 = k.copy()
    k2[1, 2] += 1.0
    O2, L2 = ora.attention(q, k2, v, scale=0.5)
    _close(O2[0], O[0], what="other batch untouched")
    _close(O2[1, :2], O[1, :2], what="other head untouched")


def check_torch_sdpa(ora):
    import torch
    import torch.nn.functional as F

    g = torch.Generator().manual_seed(16)
    for (B, H, Nq, Nk, d) in [(2, 3, 17, 17, 8), (1, 2, 5, 11, 4), (1, 1, 33, 33, 16)]:
        for causal in (False, True):
            if causal and Nq != Nk:
                continue
            q = torch.randn(B, H, Nq, d, generator=g, dtype=torch.float64)
            k = torch.randn(B, H, Nk, d, generator=g, dtype=torch.float64)
            v = torch.randn(B, H, Nk, d, generator=g, dtype=torch.float64)
            ref = F.scaled_dot_product_attention(q, k, v, is_causal=causal)  # default scale
            O, L = ora.attention(q.numpy(), k.numpy(), v.numpy(), causal=causal)
            _close(O, ref.numpy(), tol=1e-12, what="sdpa O")
            s = (q @ k.transpose(-1, -2)) / math.sqrt(d)
            if causal:
                s = s.masked_fill(torch.ones(Nq, Nk, dtype=torch.bool).triu(1), float("-inf"))
            _close(L, torch.logsumexp(s, dim=-1).numpy(), tol=1e-12, what="logsumexp LSE")


ALL_CHECKS = [
    check_brute_force,
    check_brute_force_row_blocks,
    check_attention_rows,
    check_closed_forms,
    check_golden,
    check_rows_sum_to_one,
    check_identical_v_rows,
    check_identical_k_rows,
    check_permutation,
    check_scale_zero,
    check_causal_rows,
    check_logit_shift,
    check_affine_v,
    check_batch_head_independence,
    check_torch_sdpa,
]
