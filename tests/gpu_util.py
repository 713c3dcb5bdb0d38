"""Helpers shared by the GPU tests: run the HIP path, compare with the oracle."""
from __future__ import annotations

import math
import sys

import numpy as np
import torch

import exact_attention_23_amd as fa
import oracle

# Tolerances for fp16/bf16 inputs against the fp64 oracle.
MAX_ABS_O = 1e-2
MEAN_ABS_O = 1e-3
MAX_ABS_LSE = 1e-3


def require_gpu():
    if not torch.cuda.is_available():
        import pytest

        pytest.skip("no GPU in this process")
    fa._lib.load()  # a GPU machine without the built library must fail, not skip


def note(msg: str):
    """Print and flush what names the case before its GPU step."""
    print(msg, file=sys.stderr, flush=True)


def run_gpu(q, k, v, causal, scale=None, with_lse=True, path="auto"):
    dev = torch.device("cuda:0")
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    o, lse = fa.attention(qd, kd, vd, causal=causal, scale=scale, return_lse=with_lse, path=path)
    torch.cuda.synchronize()
    return o.cpu(), (lse.cpu() if lse is not None else None)


def compare(o_gpu, lse_gpu, O_ref, L_ref, what=""):
    """Element-wise comparison to the oracle; returns the error summary."""
    og = o_gpu.double().numpy()
    d = np.abs(og - O_ref)
    assert np.all(np.isfinite(og)), f"{what}: non-finite output"
    max_o, mean_o = float(d.max()), float(d.mean())
    worst = np.unravel_index(int(d.argmax()), d.shape)
    max_l = 0.0
    if lse_gpu is not None:
        lg = lse_gpu.double().numpy()
        assert np.all(np.isfinite(lg)), f"{what}: non-finite LSE"
        max_l = float(np.abs(lg - L_ref).max())
    msg = (f"{what}: max|dO|={max_o:.3e} at {tuple(int(x) for x in worst)} "
           f"(|O|={abs(O_ref[worst]):.3f}) mean|dO|={mean_o:.3e} max|dLSE|={max_l:.3e}")
    assert max_o <= MAX_ABS_O, msg
    assert mean_o <= MEAN_ABS_O, msg
    assert max_l <= MAX_ABS_LSE, msg
    return max_o, mean_o, max_l


# The 16-bit matrix instructions' accumulation, relative to sum |a b| (taken
# as the e4m3 instruction's measured 2^-14.7, rounded up to 2^-13).
EPS_ACC_16 = 2.0 ** -13
U_TYPE = {torch.float16: 2.0 ** -11, torch.bfloat16: 2.0 ** -8}  # half an ulp, relative


def compare_derived(o_gpu, lse_gpu, q, k, v, scale, causal, what=""):
    """Element-wise comparison against a bound derived from the arithmetic,
    for large logits in bf16, where rounding the output alone can take
    |dO| past 1e-2 (half an ulp of bf16 at |O| in [2, 4) is 0.0078): per
    element |dO| <= (u + 2 e) A + u |O| + 1e-5 and |dLSE| <= 1e-3 + e, with u
    half an ulp of the type (P and O are rounded to it), e = EPS_ACC_16 times
    the row's largest sum_c |scale q_ic k_jc| (score accumulation), and A the
    attention output of |V| (which bounds sum_j |dP_ij| |V_jc|)."""
    O, L = oracle.attention(q, k, v, scale=scale, causal=causal)
    A, _ = oracle.attention(q, k, v.abs(), scale=scale, causal=causal)
    B, H = q.shape[:2]
    M = np.empty(q.shape[:3])
    for b in range(B):
        for h in range(H):
            qa, ka = q[b, h].float().abs().numpy(), k[b, h].float().abs().numpy()
            S = oracle.scores(qa, ka, abs(scale))
            M[b, h] = S.max(axis=1)
    u = U_TYPE[q.dtype]
    e = EPS_ACC_16 * M[..., None]
    og = o_gpu.double().numpy()
    assert np.all(np.isfinite(og)), f"{what}: non-finite output"
    d = np.abs(og - O)
    bound = (u + 2 * e) * A + u * np.abs(O) + 1e-5
    ratio = d / bound
    worst = np.unravel_index(int(ratio.argmax()), ratio.shape)
    dl = np.abs(lse_gpu.double().numpy() - L)
    lratio = dl / (1e-3 + EPS_ACC_16 * M)
    msg = (f"{what}: worst |dO|/bound={ratio.max():.3f} at {tuple(int(x) for x in worst)} "
           f"(|dO|={d[worst]:.3e}, bound={bound[worst]:.3e}); max|dO|={d.max():.3e} "
           f"mean|dO|={d.mean():.3e}; max|dLSE|={dl.max():.3e} (worst ratio {lratio.max():.3f})")
    assert ratio.max() <= 1.0, msg
    assert lratio.max() <= 1.0, msg
    return msg


def rand_inputs(B, H, Nq, Nk, d, dtype, seed, sigma_qk=1.0, v_uniform=False):
    from workloads import Workload, make_inputs

    w = Workload("t", B, H, Nq, Nk, d, dtype, False,
                 q_dist=("normal", sigma_qk), k_dist=("normal", sigma_qk),
                 v_dist=("uniform", 1.0) if v_uniform else ("normal", 1.0), seed=seed)
    return make_inputs(w)


def default_scale(d):
    return 1.0 / math.sqrt(d)
