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


def rand_inputs(B, H, Nq, Nk, d, dtype, seed, sigma_qk=1.0, v_uniform=False):
    from workloads import Workload, make_inputs

    w = Workload("t", B, H, Nq, Nk, d, dtype, False,
                 q_dist=("normal", sigma_qk), k_dist=("normal", sigma_qk),
                 v_dist=("uniform", 1.0) if v_uniform else ("normal", 1.0), seed=seed)
    return make_inputs(w)


def default_scale(d):
    return 1.0 / math.sqrt(d)
