"""Helpers shared by the GPU tests: run the HIP path, compare with the oracle."""
from __future__ import annotations

import math
import sys

import numpy as np
import torch

import exact_attention_23_amd as fa
import oracle
from oracle import pool as oracle_pool

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


# bf16 keeps 8 significant bits: rounding moves a value by at most 2^-8 of
# itself. Half an ulp of a bf16 output at |O| in [4, 8) is 2^-6 = 0.0156,
# above the 1e-2 bar, so from |O| = 4 on no bf16 output can be held to it.
U_BF16 = 2.0 ** -8
BF16_EXEMPT_ABS_O = 4.0


def compare(o_gpu, lse_gpu, O_ref, L_ref, what="", vmax=None):
    """Element-wise comparison with the oracle at the stated bar: max|dO| <=
    1e-2, mean|dO| <= 1e-3 and max|dLSE| <= 1e-3, on every element.

    The one exception is bf16 outputs whose reference |O| is 4 or more, where
    rounding the output alone can exceed 1e-2. Those elements are held to a
    bound derived from the arithmetic instead: |dO| <= 2^-8 (2|O| + vmax) +
    1e-5, with vmax = max|V| of the inputs (needed only when such an element
    misses 1e-2). The terms: the output's rounding (2^-8 |O|) and the rounding
    of the weights P, which the kernel normalises by the sum of the rounded
    weights, so the output moves by sum_j w_j d_j (v_j - O) with |d_j| <= 2^-8,
    at most 2^-8 (sum_j w_j |v_j| + |O|) <= 2^-8 (vmax + |O|); fp32 sums add
    far less than 1e-5 here. Returns the error summary."""
    og = o_gpu.double().numpy()
    assert np.all(np.isfinite(og)), f"{what}: non-finite output"
    d = np.abs(og - O_ref)
    absO = np.abs(O_ref)
    max_o, mean_o = float(d.max()), float(d.mean())
    worst = np.unravel_index(int(d.argmax()), d.shape)
    max_l = 0.0
    if lse_gpu is not None:
        lg = lse_gpu.double().numpy()
        assert np.all(np.isfinite(lg)), f"{what}: non-finite LSE"
        max_l = float(np.abs(lg - L_ref).max())
    msg = (f"{what}: max|dO|={max_o:.3e} at {tuple(int(x) for x in worst)} "
           f"(|O|={absO[worst]:.3f}) mean|dO|={mean_o:.3e} max|dLSE|={max_l:.3e}")
    if o_gpu.dtype == torch.bfloat16:
        big = absO >= BF16_EXEMPT_ABS_O
        small_max = float(d[~big].max()) if (~big).any() else 0.0
        assert small_max <= MAX_ABS_O, msg + f"; max over |O| < 4: {small_max:.3e}"
        over = big & (d > MAX_ABS_O)
        if over.any():
            assert vmax is not None, msg + ": elements with |O| >= 4 miss 1e-2 and no vmax was given"
            bound = U_BF16 * (2.0 * absO + float(vmax)) + 1e-5
            ratio = float((d[over] / bound[over]).max())
            assert ratio <= 1.0, msg + f"; |O| >= 4 elements reach {ratio:.3f} of their bound"
    else:
        assert max_o <= MAX_ABS_O, msg
    assert mean_o <= MEAN_ABS_O, msg
    assert max_l <= MAX_ABS_LSE, msg
    return max_o, mean_o, max_l


def compare_oracle(o_gpu, lse_gpu, q, k, v, scale, causal, what=""):
    """The whole output of a call against the oracle (run on the host's
    process pool), at the stated bar (see compare)."""
    O, L = oracle_pool.attention(q, k, v, scale=scale, causal=causal)
    return compare(o_gpu, lse_gpu, O, L, what=what, vmax=float(v.float().abs().max()))


def rand_inputs(B, H, Nq, Nk, d, dtype, seed, sigma_qk=1.0, v_uniform=False):
    from workloads import Workload, make_inputs

    w = Workload("t", B, H, Nq, Nk, d, dtype, False,
                 q_dist=("normal", sigma_qk), k_dist=("normal", sigma_qk),
                 v_dist=("uniform", 1.0) if v_uniform else ("normal", 1.0), seed=seed)
    return make_inputs(w)


def default_scale(d):
    return 1.0 / math.sqrt(d)
