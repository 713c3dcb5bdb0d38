"""Parity of the FP8 (e4m3) forward with the fp64 oracle on the dequantised inputs.

The oracle computes exact attention on the values the e4m3 tensors stand for
(descale * e4m3), so input quantisation is not an error here. The kernel
rounds each attention weight to e4m3 for the P V product (after scaling a
row's largest weight to 2^8) and divides by the fp32 sum of the unrounded
weights; its error per output element is therefore bounded by

    |dO_ic| <= 2^-4 * sum_j p_ij |V_jc|            (relative rounding of e4m3
              + 2^-18 * sum_j |V_jc|               normals; absolute step of
              + u_out * |O_ic| + 1e-5              subnormal weights below 2^-6,
                                                   over a row sum >= 2^8; and
                                                   the output rounding)

where p are the exact weights. sum_j p_ij |V_jc| is attention with |V| in
place of V, which the oracle computes.

The scores carry one more error: the e4m3 matrix instruction sums its 64
products to about 2^-14.7 of sum_k |a_k b_k| (measured on the MI355X over 64
random e4m3 MFMAs with operands up to 448, while sums of exactly
representable structured operands come out exact). With
M_i = max_j sum_c |scale q_ic k_jc| (the oracle's scores of |q| and |k|) and
e_i = 2^-13 M_i, each score is off by at most e_i, which moves the LSE by at
most e_i and each weight by a factor within exp(+-2 e_i). The tests therefore
require every element within 1.01 times the bound above plus 2 e_i * sum_j p_ij
|V_jc|, the mean error within half the mean bound, and |dLSE| <= 1e-3 + e_i
(the LSE comes from the unrounded weights). For inputs ~ N(0, 1), e_i is
below 1e-3; it matters for logits of several hundred.
"""
import numpy as np
import pytest
import torch

import exact_attention_23_amd as fa
import oracle
from tests.gpu_util import note, require_gpu
from workloads import WORKLOADS, Workload, dequantize_fp8, make_inputs_fp8

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
U_OUT = {torch.float16: 2.0 ** -11, torch.bfloat16: 2.0 ** -8}


def run_fp8(q8, k8, v8, sq, sk, sv, causal, scale, out_dtype):
    o, lse = fa.attention_fp8(q8.to(DEV), k8.to(DEV), v8.to(DEV), sq, sk, sv, causal=causal,
                              scale=scale, out_dtype=out_dtype)
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu()


EPS_ACC = 2.0 ** -13  # accumulation of the e4m3 matrix instruction, relative to sum |a b|


def score_abs_max(q, k, scale, rows=None):
    """M [..., rows] = max_j sum_c |scale q_ic k_jc| per head (oracle scores of |q|, |k|)."""
    qa, ka = q.abs().numpy(), k.abs().numpy()
    if qa.ndim == 2:  # one head
        qa = qa if rows is None else qa[rows]
        return oracle.scores(qa, ka, abs(scale)).max(axis=1)
    out = np.empty(qa.shape[:3])
    for b in range(qa.shape[0]):
        for h in range(qa.shape[1]):
            out[b, h] = oracle.scores(qa[b, h], ka[b, h], abs(scale)).max(axis=1)
    return out


def check_fp8(o, lse, O, L, A, vabs_sum, M, out_dtype, what):
    """A = attention with |V| (same rows as O); vabs_sum = sum_j |V_jc| per head;
    M = max_j sum_c |scale q_ic k_jc| per row."""
    og = o.double().numpy()
    assert np.all(np.isfinite(og)), f"{what}: non-finite output"
    d = np.abs(og - O)
    e = EPS_ACC * M[..., None]
    bound = ((2.0 ** -4 + 2 * e) * A + 2.0 ** -18 * vabs_sum + U_OUT[out_dtype] * np.abs(O)
             + 1e-5)
    ratio = d / bound
    worst = np.unravel_index(int(ratio.argmax()), ratio.shape)
    dlse = np.abs(lse.double().numpy() - L)
    lratio = dlse / (1e-3 + EPS_ACC * M)
    dl = float(dlse.max())
    msg = (f"{what}: worst |dO|/bound={ratio.max():.3f} at {tuple(int(x) for x in worst)} "
           f"(|dO|={d[worst]:.3e}, bound={bound[worst]:.3e}); mean|dO|={d.mean():.3e} "
           f"mean bound={bound.mean():.3e}; max|dO|={d.max():.3e}; max|dLSE|={dl:.3e} "
           f"(worst |dLSE|/bound={lratio.max():.3f})")
    assert ratio.max() <= 1.01, msg
    assert d.mean() <= 0.5 * bound.mean(), msg
    assert lratio.max() <= 1.0, msg
    return msg


def full_compare(B, H, Nq, Nk, d, causal, seed, out_dtype, scale=None, sigma=1.0, what=""):
    w = Workload("t", B, H, Nq, Nk, d, "bf16", causal, q_dist=("normal", sigma),
                 k_dist=("normal", sigma), seed=seed)
    q8, k8, v8, sq, sk, sv = make_inputs_fp8(w)
    q, k, v = dequantize_fp8(q8, sq), dequantize_fp8(k8, sk), dequantize_fp8(v8, sv)
    scale = w.scale if scale is None else scale
    o, lse = run_fp8(q8, k8, v8, sq, sk, sv, causal, scale, out_dtype)
    O, L = oracle.attention(q, k, v, scale=scale, causal=causal)
    A, _ = oracle.attention(q, k, v.abs(), scale=scale, causal=causal)
    vabs_sum = v.abs().sum(dim=2, keepdim=True).numpy()
    M = score_abs_max(q, k, scale)
    return check_fp8(o, lse, O, L, A, vabs_sum, M, out_dtype, what)


SMALL = [
    # (B, H, Nq, Nk, d, causal)
    (1, 1, 1, 1, 64, False),
    (1, 2, 17, 17, 128, True),
    (2, 1, 63, 65, 64, False),
    (1, 2, 128, 128, 64, True),
    (2, 1, 129, 129, 128, True),
    (1, 2, 361, 361, 64, False),
    (1, 1, 1000, 1000, 128, True),
    (2, 2, 100, 700, 64, False),
    (1, 2, 700, 100, 128, True),
    (1, 1, 1, 513, 64, False),
    # d = 32: half of each 64-deep Q K^T step, K and V loaded by separate waves
    (1, 1, 1, 1, 32, False),
    (2, 2, 63, 65, 32, True),
    (1, 2, 300, 257, 32, False),
    (1, 1, 700, 100, 32, True),
]


@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float16], ids=["bf16", "fp16"])
@pytest.mark.parametrize("case", SMALL, ids=lambda c: "B%dH%d_q%dk%d_d%d_%s" % (
    c[0], c[1], c[2], c[3], c[4], "causal" if c[5] else "full"))
def test_fp8_small_shapes(case, out_dtype):
    require_gpu()
    B, H, Nq, Nk, d, causal = case
    note(f"fp8 parity {case} {out_dtype}")
    full_compare(B, H, Nq, Nk, d, causal, seed=Nq * 13 + Nk + d, out_dtype=out_dtype, what=str(case))


@pytest.mark.parametrize("scale", [0.0, -0.125, 0.5])
def test_fp8_scales(scale):
    require_gpu()
    note(f"fp8 scale {scale}")
    for causal in (False, True):
        full_compare(2, 2, 150, 170, 64, causal, seed=41, out_dtype=torch.bfloat16, scale=scale,
                     what=f"scale={scale} causal={causal}")


def test_fp8_large_logits():
    """q, k ~ N(0, 8^2): nearly one-hot rows."""
    require_gpu()
    note("fp8 large logits")
    for d in (32, 64, 128):
        for causal in (False, True):
            full_compare(2, 2, 361, 361, d, causal, seed=d, out_dtype=torch.float16, sigma=8.0,
                         what=f"large logits d={d} causal={causal}")


def test_fp8_rejects_d16_and_bad_descale():
    require_gpu()
    w = Workload("t", 1, 1, 64, 64, 64, "bf16", False, seed=1)
    q8, k8, v8, sq, sk, sv = make_inputs_fp8(w)
    q8, k8, v8 = (t.to(DEV) for t in (q8, k8, v8))
    with pytest.raises(fa.FaError) as e:
        fa.attention_fp8(q8[..., :16].contiguous(), k8[..., :16].contiguous(),
                         v8[..., :16].contiguous(), sq, sk, sv)
    assert e.value.status == fa._lib.FA_ERR_HEADDIM
    for bad in (0.0, -1.0, float("nan"), float("inf")):
        with pytest.raises(fa.FaError) as e:
            fa.attention_fp8(q8, k8, v8, bad, sk, sv)
        assert e.value.status == fa._lib.FA_ERR_SCALE


def _sample_rows(N, rng, n=40):
    fixed = [0, 1, 31, 32, 127, 128, N // 2, N - 1]
    rows = set(r for r in fixed if 0 <= r < N)
    rows.update(int(x) for x in rng.integers(0, N, n))
    return sorted(rows)


@pytest.mark.parametrize("name", ["yolo80b16", "seq2048", "long16k", "tail361"])
def test_fp8_named_workload_full_size(name):
    """The named workloads with their inputs quantised to e4m3, at full size;
    sampled rows of a few heads."""
    require_gpu()
    w = WORKLOADS[name]
    note(f"fp8 workload {name}: B={w.B} H={w.H} N={w.Nq} d={w.d} causal={w.causal}")
    q8, k8, v8, sq, sk, sv = make_inputs_fp8(w)
    o, lse = run_fp8(q8, k8, v8, sq, sk, sv, w.causal, w.scale, torch.bfloat16)
    assert torch.isfinite(o.float()).all() and torch.isfinite(lse).all()
    q, k, v = dequantize_fp8(q8, sq), dequantize_fp8(k8, sk), dequantize_fp8(v8, sv)
    rng = np.random.default_rng(w.seed)
    heads = sorted(set([(0, 0), (w.B - 1, w.H - 1), (int(rng.integers(0, w.B)), int(rng.integers(0, w.H)))]))
    for (b, h) in heads:
        rows = _sample_rows(w.Nq, rng)
        O, L = oracle.attention_rows(q, k, v, b, h, rows, scale=w.scale, causal=w.causal)
        A, _ = oracle.attention_rows(q, k, v.abs(), b, h, rows, scale=w.scale, causal=w.causal)
        vabs_sum = v[b, h].abs().sum(dim=0, keepdim=True).numpy()
        M = score_abs_max(q[b, h], k[b, h], w.scale, rows)
        check_fp8(o[b, h][rows], lse[b, h][rows], O, L, A, vabs_sum, M, torch.bfloat16,
                  f"{name} head ({b},{h})")
