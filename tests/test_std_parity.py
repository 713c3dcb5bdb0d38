"""Parity of the standard (unfused) attention baseline, fa_std_fwd, with the
oracle: its O and LSE at the stated bar (as for fa_fwd), and its two
intermediates, the fp32 scores S and the rounded probabilities P, against the
oracle's S and softmax element by element. Padding columns of P are zero."""
import numpy as np
import pytest
import torch

import exact_attention_23_amd as fa
import oracle
from tests.gpu_util import compare, compare_oracle, default_scale, note, rand_inputs, require_gpu
from workloads import WORKLOADS, make_inputs

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
U_TYPE = {torch.float16: 2.0 ** -11, torch.bfloat16: 2.0 ** -8}

CASES = [
    # (B, H, Nq, Nk, d, dtype, causal)
    (1, 1, 1, 1, 64, "fp16", False),
    (1, 2, 17, 17, 32, "bf16", True),
    (2, 1, 63, 65, 64, "fp16", True),
    (1, 2, 129, 200, 128, "bf16", False),
    (2, 2, 300, 257, 64, "fp16", False),
    (1, 1, 700, 100, 32, "fp16", True),
    (1, 1, 100, 700, 128, "fp16", True),
    (1, 2, 361, 361, 64, "bf16", True),
]


def _check_intermediates(q, k, v, s, p, scale, causal, what):
    B, H, Nq, _ = q.shape
    Nk = k.shape[2]
    u = U_TYPE[q.dtype]
    sg = s.cpu().double().numpy()[..., :Nk]
    pg = p.cpu().double().numpy()
    assert np.all(pg[..., Nk:] == 0.0), f"{what}: padding columns of P not zero"
    for b in range(B):
        for h in range(H):
            qh, kh = oracle.to_f64(q[b, h]), oracle.to_f64(k[b, h])
            S = oracle.scores(qh, kh, scale)
            # fp32 accumulation of d products, then one fp32 scaling
            bound_s = (qh.shape[1] + 2) * 2.0 ** -24 * (np.abs(qh) @ np.abs(kh).T) * abs(scale) + 1e-30
            ds = np.abs(sg[b, h] - S)
            assert np.all(ds <= bound_s), f"{what}: S off by {ds.max():.3e} (head {b},{h})"
            P = oracle.probabilities(q[b, h], k[b, h], scale, causal)
            dp = np.abs(pg[b, h, :, :Nk] - P)
            bound_p = (u + 1e-5) * P + 1e-7
            assert np.all(dp <= bound_p), f"{what}: P off by {dp.max():.3e} (head {b},{h})"


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B%dH%d_q%dk%d_d%d_%s_%s" % (
    c[0], c[1], c[2], c[3], c[4], c[5], "causal" if c[6] else "full"))
def test_std_small_shapes(case):
    require_gpu()
    B, H, Nq, Nk, d, dt, causal = case
    note(f"std parity {case}")
    q, k, v = rand_inputs(B, H, Nq, Nk, d, dt, seed=Nq * 7 + Nk + d)
    scale = default_scale(d)
    o, lse, s, p = fa.standard_attention(q.to(DEV), k.to(DEV), v.to(DEV), causal=causal, scale=scale,
                                         return_intermediates=True)
    torch.cuda.synchronize()
    assert s.shape[-1] == (Nk + 63) // 64 * 64
    O, L = oracle.attention(q, k, v, scale=scale, causal=causal)
    compare(o.cpu(), lse.cpu(), O, L, what=f"std {case}", vmax=float(v.float().abs().max()))
    _check_intermediates(q, k, v, s, p, scale, causal, f"std {case}")


def test_std_streaming_softmax_past_16384_keys():
    """Rows longer than the register-resident softmax (NkP > 16384) take the
    streaming form, which reads each row three times."""
    require_gpu()
    note("std parity Nk=17000")
    q, k, v = rand_inputs(1, 2, 40, 17000, 64, "fp16", seed=5)
    for causal in (False, True):
        o, lse = fa.standard_attention(q.to(DEV), k.to(DEV), v.to(DEV), causal=causal)
        O, L = oracle.attention(q, k, v, scale=default_scale(64), causal=causal)
        compare(o.cpu(), lse.cpu(), O, L, what=f"std Nk=17000 causal={causal}",
                vmax=float(v.float().abs().max()))


def test_std_large_logits():
    require_gpu()
    note("std parity large logits")
    q, k, v = rand_inputs(2, 2, 361, 361, 64, "fp16", seed=9, sigma_qk=8.0, v_uniform=True)
    o, lse = fa.standard_attention(q.to(DEV), k.to(DEV), v.to(DEV))
    O, L = oracle.attention(q, k, v, scale=default_scale(64))
    compare(o.cpu(), lse.cpu(), O, L, what="std large logits")


@pytest.mark.parametrize("name", ["yolo20", "seq2048", "tail361"])
def test_std_named_workload_full_size(name):
    """The baseline at the named workloads' full size (the one the benchmark
    compares with the fused forward is seq2048), every element of O and LSE."""
    require_gpu()
    w = WORKLOADS[name]
    note(f"std parity workload {name}")
    q, k, v = make_inputs(w)
    o, lse = fa.standard_attention(q.to(DEV), k.to(DEV), v.to(DEV), causal=w.causal, scale=w.scale)
    torch.cuda.synchronize()
    compare_oracle(o.cpu(), lse.cpu(), q, k, v, w.scale, w.causal, what=f"std {name}")


def test_std_matches_fused_within_rounding():
    """Same inputs through both paths: each is within the bar of the oracle, so
    they are within twice the bar of each other; also the LSEs agree."""
    require_gpu()
    q, k, v = (t.to(DEV) for t in rand_inputs(2, 4, 500, 500, 64, "fp16", seed=77))
    o1, l1 = fa.attention(q, k, v, causal=True)
    o2, l2 = fa.standard_attention(q, k, v, causal=True)
    assert float((o1.float() - o2.float()).abs().max()) <= 2e-2
    assert float((l1 - l2).abs().max()) <= 2e-3
