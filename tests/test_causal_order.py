"""Parity of causal launches under each branch of the block order the
library picks (groups of heads interleaved heaviest first, per-XCD ranges
when B*H is a multiple of 8, launch order otherwise): whole outputs of the
forward and the gradients of the backward against the oracles, on shapes
where a group holds several heads and every head several blocks. A block
mapped twice or not at all shows as wrong or untouched rows.

The forward is held to the stated bar on every element (bf16 elements with
reference |O| >= 4 to the bound in tests/gpu_util.compare), the backward to
its derived tolerance (tests/test_bwd_parity.compare_grads)."""
import pytest

import oracle
from tests.gpu_util import compare, default_scale, note, rand_inputs, require_gpu, run_gpu
from tests.test_bwd_parity import compare_grads, grad_like, run_bwd

pytestmark = pytest.mark.gpu

# (B, H, N, d, dtype): B*H = 16, 32, 64 take per-XCD ranges with groups of
# 2, 4 and 8 heads; 15 and 3 take the launch order with one group of all
# heads.
CASES = [
    (2, 8, 600, 64, "fp16"),
    (4, 8, 1000, 32, "fp16"),
    (8, 8, 700, 128, "bf16"),
    (3, 5, 900, 64, "fp16"),
    (1, 3, 1500, 128, "bf16"),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B{}H{}_n{}_d{}_{}".format(*c))
def test_causal_order_forward(case):
    require_gpu()
    B, H, N, d, dtype = case
    note(f"causal order forward {case}")
    q, k, v = rand_inputs(B, H, N, N, d, dtype, seed=31000 + B * 100 + H)
    o, lse = run_gpu(q, k, v, True, path="tiled")
    O, L = oracle.attention(q, k, v, scale=default_scale(d), causal=True)
    compare(o, lse, O, L, what=str(case), vmax=float(v.float().abs().max()))


@pytest.mark.parametrize("case", [CASES[0], CASES[3]], ids=lambda c: "B{}H{}_n{}_d{}_{}".format(*c))
def test_causal_order_backward(case):
    require_gpu()
    B, H, N, d, dtype = case
    note(f"causal order backward {case}")
    q, k, v = rand_inputs(B, H, N, N, d, dtype, seed=32000 + B * 100 + H)
    do = grad_like(q, 33000 + B * 100 + H)
    scale = default_scale(d)
    got = run_bwd(q, k, v, do, True, scale)
    ref = oracle.attention_backward(q, k, v, do, scale=scale, causal=True)
    compare_grads(got, ref, q.dtype, what=str(case))
