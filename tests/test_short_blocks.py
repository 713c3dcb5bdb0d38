"""Parity of the short-range kernel with one and with two 16-row blocks per
workgroup: the library takes one block while B*H*ceil(Nq/16) workgroups fit
one per compute unit and two otherwise, so the shapes below reach both
forms (B*H = 2 at N = 400: 50 workgroups of one block; B*H = 16 at N = 361:
368 one-block workgroups would have to share units, so 192 of two blocks),
for every head width, both masks and both 16-bit types, each compared
element by element with the oracle at the stated bar (bf16 elements with
reference |O| >= 4 held to the bound in tests/gpu_util.compare)."""
import pytest

import oracle
from tests.gpu_util import compare, default_scale, note, rand_inputs, require_gpu, run_gpu

pytestmark = pytest.mark.gpu

CASES = [dict(B=B, H=H, N=N, d=d, causal=causal, dtype=("bf16" if (d == 128) != causal else "fp16"))
         for d in (32, 64, 128) for causal in (False, True) for (B, H, N) in ((1, 2, 400), (8, 2, 361))]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B{B}H{H}_n{N}_d{d}_{dtype}_{m}".format(
    m="causal" if c["causal"] else "full", **c))
def test_short_blocks(case):
    require_gpu()
    c = case
    note(f"short blocks {c}")
    q, k, v = rand_inputs(c["B"], c["H"], c["N"], c["N"], c["d"], c["dtype"],
                          seed=41000 + c["d"] + 7 * c["N"] + int(c["causal"]))
    o, lse = run_gpu(q, k, v, c["causal"], path="short")
    O, L = oracle.attention(q, k, v, scale=default_scale(c["d"]), causal=c["causal"])
    compare(o, lse, O, L, what=str(c), vmax=float(v.float().abs().max()))
