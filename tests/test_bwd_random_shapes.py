"""Backward parity on seeded random shapes: batch, heads, both sequence
lengths (1 to 500), head width, type and mask drawn at random (default
scale), each gradient compared element by element with the fp64 gradient
oracle under the backward's derived tolerance (test_bwd_parity)."""
import numpy as np
import pytest

import oracle
from tests.gpu_util import default_scale, note, rand_inputs, require_gpu
from tests.test_bwd_parity import compare_grads, grad_like, run_bwd

pytestmark = pytest.mark.gpu

N_CASES = 24


def _cases():
    rng = np.random.default_rng(8080)
    return [dict(B=int(rng.integers(1, 3)), H=int(rng.integers(1, 4)),
                 Nq=int(rng.integers(1, 501)), Nk=int(rng.integers(1, 501)),
                 d=int(rng.choice([32, 64, 128])), dtype=str(rng.choice(["fp16", "bf16"])),
                 causal=bool(rng.integers(0, 2)), seed=9000 + i) for i in range(N_CASES)]


@pytest.mark.parametrize("case", _cases(), ids=lambda c: "B{B}H{H}_q{Nq}k{Nk}_d{d}_{dtype}_{m}".format(
    m="causal" if c["causal"] else "full", **c))
def test_bwd_random_shape(case):
    require_gpu()
    c = case
    note(f"bwd parity random {c}")
    q, k, v = rand_inputs(c["B"], c["H"], c["Nq"], c["Nk"], c["d"], c["dtype"], seed=c["seed"])
    do = grad_like(q, c["seed"] + 1)
    scale = default_scale(c["d"])
    got = run_bwd(q, k, v, do, c["causal"], scale)
    ref = oracle.attention_backward(q, k, v, do, scale=scale, causal=c["causal"])
    compare_grads(got, ref, q.dtype, what=str(c))
