"""Parity on seeded random shapes with more heads and longer key ranges than
tests/test_random_shapes.py: batch 1-6, heads 1-8, Nq 1-699, Nk up to the
short-range kernel's limit (1024 keys, 576 at d = 128), every head width,
both types and masks, and the kernel choice drawn from short, auto and
tiled, so that the short-range kernel meets one- and two-block workgroups
and the tiled kernel both orders of causal blocks. Each case is compared
element by element with the oracle at the stated bar (bf16 elements with
reference |O| >= 4 held to the bound in tests/gpu_util.compare)."""
import math

import numpy as np
import pytest

import oracle
from tests.gpu_util import compare, note, rand_inputs, require_gpu, run_gpu

pytestmark = pytest.mark.gpu

N_CASES = 150


def _cases():
    rng = np.random.default_rng(5)
    out = []
    for i in range(N_CASES):
        d = int(rng.choice([32, 64, 128]))
        kmax = 576 if d == 128 else 1024
        out.append(dict(B=int(rng.integers(1, 7)), H=int(rng.integers(1, 9)), Nq=int(rng.integers(1, 700)),
                        Nk=int(rng.integers(1, kmax + 1)), d=d, dtype=str(rng.choice(["fp16", "bf16"])),
                        causal=bool(rng.integers(0, 2)), path=str(rng.choice(["short", "auto", "tiled"])),
                        seed=50000 + i))
    return out


@pytest.mark.parametrize("case", _cases(), ids=lambda c: "B{B}H{H}_q{Nq}k{Nk}_d{d}_{dtype}_{m}_{path}".format(
    m="causal" if c["causal"] else "full", **c))
def test_random_shape_wide(case):
    require_gpu()
    c = case
    note(f"parity wide random {c}")
    q, k, v = rand_inputs(c["B"], c["H"], c["Nq"], c["Nk"], c["d"], c["dtype"], seed=c["seed"])
    o, lse = run_gpu(q, k, v, c["causal"], path=c["path"])
    O, L = oracle.attention(q, k, v, scale=1.0 / math.sqrt(c["d"]), causal=c["causal"])
    compare(o, lse, O, L, what=str(c), vmax=float(v.float().abs().max()))
