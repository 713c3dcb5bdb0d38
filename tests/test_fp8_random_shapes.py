"""FP8 (e4m3) forward on seeded random shapes: batch, heads, both sequence
lengths (1 to 700, ragged against the 64-key tiles and the query blocks),
head width, mask, output type, scale and input spread drawn at random, each
held element by element to the per-element bound of the FP8 path derived
in tests/test_fp8.py (check_fp8) against the fp64 oracle on the
dequantised inputs. The draws are fixed by the seed, so a failure names a
reproducible case."""
import numpy as np
import pytest
import torch

from tests.gpu_util import note, require_gpu
from tests.test_fp8 import full_compare

pytestmark = pytest.mark.gpu

N_CASES = 20


def _cases():
    rng = np.random.default_rng(20240911)
    out = []
    for i in range(N_CASES):
        out.append(dict(
            B=int(rng.integers(1, 4)), H=int(rng.integers(1, 5)),
            Nq=int(rng.integers(1, 701)), Nk=int(rng.integers(1, 701)),
            d=int(rng.choice([32, 64, 128])), causal=bool(rng.integers(0, 2)),
            out_dtype=str(rng.choice(["bf16", "fp16"])),
            scale=(None if rng.random() < 0.5 else float(rng.uniform(-1.0, 1.0))),
            sigma=float(rng.choice([1.0, 2.0])), seed=8000 + i))
    return out


@pytest.mark.parametrize("case", _cases(), ids=lambda c: "B{B}H{H}_q{Nq}k{Nk}_d{d}_{m}_{out_dtype}".format(
    m="causal" if c["causal"] else "full", **c))
def test_fp8_random_shape(case):
    require_gpu()
    c = case
    note(f"fp8 parity random {c}")
    out_dtype = torch.bfloat16 if c["out_dtype"] == "bf16" else torch.float16
    full_compare(c["B"], c["H"], c["Nq"], c["Nk"], c["d"], c["causal"], seed=c["seed"],
                 out_dtype=out_dtype, scale=c["scale"], sigma=c["sigma"], what=str(c))
