"""What the forward's bf16 arithmetic must produce, from the CPU rounding
model (tests/rounding_model.py), against the oracle.

These tests justify the tolerance the GPU tests apply to bf16. With O divided
by the fp32 sum of the unrounded weights while P V uses the rounded ones (the
normalisation of an earlier version of the kernels), the model reproduces the
excess that version showed on the GPU: max|dO| 0.0114 at row 2 (|O| 2.12) of
the seeded random-layout case with seed 9012. Dividing by the sum of the
rounded weights, as the kernels now do, brings every bf16 random case and the
16384-token workload's first rows within the stated 1e-2 wherever |O| < 4.
"""
import math

import numpy as np
import pytest

import oracle
from tests import rounding_model
from tests.gpu_util import rand_inputs
from tests.test_layouts_random import _cases as layout_cases
from tests.test_random_shapes import _cases as shape_cases
from workloads import WORKLOADS, make_inputs


def _short_per_cu(d, tiles):
    """Two-block short-range workgroups a compute unit holds (LDS for NWMAX
    waves, at most 16 waves), as the library counts them."""
    nwmax = 9 if d == 128 else (8 if tiles <= 8 else 16)
    region = max(64 * d * 2, 32 * (d + 4) * 4)
    lds = nwmax * region + 3 * nwmax * 32 * 4
    return max(1, min((160 * 1024) // lds, 16 // nwmax))


def _kernel_of(c):
    """The forward kernel a random case runs: its explicit path, or the
    automatic choice (the short-range kernel when its key range fits and its
    workgroups all run at once: one per 16 rows at most one per compute unit
    of 256, else one per 32 rows as many as the units hold)."""
    path = c.get("path", "auto")
    if path != "auto":
        return path
    tiles = (c["Nk"] + 63) // 64
    fits = tiles <= (9 if c["d"] == 128 else 16)
    heads = c["B"] * c["H"]
    t1, t2 = heads * ((c["Nq"] + 15) // 16), heads * ((c["Nq"] + 31) // 32)
    short = fits and (t1 <= 256 or t2 <= _short_per_cu(c["d"], tiles) * 256)
    return "short" if short else "tiled"


def _errors(c, norm, kernel):
    q, k, v = rand_inputs(c["B"], c["H"], c["Nq"], c["Nk"], c["d"], c["dtype"], seed=c["seed"])
    scale = c.get("scale") if c.get("scale") is not None else 1.0 / math.sqrt(c["d"])
    O, L = oracle.attention(q, k, v, scale=scale, causal=c["causal"])
    Om, Lm = rounding_model.forward(q, k, v, scale, c["causal"], norm=norm, kernel=kernel)
    return np.abs(Om - O), np.abs(O), np.abs(Lm - L)


def test_model_reproduces_the_measured_excess():
    c = [c for c in layout_cases() if c["seed"] == 9012][0]
    assert (c["dtype"], c["d"], c["causal"], c["Nq"], c["Nk"]) == ("bf16", 128, True, 280, 579)
    d, absO, _ = _errors(c, "fp32", "tiled")
    worst = np.unravel_index(int(d.argmax()), d.shape)
    assert 0.0105 <= d.max() <= 0.0125, d.max()
    assert worst[2] == 2 and 2.0 <= absO[worst] <= 2.3
    d2, absO2, _ = _errors(c, "rounded", "tiled")
    assert d2[absO2 < 4].max() <= 0.0090


BF16_CASES = [c for c in layout_cases() + shape_cases() if c["dtype"] == "bf16"]


@pytest.mark.parametrize("c", BF16_CASES, ids=lambda c: f"seed{c['seed']}")
def test_bf16_random_cases_within_bar(c):
    d, absO, dl = _errors(c, "rounded", _kernel_of(c))
    small = absO < 4
    assert d[small].max() <= 1e-2, d[small].max()
    assert d.mean() <= 1e-3 and dl.max() <= 1e-4


def test_long16k_first_rows_within_bar():
    """Rows 0-255 of all 32 heads of the 16384-token causal bf16 workload (a
    causal row i sees keys 0..i only, so keys past 255 are left out)."""
    w = WORKLOADS["long16k"]
    q, k, v = make_inputs(w)
    q, k, v = q[:, :, :256], k[:, :, :256], v[:, :, :256]
    O, _ = oracle.attention(q, k, v, scale=w.scale, causal=True)
    worst = {}
    for norm in ("fp32", "rounded"):
        Om, _ = rounding_model.forward(q, k, v, w.scale, True, norm=norm, kernel="tiled")
        worst[norm] = float(np.abs(Om - O).max())
    assert worst["rounded"] <= 0.0090 < worst["fp32"] + 0.001, worst
    assert worst["rounded"] < worst["fp32"]
