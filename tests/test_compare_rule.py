"""The comparison the GPU parity tests apply (tests/gpu_util.compare), checked
on the CPU with planted errors: the stated bar on every element, and for bf16
only elements with |O| >= 4 held to the derived bound instead."""
import numpy as np
import pytest
import torch

from tests.gpu_util import compare


def _case(dtype, err_at, err, O_val=1.0):
    O = np.full((1, 1, 8, 4), 0.5)
    O[0, 0, 3, 2] = O_val
    L = np.zeros((1, 1, 8))
    og = O.copy()
    og[err_at] += err
    return torch.from_numpy(og).to(dtype), torch.zeros(1, 1, 8), O, L


@pytest.mark.parametrize("dtype", [torch.float16, torch.bfloat16])
def test_bar_on_every_element(dtype):
    o, lse, O, L = _case(torch.float64, (0, 0, 5, 1), 0.0)
    compare(o.to(dtype).double(), lse, O, L)
    o, lse, O, L = _case(torch.float64, (0, 0, 5, 1), 0.02)
    with pytest.raises(AssertionError):
        compare(o, lse, O, L)


def test_bf16_small_outputs_get_no_exemption():
    # |O| = 3.9: an error of 0.0105 must fail even in bf16
    O = np.full((1, 1, 4, 2), 3.9)
    og = torch.from_numpy(O + np.array([0.0105, 0, 0, 0, 0, 0, 0, 0]).reshape(1, 1, 4, 2)).to(torch.float32)
    with pytest.raises(AssertionError):
        compare(og.to(torch.bfloat16), None, O, None, vmax=4.0)


class _Bf16Out:
    """Stands in for a bf16 GPU output holding arbitrary float64 values (a
    real bf16 tensor could not hold the planted 5.015)."""
    dtype = torch.bfloat16

    def __init__(self, a):
        self.a = a

    def double(self):
        return torch.from_numpy(self.a)


def test_bf16_large_outputs_derived_bound():
    O = np.full((1, 1, 64, 8), 0.1)
    O[0, 0, 0, 0] = 5.0
    good = O.copy()
    good[0, 0, 0, 0] += 0.015  # past 1e-2, inside 2^-8 (2*5 + vmax) with vmax = 5
    compare(_Bf16Out(good), None, O, None, vmax=5.0)
    bad = O.copy()
    bad[0, 0, 0, 0] += 0.2
    with pytest.raises(AssertionError):
        compare(_Bf16Out(bad), None, O, None, vmax=5.0)
    with pytest.raises(AssertionError):  # no vmax: the exemption cannot be checked
        compare(_Bf16Out(good), None, O, None)
    # fp16 gets no exemption at all
    class Fp16Out(_Bf16Out):
        dtype = torch.float16
    with pytest.raises(AssertionError):
        compare(Fp16Out(good), None, O, None, vmax=5.0)


def test_mean_and_lse_bars():
    O = np.zeros((1, 1, 100, 4))
    og = torch.from_numpy(O + 0.002)
    with pytest.raises(AssertionError):
        compare(og, None, O, None)
    L = np.zeros((1, 1, 100))
    with pytest.raises(AssertionError):
        compare(torch.from_numpy(O), torch.from_numpy(L + 0.0011), O, L)
