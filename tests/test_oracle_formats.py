"""Pins of the oracle's input conversion (to_f64, its torch branch) and of the
FP8 dequantisation the FP8 parity tests feed it (workloads.dequantize_fp8).

Every GPU parity test hands the oracle fp16, bf16 or e4m3 torch tensors, so
the conversion of those bit patterns to float64 must be exact. The expected
values below are decoded by hand from the formats' definitions, not by any
library conversion:
  * binary16 (IEEE 754): 1 sign bit, 5 exponent bits (bias 15), 10 fraction
    bits; exponent 0 is subnormal, (fraction / 2^10) * 2^-14;
  * bfloat16: the upper half of a binary32: 1 sign, 8 exponent bits (bias
    127), 7 fraction bits; exponent 0 is subnormal, (fraction / 2^7) * 2^-126;
  * OCP 8-bit floating point, E4M3 ("fn": no infinities): 1 sign, 4 exponent
    bits (bias 7), 3 fraction bits; exponent 0 is subnormal,
    (fraction / 8) * 2^-6; S.1111.111 is NaN, so 448 = 2^8 * 1.75 is the
    largest finite value.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from workloads import dequantize_fp8

# (bits, value) pairs, each value worked out from the fields of the bits
FP16 = [
    (0x3C00, 1.0),                      # exp 15 -> 2^0
    (0xC000, -2.0),                     # sign, exp 16
    (0x7BFF, (1 + 1023 / 1024) * 2.0 ** 15),  # largest finite: 65504
    (0x0400, 2.0 ** -14),               # smallest normal
    (0x0001, 2.0 ** -24),               # smallest subnormal
    (0x03FF, 1023 * 2.0 ** -24),        # largest subnormal
    (0x3555, (1 + 341 / 1024) * 2.0 ** -2),  # 0.333251953125, the fp16 nearest 1/3
    (0x8000, -0.0),
]
BF16 = [
    (0x3F80, 1.0),                      # exp 127
    (0xC040, -3.0),                     # sign, exp 128, fraction 64/128
    (0x7F7F, (1 + 127 / 128) * 2.0 ** 127),  # largest finite
    (0x0080, 2.0 ** -126),              # smallest normal
    (0x0001, 2.0 ** -133),              # smallest subnormal
    (0x007F, 127 * 2.0 ** -133),        # largest subnormal
    (0x3EAB, (1 + 43 / 128) * 2.0 ** -2),  # 0.333984375
]
E4M3 = [
    (0x38, 1.0),                        # exp 7
    (0xB8, -1.0),
    (0x7E, (1 + 6 / 8) * 2.0 ** 8),     # largest finite: 448
    (0x77, (1 + 7 / 8) * 2.0 ** 7),     # 240
    (0x3C, 1.5),
    (0x08, 2.0 ** -6),                  # smallest normal
    (0x01, 2.0 ** -9),                  # smallest subnormal
    (0x07, 7 * 2.0 ** -9),              # largest subnormal
    (0x80, -0.0),
]


def _from_bits(pairs, int_dtype, view_dtype):
    bits = np.array([b for b, _ in pairs], dtype=int_dtype)
    signed = {np.uint16: np.int16, np.uint8: np.uint8}[int_dtype]
    t = torch.from_numpy(bits.view(signed).copy()).view(view_dtype)
    return t, np.array([v for _, v in pairs], dtype=np.float64)


@pytest.mark.parametrize("pairs,int_dtype,dtype", [
    (FP16, np.uint16, torch.float16), (BF16, np.uint16, torch.bfloat16),
    (E4M3, np.uint8, torch.float8_e4m3fn)], ids=["fp16", "bf16", "e4m3"])
def test_to_f64_decodes_bit_patterns(pairs, int_dtype, dtype):
    t, want = _from_bits(pairs, int_dtype, dtype)
    got = oracle.to_f64(t)
    assert got.dtype == np.float64
    assert np.array_equal(got, want)
    assert np.array_equal(np.signbit(got), np.signbit(want))  # -0.0 stays negative


def test_to_f64_e4m3_nan():
    t = torch.tensor([0x7F], dtype=torch.uint8).view(torch.float8_e4m3fn)
    assert math.isnan(float(oracle.to_f64(t)[0]))


def test_to_f64_keeps_shape_and_numpy_branch():
    t, want = _from_bits(FP16[:6], np.uint16, torch.float16)
    t = t.reshape(2, 3)
    assert oracle.to_f64(t).shape == (2, 3)
    assert np.array_equal(oracle.to_f64(want.reshape(2, 3)), want.reshape(2, 3))


def test_attention_of_torch_tensor_matches_decoded_values():
    """The oracle on fp16/bf16 torch tensors equals the oracle on the
    hand-decoded float64 values of the same bits."""
    rng = np.random.default_rng(3)
    for pairs, dt in ((FP16, torch.float16), (BF16, torch.bfloat16)):
        finite = [(b, v) for b, v in pairs if abs(v) < 1e4 and abs(v) > 1e-30 or v == 0.0]
        idx = rng.integers(0, len(finite), size=(1, 1, 5, 4))
        bits = np.array([[finite[i][0] for i in row] for row in idx.reshape(-1, 4)], dtype=np.uint16)
        vals = np.array([[finite[i][1] for i in row] for row in idx.reshape(-1, 4)])
        t = torch.from_numpy(bits.view(np.int16).copy()).view(dt).reshape(1, 1, 5, 4)
        O_t, L_t = oracle.attention(t, t, t, scale=0.5)
        v = vals.reshape(1, 1, 5, 4)
        O_n, L_n = oracle.attention(v, v, v, scale=0.5)
        assert np.array_equal(O_t, O_n) and np.array_equal(L_t, L_n)


def test_dequantize_fp8_exact():
    """dequantize_fp8 multiplies the decoded e4m3 value by the float32 value of
    the factor (0.1 as float32 is 13421773 * 2^-27), exactly."""
    t, want = _from_bits(E4M3, np.uint8, torch.float8_e4m3fn)
    got = dequantize_fp8(t, 0.1).numpy()
    assert got.dtype == np.float64
    f32_tenth = 13421773 * 2.0 ** -27
    assert np.array_equal(got, want * f32_tenth)
    # a factor that is exact in float32 scales exactly too
    assert np.array_equal(dequantize_fp8(t, 0.25).numpy(), want * 0.25)
