"""The seeded input generator: determinism, shapes and value distributions."""
import math

import pytest
import torch

from workloads import WORKLOADS, WORKLOAD_ORDER, Workload, make_inputs, sha256


def test_workload_table():
    assert WORKLOAD_ORDER == list(WORKLOADS)
    w = WORKLOADS["yolo20"]
    assert (w.B, w.H, w.Nq, w.Nk, w.d, w.dtype, w.causal) == (1, 2, 400, 400, 64, "fp16", False)
    w = WORKLOADS["yolo80b16"]
    assert (w.B, w.H, w.Nq, w.Nk, w.d, w.dtype, w.causal) == (16, 4, 6400, 6400, 32, "fp16", False)
    w = WORKLOADS["seq2048"]
    assert (w.B, w.H, w.Nq, w.Nk, w.d, w.dtype, w.causal) == (32, 16, 2048, 2048, 64, "fp16", True)
    w = WORKLOADS["long16k"]
    assert (w.B, w.H, w.Nq, w.Nk, w.d, w.dtype, w.causal) == (1, 32, 16384, 16384, 128, "bf16", True)
    w = WORKLOADS["tail361"]
    assert (w.B, w.H, w.Nq, w.Nk, w.d, w.dtype, w.causal) == (8, 2, 361, 361, 64, "fp16", False)
    assert w.q_dist == ("normal", 8.0) and w.v_dist == ("uniform", 1.0)


def test_flop_and_byte_counts():
    w = WORKLOADS["yolo80b16"]
    assert w.flops() == 4.0 * 16 * 4 * 6400 * 6400 * 32
    w = WORKLOADS["seq2048"]
    assert w.flops() == 4.0 * 32 * 16 * 2048 * 2048 * 64 / 2
    w = WORKLOADS["yolo20"]
    assert w.algorithmic_bytes() == 2 * 2 * 400 * 64 * 4 + 4 * 2 * 400
    assert math.isclose(w.scale, 0.125)


@pytest.mark.parametrize("name", ["yolo20", "tail361"])
def test_deterministic(name):
    w = WORKLOADS[name]
    a = make_inputs(w)
    b = make_inputs(w)
    for x, y in zip(a, b):
        assert x.dtype == w.torch_dtype and x.is_contiguous()
        assert sha256(x) == sha256(y)
    c = make_inputs(w, seed=w.seed + 1)
    assert sha256(a[0]) != sha256(c[0])


def test_shapes_and_distributions():
    w = WORKLOADS["tail361"]
    q, k, v = make_inputs(w)
    assert q.shape == (8, 2, 361, 64) and k.shape == (8, 2, 361, 64) and v.shape == (8, 2, 361, 64)
    qf, vf = q.float(), v.float()
    assert abs(qf.std().item() - 8.0) < 0.1
    assert abs(qf.mean().item()) < 0.1
    assert vf.min().item() >= -1.0 and vf.max().item() <= 1.0
    assert abs(vf.std().item() - 1 / math.sqrt(3)) < 0.01
    w = WORKLOADS["yolo20"].replace(dtype="bf16")
    q, _, _ = make_inputs(w)
    assert q.dtype == torch.bfloat16
    assert abs(q.float().std().item() - 1.0) < 0.02


def test_rectangular_workload():
    w = Workload("rect", 2, 3, 17, 45, 32, "fp16", False, seed=5)
    q, k, v = make_inputs(w)
    assert q.shape == (2, 3, 17, 32) and k.shape == (2, 3, 45, 32) and v.shape == k.shape
