"""The process-pool runner of the oracle returns what the oracle itself
returns: it only distributes heads and row blocks (no arithmetic of its own)."""
import numpy as np

import oracle
from oracle import pool
from tests.gpu_util import rand_inputs


def test_pool_equals_oracle():
    q, k, v = rand_inputs(2, 3, 150, 170, 32, "bf16", seed=11)
    for causal in (False, True):
        O, L = oracle.attention(q, k, v, scale=0.2, causal=causal)
        Op, Lp = pool.attention(q, k, v, scale=0.2, causal=causal, row_block=64, workers=3)
        assert np.allclose(Op, O, rtol=0, atol=1e-12) and np.allclose(Lp, L, rtol=0, atol=1e-12)


def test_pool_selected_heads_and_rows():
    q, k, v = rand_inputs(2, 2, 90, 90, 64, "fp16", seed=12)
    rows = [0, 1, 5, 40, 89]
    heads = [(1, 0), (0, 1)]
    Op, Lp = pool.attention_heads(q, k, v, heads, causal=True, rows=rows, row_block=2, workers=2)
    for i, (b, h) in enumerate(heads):
        O, L = oracle.attention_rows(q, k, v, b, h, rows, causal=True)
        assert np.allclose(Op[i], O, rtol=0, atol=1e-12) and np.allclose(Lp[i], L, rtol=0, atol=1e-12)


def test_host_description():
    assert pool.host_cores() >= 1
    assert isinstance(pool.cpu_model(), str) and pool.cpu_model()
