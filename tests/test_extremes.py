"""Parity at the edges of the accepted sizes.

* Many heads: B*H = 8192 small heads, through the tiled and the short-range
  kernel, so head and block indices reach values no named workload uses.
* The longest key range the library accepts: N*d must stay below 2^29
  elements per head (32-bit byte offsets within a head, include/fa.h), so for
  d = 128 that is Nk = 2^22 - 1 keys, a ragged last tile included, every one
  of them visible to every query. The oracle checks sampled query rows.
"""
import numpy as np
import pytest
import torch

import oracle
from tests.gpu_util import compare, default_scale, note, rand_inputs, require_gpu, run_gpu

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("path", ["auto", "short"])
@pytest.mark.parametrize("causal", [False, True])
def test_many_heads(path, causal):
    require_gpu()
    B, H, N, d = 32, 256, 70, 64
    note(f"parity many heads B={B} H={H} N={N} causal={causal} path={path}")
    q, k, v = rand_inputs(B, H, N, N, d, "fp16", seed=6100 + int(causal))
    o, lse = run_gpu(q, k, v, causal, path=path)
    rng = np.random.default_rng(6100)
    heads = sorted(set([(0, 0), (0, H - 1), (B - 1, 0), (B - 1, H - 1)] +
                       [(int(rng.integers(0, B)), int(rng.integers(0, H))) for _ in range(12)]))
    rows = list(range(N))
    for (b, h) in heads:
        O, L = oracle.attention_rows(q, k, v, b, h, rows, scale=default_scale(d), causal=causal)
        compare(o[b, h], lse[b, h], O, L, what=f"many heads ({b},{h}) causal={causal} {path}")
    assert torch.isfinite(o.float()).all() and torch.isfinite(lse).all()


def test_longest_key_range():
    require_gpu()
    d = 128
    Nk = (1 << 29) // d - 1
    Nq = 70
    note(f"parity longest key range Nq={Nq} Nk={Nk} d={d} bf16")
    q, k, v = rand_inputs(1, 1, Nq, Nk, d, "bf16", seed=6200)
    o, lse = run_gpu(q, k, v, False)
    rows = [0, 1, 31, 32, 63, 64, 69]
    O, L = oracle.attention_rows(q, k, v, 0, 0, rows, scale=default_scale(d), causal=False)
    compare(o[0, 0][rows], lse[0, 0][rows], O, L, what=f"Nk={Nk} sampled rows")
    assert torch.isfinite(o.float()).all() and torch.isfinite(lse).all()
