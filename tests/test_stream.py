"""Parity of the persistent (stream) forward, fa_fwd_stream, with the fp64 oracle.

Shapes are chosen so that query blocks get cut between workgroups in every
way the split can produce: blocks in two pieces, blocks in many pieces (fewer
tiles than workgroups, so some workgroups have nothing to do), key tails,
Nq != Nk, and the full-size 80x80 batch-16 workload the benchmark times.
"""
import numpy as np
import pytest
import torch

import exact_attention_23_amd as fa
import oracle
from tests.gpu_util import compare, default_scale, note, rand_inputs, require_gpu
from workloads import WORKLOADS, make_inputs

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")

CASES = [
    # (B, H, Nq, Nk, d, dtype)
    (1, 1, 40, 70, 32, "fp16"),       # far fewer tiles than workgroups
    (1, 2, 300, 900, 64, "bf16"),
    (4, 8, 1000, 1000, 32, "fp16"),
    (2, 4, 3000, 2500, 64, "bf16"),
    (1, 16, 2000, 777, 128, "fp16"),
    (3, 5, 1500, 4097, 128, "bf16"),
    (8, 8, 2100, 2100, 32, "bf16"),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B%dH%d_q%dk%d_d%d_%s" % c)
def test_stream_matches_oracle(case):
    require_gpu()
    B, H, Nq, Nk, d, dt = case
    note(f"stream parity {case}")
    q, k, v = rand_inputs(B, H, Nq, Nk, d, dt, seed=Nq + 3 * Nk + d)
    o, lse = fa.attention(q.to(DEV), k.to(DEV), v.to(DEV), causal=False, path="stream")
    torch.cuda.synchronize()
    if B * H * Nq <= 40000:
        O, L = oracle.attention(q, k, v, scale=default_scale(d), causal=False)
        compare(o.cpu(), lse.cpu(), O, L, what=f"stream {case}")
    else:
        rng = np.random.default_rng(Nq)
        for (b, h) in ((0, 0), (B - 1, H - 1), (B // 2, H // 2)):
            rows = sorted(set([0, 255, 256, Nq - 1] + [int(x) for x in rng.integers(0, Nq, 40)]))
            O, L = oracle.attention_rows(q, k, v, b, h, rows, scale=default_scale(d), causal=False)
            compare(o[b, h][rows].cpu(), lse[b, h][rows].cpu(), O, L, what=f"stream {case} ({b},{h})")


def test_stream_full_size_80x80_and_auto_choice():
    """yolo80b16 at full size through the stream form: every sampled row of
    three heads matches the oracle. The automatic choice keeps the tiled
    kernel there (3.1 rounds of blocks) and takes the stream form for a
    shape just past one round."""
    require_gpu()
    w = WORKLOADS["yolo80b16"]
    note("stream yolo80b16")
    lib = fa._lib.load()
    assert lib.fa_fwd_stream_advised(w.B, w.H, w.Nq, w.Nk, w.d, 0, 0) == 0
    assert lib.fa_fwd_stream_advised(1, 16, 8448, 8448, 32, 0, 0) == 1   # 528 blocks
    assert lib.fa_fwd_stream_advised(1, 16, 8448, 8448, 32, 0, 1) == 0   # causal: never
    q, k, v = make_inputs(w)
    o, lse = fa.attention(q.to(DEV), k.to(DEV), v.to(DEV), causal=False, scale=w.scale,
                          path="stream")
    o_t, lse_t = fa.attention(q.to(DEV), k.to(DEV), v.to(DEV), causal=False, scale=w.scale,
                              path="tiled")
    torch.cuda.synchronize()
    # the two forms agree closely (only the summation order of split blocks differs)
    assert float((o.float() - o_t.float()).abs().max()) <= 2e-3
    assert float((lse - lse_t).abs().max()) <= 1e-4
    for (b, h) in ((0, 0), (7, 2), (15, 3)):
        rows = list(range(0, w.Nq, 97)) + [w.Nq - 1]
        O, L = oracle.attention_rows(q, k, v, b, h, rows, scale=w.scale, causal=False)
        compare(o[b, h][rows].cpu(), lse[b, h][rows].cpu(), O, L, what=f"yolo80b16 stream ({b},{h})")


def test_stream_rejects_causal_and_is_deterministic():
    require_gpu()
    note("stream causal / determinism")
    q, k, v = (t.to(DEV) for t in rand_inputs(2, 4, 1200, 1300, 64, "fp16", seed=4))
    with pytest.raises(fa.FaError) as e:
        fa.attention(q, k, v, causal=True, path="stream")
    assert e.value.status == fa._lib.FA_ERR_PATH
    a = fa.attention(q, k, v, path="stream")
    b = fa.attention(q, k, v, path="stream")
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    o, lse = fa.attention(q, k, v, path="stream", return_lse=False)
    torch.cuda.synchronize()
    assert lse is None and torch.equal(o, a[0])
