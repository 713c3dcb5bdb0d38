"""Properties of the HIP path that hold at any size: determinism, streams,
and invariants of attention replayed on the GPU."""
import numpy as np
import pytest
import torch

import exact_attention_23_amd as fa
from tests.gpu_util import note, rand_inputs, require_gpu

pytestmark = pytest.mark.gpu


def test_bitwise_deterministic_and_stream_independent():
    require_gpu()
    note("determinism")
    dev = torch.device("cuda:0")
    for (d, dt, causal) in [(32, "fp16", False), (64, "fp16", True), (128, "bf16", True)]:
        q, k, v = (t.to(dev) for t in rand_inputs(2, 3, 517, 517, d, dt, seed=d))
        o1, l1 = fa.attention(q, k, v, causal=causal)
        o2, l2 = fa.attention(q, k, v, causal=causal)
        s = torch.cuda.Stream()
        with torch.cuda.stream(s):
            o3, l3 = fa.attention(q, k, v, causal=causal)
        s.synchronize()
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(l1, l2)
        assert torch.equal(o1, o3) and torch.equal(l1, l3)


def test_identical_v_rows_give_that_row():
    require_gpu()
    note("identical V rows")
    dev = torch.device("cuda:0")
    q, k, v = rand_inputs(1, 2, 300, 300, 64, "fp16", seed=3)
    v[:] = v[:, :, :1, :]
    o, _ = fa.attention(q.to(dev), k.to(dev), v.to(dev), causal=False)
    torch.cuda.synchronize()
    ref = v[:, :, :1, :].float().expand(-1, -1, 300, -1)
    assert (o.cpu().float() - ref).abs().max().item() <= 2e-3


def test_identical_k_rows_give_mean_v():
    require_gpu()
    note("identical K rows")
    dev = torch.device("cuda:0")
    q, k, v = rand_inputs(1, 1, 200, 200, 32, "bf16", seed=4)
    k[:] = k[:, :, :1, :]
    o, lse = fa.attention(q.to(dev), k.to(dev), v.to(dev), causal=True)
    torch.cuda.synchronize()
    vf = v[0, 0].double()
    prefix = torch.cumsum(vf, 0) / torch.arange(1, 201, dtype=torch.float64)[:, None]
    assert (o[0, 0].cpu().double() - prefix).abs().max().item() <= 1e-2


def test_key_value_permutation():
    require_gpu()
    note("permutation")
    dev = torch.device("cuda:0")
    q, k, v = rand_inputs(1, 2, 257, 333, 64, "fp16", seed=6)
    perm = torch.randperm(333, generator=torch.Generator().manual_seed(1))
    o1, l1 = fa.attention(q.to(dev), k.to(dev), v.to(dev))
    o2, l2 = fa.attention(q.to(dev), k[:, :, perm].contiguous().to(dev),
                          v[:, :, perm].contiguous().to(dev))
    torch.cuda.synchronize()
    assert (o1.float() - o2.float()).abs().max().item() <= 2e-3
    assert (l1 - l2).abs().max().item() <= 1e-4


def test_causal_first_row_is_first_value_exactly():
    require_gpu()
    note("causal row 0")
    dev = torch.device("cuda:0")
    for d, dt in [(32, "fp16"), (64, "bf16"), (128, "fp16")]:
        q, k, v = rand_inputs(2, 2, 150, 150, d, dt, seed=d + 1)
        o, lse = fa.attention(q.to(dev), k.to(dev), v.to(dev), causal=True)
        torch.cuda.synchronize()
        assert torch.equal(o[:, :, 0].cpu(), v[:, :, 0])
        s00 = (q[:, :, 0].double() * k[:, :, 0].double()).sum(-1) / np.sqrt(d)
        assert (lse[:, :, 0].cpu().double() - s00).abs().max().item() <= 1e-3


def test_output_only_written_in_bounds():
    """Guard bytes around o and lse stay untouched (ragged tails, many blocks)."""
    require_gpu()
    note("bounds")
    dev = torch.device("cuda:0")
    B, H, N, d = 2, 3, 333, 64
    q, k, v = (t.to(dev) for t in rand_inputs(B, H, N, N, d, "fp16", seed=9))
    n_o = B * H * N * d
    big = torch.full((n_o + 4096,), 7.0, dtype=torch.float16, device=dev)
    out = big[2048:2048 + n_o].view(B, H, N, d)
    lbig = torch.full((B * H * N + 128,), 5.0, dtype=torch.float32, device=dev)
    lse = lbig[64:64 + B * H * N].view(B, H, N)
    fa.attention(q, k, v, causal=True, out=out, lse=lse)
    torch.cuda.synchronize()
    assert torch.all(big[:2048] == 7.0) and torch.all(big[2048 + n_o:] == 7.0)
    assert torch.all(lbig[:64] == 5.0) and torch.all(lbig[64 + B * H * N:] == 5.0)


def test_graph_replay_matches_eager():
    """Calls captured in a HIP graph give the eager result on every replay,
    with eager work and synchronisation between the replays (both paths)."""
    require_gpu()
    note("graph replay")
    import torch

    import exact_attention_23_amd as fa

    dev = torch.device("cuda:0")
    for path, (Nq, Nk) in (("short", (200, 300)), ("tiled", (300, 500))):
        q, k, v = (t.to(dev) for t in rand_inputs(2, 2, Nq, Nk, 64, "fp16", seed=Nk))
        o = torch.empty_like(q)
        lse = torch.empty((2, 2, Nq), dtype=torch.float32, device=dev)
        o_ref, lse_ref = fa.attention(q, k, v, causal=True, path=path)
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            fa.attention(q, k, v, causal=True, out=o, lse=lse, path=path)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for _ in range(3):
                fa.attention(q, k, v, causal=True, out=o, lse=lse, path=path)
        for rep in range(4):
            o.zero_()
            lse.fill_(float("nan"))
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            assert torch.equal(o, o_ref), f"{path}: replay {rep} output differs"
            assert torch.equal(lse, lse_ref), f"{path}: replay {rep} LSE differs"
            fa.attention(q, k, v, causal=False, path=path)  # eager work between replays
