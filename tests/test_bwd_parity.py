"""Parity of the backward kernels (through the C ABI) with the fp64 gradient oracle.

Each case runs the GPU forward (O and LSE, as a training step would), then
the GPU backward for a seeded upstream gradient dO, and compares dQ, dK, dV
element by element with oracle.attention_backward on the same fp16/bf16
inputs.

Tolerance. The kernels round P and dS to the input type before the matrix
products (as the forward rounds P) and round the gradients to it at the end;
every sum runs in fp32. With u the unit roundoff of the input type (2^-11
fp16, 2^-8 bf16), that puts the error of each gradient at a few u relative to
its own scale. An fp32 emulation of exactly these roundings against the fp64
oracle, over the shapes of the five named workloads, gave at most 1.0u of
max|ref| for the largest error and 4.2u of mean|ref| for the mean error. The
test allows 4u and 8u:
    max|d| <= 4u * max|ref| + 1e-4     mean|d| <= 8u * mean|ref| + 1e-5
(the absolute floors only matter for gradients that vanish, e.g. dQ and dK at
scale 0 or with a single key).
"""
import numpy as np
import pytest
import torch

import exact_attention_23_amd as fa
import oracle
from tests.gpu_util import default_scale, note, rand_inputs, require_gpu
from workloads import WORKLOADS, make_grad, make_inputs

pytestmark = pytest.mark.gpu

UNIT_ROUNDOFF = {torch.float16: 2.0 ** -11, torch.bfloat16: 2.0 ** -8}


def grad_like(q, seed):
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    return torch.randn(q.shape, generator=g, dtype=torch.float32).to(q.dtype).contiguous()


def run_bwd(q, k, v, do, causal, scale):
    dev = torch.device("cuda:0")
    qd, kd, vd, dod = q.to(dev), k.to(dev), v.to(dev), do.to(dev)
    o, lse = fa.attention(qd, kd, vd, causal=causal, scale=scale)
    dq, dk, dv = fa.attention_backward(qd, kd, vd, o, dod, lse, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return dq.cpu(), dk.cpu(), dv.cpu()


def compare_grads(got, ref, dtype, what=""):
    u = UNIT_ROUNDOFF[dtype]
    out = []
    for name, g, r in zip(("dQ", "dK", "dV"), got, ref):
        g = g.double().numpy()
        assert np.all(np.isfinite(g)), f"{what} {name}: non-finite gradient"
        d = np.abs(g - r)
        max_d, mean_d = float(d.max()), float(d.mean())
        max_r, mean_r = float(np.abs(r).max()), float(np.abs(r).mean())
        worst = tuple(int(x) for x in np.unravel_index(int(d.argmax()), d.shape))
        msg = (f"{what} {name}: max|d|={max_d:.3e} at {worst} (max|ref|={max_r:.3e}, "
               f"{max_d / max(max_r, 1e-30) / u:.2f}u) mean|d|={mean_d:.3e} "
               f"(mean|ref|={mean_r:.3e}, {mean_d / max(mean_r, 1e-30) / u:.2f}u)")
        assert max_d <= 4 * u * max_r + 1e-4, msg
        assert mean_d <= 8 * u * mean_r + 1e-5, msg
        out.append((max_d, mean_d))
    return out


SMALL = [
    # (B, H, Nq, Nk, d, dtype, causal)
    (1, 1, 1, 1, 64, "fp16", False),
    (1, 1, 1, 1, 32, "bf16", True),
    (1, 2, 2, 2, 32, "fp16", True),
    (2, 1, 15, 15, 64, "fp16", False),
    (1, 2, 17, 17, 128, "bf16", True),
    (1, 1, 31, 33, 32, "bf16", False),
    (2, 2, 63, 63, 64, "fp16", True),
    (1, 1, 64, 64, 128, "fp16", False),
    (1, 3, 65, 65, 32, "fp16", True),
    (1, 1, 127, 129, 64, "bf16", False),
    (1, 2, 128, 128, 64, "fp16", True),
    (2, 1, 129, 129, 128, "bf16", True),
    (1, 2, 255, 257, 32, "fp16", False),
    (1, 1, 257, 255, 32, "bf16", True),
    (3, 2, 361, 361, 64, "fp16", False),
    (1, 2, 400, 400, 64, "bf16", True),
    (1, 1, 1000, 1000, 128, "fp16", True),
    (1, 1, 1000, 1000, 32, "bf16", False),
    (2, 2, 100, 700, 64, "fp16", False),   # Nq < Nk
    (1, 2, 700, 100, 64, "fp16", True),    # Nq > Nk, causal
    (1, 2, 100, 700, 128, "bf16", True),   # Nq < Nk, causal: keys past Nq get zero gradients
    (1, 1, 33, 1, 32, "fp16", False),      # one key
    (1, 1, 1, 513, 128, "bf16", False),    # one query
]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: "B%dH%d_q%dk%d_d%d_%s_%s" % (
    c[0], c[1], c[2], c[3], c[4], c[5], "causal" if c[6] else "full"))
def test_bwd_small_shapes(case):
    require_gpu()
    B, H, Nq, Nk, d, dt, causal = case
    note(f"bwd parity small {case}")
    q, k, v = rand_inputs(B, H, Nq, Nk, d, dt, seed=Nq * 1000 + Nk + d)
    do = grad_like(q, seed=Nq * 7 + Nk * 3 + d)
    scale = default_scale(d)
    got = run_bwd(q, k, v, do, causal, scale)
    ref = oracle.attention_backward(q, k, v, do, scale=scale, causal=causal)
    compare_grads(got, ref, q.dtype, what=str(case))


@pytest.mark.parametrize("scale", [0.0, -0.125, 0.5, 2.0])
def test_bwd_scales(scale):
    require_gpu()
    note(f"bwd parity scale {scale}")
    q, k, v = rand_inputs(2, 2, 150, 170, 64, "fp16", seed=78)
    do = grad_like(q, seed=79)
    for causal in (False, True):
        got = run_bwd(q, k, v, do, causal, scale)
        ref = oracle.attention_backward(q, k, v, do, scale=scale, causal=causal)
        compare_grads(got, ref, q.dtype, what=f"scale={scale} causal={causal}")


def test_bwd_large_logits_tail():
    """q, k ~ N(0, 8^2) over a 19x19 map: nearly one-hot rows of P."""
    require_gpu()
    note("bwd parity large logits")
    for d in (32, 64, 128):
        q, k, v = rand_inputs(2, 2, 361, 361, d, "fp16", seed=d, sigma_qk=8.0, v_uniform=True)
        do = grad_like(q, seed=d + 1)
        for causal in (False, True):
            got = run_bwd(q, k, v, do, causal, default_scale(d))
            ref = oracle.attention_backward(q, k, v, do, scale=default_scale(d), causal=causal)
            compare_grads(got, ref, q.dtype, what=f"large logits d={d} causal={causal}")


def test_bwd_deterministic():
    """No atomics: two calls give bitwise-equal gradients."""
    require_gpu()
    note("bwd determinism")
    dev = torch.device("cuda:0")
    q, k, v = (t.to(dev) for t in rand_inputs(2, 3, 300, 500, 64, "bf16", seed=5))
    do = grad_like(q.cpu(), seed=6).to(dev)
    o, lse = fa.attention(q, k, v, causal=True)
    a = fa.attention_backward(q, k, v, o, do, lse, causal=True)
    b = fa.attention_backward(q, k, v, o, do, lse, causal=True)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_autograd_function_matches_oracle():
    """flash_attention under torch.autograd: the gradients of a loss reach
    q, k, v through the backward kernels."""
    require_gpu()
    note("bwd autograd function")
    dev = torch.device("cuda:0")
    q, k, v = rand_inputs(1, 2, 200, 260, 64, "fp16", seed=12)
    do = grad_like(q, seed=13)
    qd, kd, vd = (t.to(dev).requires_grad_(True) for t in (q, k, v))
    o = fa.flash_attention(qd, kd, vd, causal=True)
    o.backward(do.to(dev))
    torch.cuda.synchronize()
    ref = oracle.attention_backward(q, k, v, do, scale=default_scale(64), causal=True)
    compare_grads((qd.grad.cpu(), kd.grad.cpu(), vd.grad.cpu()), ref, q.dtype, what="autograd")


@pytest.mark.parametrize("name", ["yolo20", "tail361", "yolo80b16", "seq2048"])
def test_bwd_named_workload_full_size(name):
    """The named workloads at full size (the call the benchmark times); for
    the large ones a few whole heads are compared (dK and dV of a head depend
    on all its query rows)."""
    require_gpu()
    w = WORKLOADS[name]
    note(f"bwd parity workload {name}: B={w.B} H={w.H} N={w.Nq} d={w.d} {w.dtype} causal={w.causal}")
    q, k, v = make_inputs(w)
    do = make_grad(w)
    got = run_bwd(q, k, v, do, w.causal, w.scale)
    for g in got:
        assert torch.isfinite(g.float()).all()
    if w.B * w.H * w.Nq <= 8 * 2 * 400:
        ref = oracle.attention_backward(q, k, v, do, scale=w.scale, causal=w.causal)
        compare_grads(got, ref, q.dtype, what=name)
        return
    rng = np.random.default_rng(w.seed)
    heads = sorted(set([(0, 0), (w.B - 1, w.H - 1), (int(rng.integers(0, w.B)), int(rng.integers(0, w.H)))]))
    for (b, h) in heads:
        ref = oracle.attention_backward_head(q[b, h], k[b, h], v[b, h], do[b, h], w.scale, w.causal)
        compare_grads(tuple(g[b, h] for g in got), ref, q.dtype, what=f"{name} head ({b},{h})")


def _raw_bwd_args(q, k, v, o, do, lse, dq, dk, dv, ws, causal, scale):
    B, H, Nq, d = q.shape
    return (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(), lse.data_ptr(),
            dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), ws.data_ptr(), ws.numel(),
            B, H, Nq, k.shape[2], d, float(scale), 1 if causal else 0, fa._dtype_code(q))


def test_bwd_kernels_on_two_streams():
    """The documented split: FA_BWD_PRE, then FA_BWD_DKDV and FA_BWD_DQ on two
    streams that both wait for it, gives the bits of one fa_bwd call."""
    require_gpu()
    note("bwd two streams")
    from exact_attention_23_amd import _lib

    dev = torch.device("cuda:0")
    for d, dt in ((64, "fp16"), (128, "bf16")):
        q, k, v = (t.to(dev) for t in rand_inputs(2, 3, 333, 517, d, dt, seed=d + 9))
        do = grad_like(q.cpu(), seed=d + 10).to(dev)
        o, lse = fa.attention(q, k, v, causal=True)
        ref = fa.attention_backward(q, k, v, o, do, lse, causal=True)
        dq, dk, dv = (torch.full_like(t, float("nan")) for t in (q, k, v))
        ws = torch.empty(fa.fa_bwd_workspace_bytes(2, 3, 333), dtype=torch.uint8, device=dev)
        args = _raw_bwd_args(q, k, v, o, do, lse, dq, dk, dv, ws, True, default_scale(d))
        lib = _lib.load()
        main = torch.cuda.current_stream()
        s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
        assert lib.fa_bwd_ex(*args, _lib.FA_BWD_PRE, main.cuda_stream) == 0
        s1.wait_stream(main)
        s2.wait_stream(main)
        assert lib.fa_bwd_ex(*args, _lib.FA_BWD_DKDV, s1.cuda_stream) == 0
        assert lib.fa_bwd_ex(*args, _lib.FA_BWD_DQ, s2.cuda_stream) == 0
        main.wait_stream(s1)
        main.wait_stream(s2)
        torch.cuda.synchronize()
        for x, y, n in zip((dq, dk, dv), ref, ("dq", "dk", "dv")):
            assert torch.equal(x, y), f"d={d}: {n} differs from one fa_bwd call"


def test_bwd_graph_replay_matches_eager():
    """The backward captured in a HIP graph gives the eager bits on every
    replay, with eager work and synchronisation between replays."""
    require_gpu()
    note("bwd graph replay")
    dev = torch.device("cuda:0")
    q, k, v = (t.to(dev) for t in rand_inputs(2, 2, 300, 400, 64, "fp16", seed=21))
    do = grad_like(q.cpu(), seed=22).to(dev)
    o, lse = fa.attention(q, k, v, causal=True)
    ref = fa.attention_backward(q, k, v, o, do, lse, causal=True)
    dq, dk, dv = (torch.empty_like(t) for t in (q, k, v))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fa.attention_backward(q, k, v, o, do, lse, causal=True, dq=dq, dk=dk, dv=dv)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(2):
            fa.attention_backward(q, k, v, o, do, lse, causal=True, dq=dq, dk=dk, dv=dv)
    for rep in range(4):
        for t in (dq, dk, dv):
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for x, y, n in zip((dq, dk, dv), ref, ("dq", "dk", "dv")):
            assert torch.equal(x, y), f"replay {rep}: {n} differs"
        fa.attention_backward(q, k, v, o, do, lse, causal=False)  # eager work between replays
        torch.cuda.synchronize()


def test_bwd_long16k_full_size_sampled():
    """The 16384-token causal bf16 workload at full size (the d = 128
    backward kernels: 8-wave workgroups, K rows in LDS): dQ of sampled rows
    and dK, dV of sampled keys of one head, from the row-blocked gradient
    oracle (tens of seconds of CPU)."""
    require_gpu()
    w = WORKLOADS["long16k"]
    note(f"bwd parity workload long16k: B={w.B} H={w.H} N={w.Nq} d={w.d} {w.dtype} causal={w.causal}")
    q, k, v = make_inputs(w)
    do = make_grad(w)
    got = run_bwd(q, k, v, do, w.causal, w.scale)
    for g in got:
        assert torch.isfinite(g.float()).all()
    rng = np.random.default_rng(w.seed)
    picks = sorted(set([0, 1, 63, 64, 255, 256, 8191, 16382, 16383] +
                       [int(x) for x in rng.integers(0, w.Nq, 24)]))
    for h in (w.H - 1,):
        dq, dk, dv = oracle.attention_backward_sampled(q[0, h], k[0, h], v[0, h], do[0, h], w.scale,
                                                       w.causal, picks, picks, row_block=2048)
        compare_grads((got[0][0, h][picks], got[1][0, h][picks], got[2][0, h][picks]),
                      (dq, dk, dv), q.dtype, what=f"long16k head {h}")
