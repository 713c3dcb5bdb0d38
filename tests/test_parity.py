"""Parity of the HIP path (through the C ABI) with the fp64 oracle.

Small shapes are compared element by element over the whole output; they span
several query blocks and key tiles and end in ragged tails. The five named
workloads run at their full sizes in the launch configuration the benchmark
times and are compared on every element (for the 16384-token workload: two
whole heads and the first 256 rows of every head), the oracle running on the
host's process pool.
"""
import pytest
import torch

import oracle
from oracle import pool as oracle_pool
from tests.gpu_util import (compare, compare_oracle, default_scale, note, rand_inputs, require_gpu,
                             run_gpu)
from workloads import WORKLOADS, make_inputs

pytestmark = pytest.mark.gpu


SMALL = [
    # (B, H, Nq, Nk, d, dtype, causal)
    (1, 1, 1, 1, 64, "fp16", False),
    (1, 1, 1, 1, 64, "fp16", True),
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
    (1, 1, 33, 1, 32, "fp16", False),      # one key
    (1, 1, 1, 513, 128, "bf16", False),    # one query
]


def short_path_fits(Nk, d):
    return (Nk + 63) // 64 <= (9 if d == 128 else 16)


@pytest.mark.parametrize("path", ["tiled", "short"])
@pytest.mark.parametrize("case", SMALL, ids=lambda c: "B%dH%d_q%dk%d_d%d_%s_%s" % (
    c[0], c[1], c[2], c[3], c[4], c[5], "causal" if c[6] else "full"))
def test_small_shapes(case, path):
    """Each shape through both kernels, whichever the automatic choice is."""
    require_gpu()
    B, H, Nq, Nk, d, dt, causal = case
    if path == "short" and not short_path_fits(Nk, d):
        pytest.skip("key range beyond the short path")
    note(f"parity small {case} path={path}")
    q, k, v = rand_inputs(B, H, Nq, Nk, d, dt, seed=Nq * 1000 + Nk + d)
    o, lse = run_gpu(q, k, v, causal, path=path)
    O, L = oracle.attention(q, k, v, scale=default_scale(d), causal=causal)
    compare(o, lse, O, L, what=f"{case} {path}", vmax=float(v.float().abs().max()))


@pytest.mark.parametrize("d,Nk", [(32, 1024), (64, 1024), (128, 576), (128, 512)])
def test_short_path_at_its_key_limit(d, Nk):
    """The short path at its largest key range (16 or 9 waves per workgroup)."""
    require_gpu()
    note(f"parity short path limit d={d} Nk={Nk}")
    for dt, causal in (("fp16", False), ("bf16", True)):
        q, k, v = rand_inputs(1, 2, 70, Nk, d, dt, seed=d + Nk)
        o, lse = run_gpu(q, k, v, causal, path="short")
        O, L = oracle.attention(q, k, v, scale=default_scale(d), causal=causal)
        compare(o, lse, O, L, what=f"short limit d={d} Nk={Nk} {dt} causal={causal}", vmax=float(v.float().abs().max()))


@pytest.mark.parametrize("scale", [0.0, -0.125, 0.5, 1e-3, 2.0])
def test_scales(scale):
    require_gpu()
    note(f"parity scale {scale}")
    q, k, v = rand_inputs(2, 2, 150, 150, 64, "fp16", seed=77)
    for causal in (False, True):
        O, L = oracle.attention(q, k, v, scale=scale, causal=causal)
        for path in ("tiled", "short"):
            o, lse = run_gpu(q, k, v, causal, scale=scale, path=path)
            compare(o, lse, O, L, what=f"scale={scale} causal={causal} {path}", vmax=float(v.float().abs().max()))


def test_lse_null():
    require_gpu()
    note("parity lse=NULL")
    q, k, v = rand_inputs(1, 2, 200, 200, 64, "bf16", seed=5)
    o, lse = run_gpu(q, k, v, True, with_lse=False)
    assert lse is None
    O, L = oracle.attention(q, k, v, scale=default_scale(64), causal=True)
    compare(o, None, O, L, what="lse=NULL", vmax=float(v.float().abs().max()))


def test_large_logits_tail():
    """Logits of a few hundred (q, k ~ N(0, 8^2)) over a 19x19 map."""
    require_gpu()
    note("parity large logits")
    for d in (32, 64, 128):
        q, k, v = rand_inputs(2, 2, 361, 361, d, "fp16", seed=d, sigma_qk=8.0, v_uniform=True)
        for causal in (False, True):
            O, L = oracle.attention(q, k, v, scale=default_scale(d), causal=causal)
            for path in ("tiled", "short"):
                o, lse = run_gpu(q, k, v, causal, path=path)
                compare(o, lse, O, L, what=f"large logits d={d} causal={causal} {path}", vmax=float(v.float().abs().max()))


@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
def test_reference_raised_midway(d, dtype):
    """Keys whose scores jump far above everything before them, placed in the
    first and in the second 32-key half of different tiles, so the running
    reference maximum has to be raised in the middle of the key range (and
    repeatedly), not only on the first tile."""
    require_gpu()
    note(f"parity raised reference d={d} {dtype}")
    q, k, v = rand_inputs(1, 2, 300, 400, d, dtype, seed=900 + d, v_uniform=True)
    q = (q.float().abs() + 0.5).to(q.dtype)  # every query row sees the jumps
    k = k.float()
    for pos, height in ((37, 2.0), (69, 4.0), (130, 5.0), (230, 7.0), (333, 9.0)):
        k[:, :, pos, :] = height
    k = k.to(q.dtype)
    for causal in (False, True):
        O, L = oracle.attention(q, k, v, scale=default_scale(d), causal=causal)
        for path in ("tiled", "short"):
            o, lse = run_gpu(q, k, v, causal, path=path)
            compare(o, lse, O, L, what=f"raised reference d={d} {dtype} causal={causal} {path}", vmax=float(v.float().abs().max()))


def test_rising_scores():
    """Scores that grow steadily along the keys: the reference falls behind
    on many tiles of every row block."""
    require_gpu()
    note("parity rising scores")
    for d in (32, 64, 128):
        q, k, v = rand_inputs(2, 1, 260, 700, d, "fp16", seed=31 + d, v_uniform=True)
        q = (q.float().abs() * 0.5 + 0.5).to(q.dtype)
        ramp = torch.linspace(0.0, 6.0, 700).view(1, 1, 700, 1)
        k = (k.float() * 0.2 + ramp).to(k.dtype)
        for causal in (False, True):
            o, lse = run_gpu(q, k, v, causal)
            O, L = oracle.attention(q, k, v, scale=default_scale(d), causal=causal)
            compare(o, lse, O, L, what=f"rising scores d={d} causal={causal}", vmax=float(v.float().abs().max()))


@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("dtype,jump", [("fp16", 15.5), ("fp16", 17.0), ("bf16", 100.0),
                                        ("bf16", 140.0)])
def test_jump_near_overflow(d, dtype, jump):
    """One key, past the first tile, whose score exceeds everything before it
    by `jump` (log2 units, i.e. after scale*log2(e)): just below and just
    above where P relative to a reference taken from the first tile stops
    fitting fp16 (2^16) or the fp32 output and row sum (bf16, ~2^127). Below,
    the tiled kernel keeps that reference; above, it must redo the block with
    a raised one. Both must match the oracle."""
    require_gpu()
    note(f"parity jump {jump} d={d} {dtype}")
    N = 300
    q, k, v = rand_inputs(1, 2, N, N, d, dtype, seed=4000 + d, v_uniform=True)
    q = torch.ones_like(q)
    k = (k.float() * 0.01).to(k.dtype)
    c = default_scale(d) * 1.4426950408889634
    k = k.float()
    k[:, :, 150, :] = jump / (c * d)  # score of key 150 (log2 units): jump
    k = k.to(q.dtype)
    for causal in (False, True):
        O, L = oracle.attention(q, k, v, scale=default_scale(d), causal=causal)
        o, lse = run_gpu(q, k, v, causal, path="tiled")
        compare(o, lse, O, L, what=f"jump {jump} d={d} {dtype} causal={causal}", vmax=float(v.float().abs().max()))


@pytest.mark.parametrize("name", ["yolo20", "yolo80b16", "seq2048", "tail361"])
def test_named_workload_full_size(name):
    """Each named workload at full size, in the call the benchmark times,
    compared with the oracle on every element of O and LSE (the oracle runs
    on the host's process pool)."""
    require_gpu()
    w = WORKLOADS[name]
    note(f"parity workload {name}: B={w.B} H={w.H} N={w.Nq} d={w.d} {w.dtype} causal={w.causal}")
    q, k, v = make_inputs(w)
    o, lse = run_gpu(q, k, v, w.causal, scale=w.scale)
    note(f"parity workload {name}: GPU done, oracle on every element")
    compare_oracle(o, lse, q, k, v, w.scale, w.causal, what=name)


def test_long16k_full_heads():
    """The 16384-token causal bf16 workload at full size: every element of two
    whole heads (the first and the last), and the first 256 rows of all 32
    heads, where a causal row sees only a few keys, |O| is largest and the
    bf16 error peaks."""
    require_gpu()
    w = WORKLOADS["long16k"]
    note(f"parity workload long16k: B={w.B} H={w.H} N={w.Nq} d={w.d} {w.dtype} causal={w.causal}")
    q, k, v = make_inputs(w)
    o, lse = run_gpu(q, k, v, w.causal, scale=w.scale)
    assert torch.isfinite(o.float()).all() and torch.isfinite(lse).all()
    vmax = float(v.float().abs().max())
    heads = [(0, 0), (0, w.H - 1)]
    note("parity long16k: whole heads (0,0) and (0,31)")
    O, L = oracle_pool.attention_heads(q, k, v, heads, scale=w.scale, causal=w.causal, row_block=512)
    for i, (b, h) in enumerate(heads):
        compare(o[b, h], lse[b, h], O[i], L[i], what=f"long16k head ({b},{h})", vmax=vmax)
    note("parity long16k: rows 0-255 of every head")
    heads = [(0, h) for h in range(w.H)]
    O, L = oracle_pool.attention_heads(q, k, v, heads, scale=w.scale, causal=w.causal,
                                       rows=range(256), row_block=256)
    compare(o[0, :, :256], lse[0, :, :256], O, L, what="long16k rows 0-255 of 32 heads", vmax=vmax)
