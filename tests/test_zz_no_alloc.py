"""fa_bwd_noalloc, the backward entry point that allocates nothing (its D/LSE
records live in the library's static scratch), against fa_bwd, the entry
point with a caller workspace, through the C ABI. Two calls in a row, the
second with smaller inputs (and another head width, type and mask), so the
second runs over scratch the first left behind. Both entry points run the
same kernels in a fixed order, so the gradients must agree bit for bit, which
is stronger than the parity bar."""
import pytest
import torch

import exact_attention_23_amd as fa
from tests.gpu_util import note, rand_inputs, require_gpu

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def _check(B, H, Nq, Nk, d, dtype, causal, seed):
    note(f"no-alloc backward B={B} H={H} Nq={Nq} Nk={Nk} d={d} {dtype} causal={causal}")
    q, k, v = (t.to(DEV) for t in rand_inputs(B, H, Nq, Nk, d, dtype, seed=seed))
    g = torch.Generator(device="cpu").manual_seed(seed + 1)
    do = torch.randn((B, H, Nq, d), generator=g).to(q.dtype).to(DEV)
    scale = d ** -0.5
    o, lse = fa.attention(q, k, v, causal=causal, scale=scale)
    dq, dk, dv = fa.attention_backward(q, k, v, o, do, lse, causal=causal, scale=scale)
    gq, gk, gv = (torch.full_like(t, float("nan")) for t in (q, k, v))
    code = fa._dtype_code(q)
    st = fa.fa_bwd_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(),
                           lse.data_ptr(), gq.data_ptr(), gk.data_ptr(), gv.data_ptr(), B, H, Nq, Nk,
                           d, scale, 1 if causal else 0, code, fa._current_stream(0))
    assert st == 0, fa.status_str(st)
    torch.cuda.synchronize()
    for name, a, b in (("dq", gq, dq), ("dk", gk, dk), ("dv", gv, dv)):
        assert torch.equal(a, b), f"{name} differs from fa_bwd: max {float((a.float() - b.float()).abs().max())}"


def test_noalloc_backward_equals_fa_bwd_twice():
    require_gpu()
    _check(2, 3, 700, 650, 64, "fp16", True, seed=61)
    _check(1, 2, 200, 333, 128, "bf16", False, seed=62)  # smaller, over the first call's scratch
