"""Seeded synthetic attention inputs.

This module draws the random Q, K, V tensors that both the HIP path and the
oracle consume. It holds no attention arithmetic: only shapes, seeds and value
distributions.

The five named workloads are the attention calls the cited articles describe:
  * a YOLO C2PSA/PSA attention over a flattened 20x20 feature map
    (YOLO11 FlashAttention-2 replacement article, kwkr.cn, sections 1.1 and 2.2;
    the map is flattened to a 400-long sequence),
  * batched YOLO inference over an 80x80 map (same article, section 1.1 and 4.2:
    a 6400-long sequence, batch 16),
  * a transformer layer at sequence 2048 with hidden size 1024, causal
    ("FlashAttention 深度解读", usage example with q, k, v of shape
    (32, 2048, 1024) and causal=True; read here as 16 heads of width 64),
  * a long-context causal head set at 16384 tokens (same page, benefits table:
    the longest sequence it quotes),
  * a 19x19 tail map whose length is not a multiple of 8 (YOLO11 article,
    section 4.2, on sequence lengths that are not multiples of 8), with large
    logits to stress the max subtraction that "FlashAttention 深度解读"
    describes under its precision-handling section.
No dataset or trained weight is used; these tensors stand in for those calls.
"""
from __future__ import annotations

import dataclasses
import hashlib
from typing import Dict, Optional, Tuple

import torch

DTYPES = {"fp16": torch.float16, "bf16": torch.bfloat16}


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    Nq: int
    Nk: int
    d: int
    dtype: str  # "fp16" | "bf16"
    causal: bool
    # value distributions: ("normal", sigma) or ("uniform", half_width)
    q_dist: Tuple[str, float] = ("normal", 1.0)
    k_dist: Tuple[str, float] = ("normal", 1.0)
    v_dist: Tuple[str, float] = ("normal", 1.0)
    seed: int = 0

    @property
    def torch_dtype(self) -> torch.dtype:
        return DTYPES[self.dtype]

    @property
    def scale(self) -> float:
        # softmax scale used for every named workload: 1/sqrt(head width)
        return float(self.d) ** -0.5

    def flops(self) -> float:
        """Nominal FLOP count: 4*B*H*Nq*Nk*d, halved when causal."""
        f = 4.0 * self.B * self.H * self.Nq * self.Nk * self.d
        return f / 2.0 if self.causal else f

    def algorithmic_bytes(self) -> int:
        """Bytes read and written once: Q, K, V, O in the storage dtype + LSE fp32."""
        es = 2
        return (es * self.B * self.H * (2 * self.Nq * self.d + 2 * self.Nk * self.d)
                + 4 * self.B * self.H * self.Nq)

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS: Dict[str, Workload] = {
    "yolo20": Workload("yolo20", 1, 2, 400, 400, 64, "fp16", False, seed=1001),
    "yolo80b16": Workload("yolo80b16", 16, 4, 6400, 6400, 32, "fp16", False, seed=1002),
    "seq2048": Workload("seq2048", 32, 16, 2048, 2048, 64, "fp16", True, seed=1003),
    "long16k": Workload("long16k", 1, 32, 16384, 16384, 128, "bf16", True, seed=1004),
    "tail361": Workload("tail361", 8, 2, 361, 361, 64, "fp16", False,
                        q_dist=("normal", 8.0), k_dist=("normal", 8.0),
                        v_dist=("uniform", 1.0), seed=1005),
}
# the order the workloads are listed in
WORKLOAD_ORDER = ["yolo20", "yolo80b16", "seq2048", "long16k", "tail361"]


def _draw(gen: torch.Generator, shape, dist: Tuple[str, float]) -> torch.Tensor:
    kind, p = dist
    if kind == "normal":
        return torch.randn(shape, generator=gen, dtype=torch.float32) * p
    if kind == "uniform":
        return (torch.rand(shape, generator=gen, dtype=torch.float32) * 2.0 - 1.0) * p
    raise ValueError(f"unknown distribution {kind!r}")


def make_inputs(w: Workload, seed: Optional[int] = None):
    """Draw (q, k, v) on the CPU in w's storage dtype, contiguous [B,H,N,d].

    q, then k, then v are drawn in float32 from one torch CPU generator seeded
    with `seed` (default w.seed) and rounded to the storage dtype
    (round-to-nearest-even, torch's conversion).
    """
    g = torch.Generator(device="cpu")
    g.manual_seed(w.seed if seed is None else seed)
    q = _draw(g, (w.B, w.H, w.Nq, w.d), w.q_dist).to(w.torch_dtype)
    k = _draw(g, (w.B, w.H, w.Nk, w.d), w.k_dist).to(w.torch_dtype)
    v = _draw(g, (w.B, w.H, w.Nk, w.d), w.v_dist).to(w.torch_dtype)
    return q.contiguous(), k.contiguous(), v.contiguous()


FP8_MAX = 448.0  # largest finite e4m3 ("fn") value


def make_inputs_fp8(w: Workload, seed: Optional[int] = None):
    """The same float32 draws as make_inputs (q, then k, then v from one
    generator), quantised per tensor to e4m3 the usual way: descale =
    max|x| / 448 in float32, stored = e4m3(x / descale) (round to nearest even,
    torch's conversion). Returns (q8, k8, v8, q_descale, k_descale, v_descale);
    element x of q8 stands for q_descale * x."""
    g = torch.Generator(device="cpu")
    g.manual_seed(w.seed if seed is None else seed)
    out = []
    scales = []
    for shape, dist in (((w.B, w.H, w.Nq, w.d), w.q_dist), ((w.B, w.H, w.Nk, w.d), w.k_dist),
                        ((w.B, w.H, w.Nk, w.d), w.v_dist)):
        x = _draw(g, shape, dist)
        amax = float(x.abs().max())
        s = torch.tensor(amax / FP8_MAX if amax > 0 else 1.0, dtype=torch.float32)
        out.append((x / s).to(torch.float8_e4m3fn).contiguous())
        scales.append(float(s))
    return tuple(out) + tuple(scales)


def dequantize_fp8(x8: torch.Tensor, descale: float) -> torch.Tensor:
    """The values an e4m3 tensor stands for, exactly, in float64."""
    return x8.to(torch.float64) * float(torch.tensor(descale, dtype=torch.float32))


# Offset between a workload's input seed and the seed of its upstream gradient.
GRAD_SEED_OFFSET = 500_000


def make_grad(w: Workload, seed: Optional[int] = None) -> torch.Tensor:
    """Draw the upstream gradient dO for the backward pass: [B,H,Nq,d] iid
    N(0, 1) in float32 from its own torch CPU generator (seeded with
    (seed or w.seed) + GRAD_SEED_OFFSET), rounded to w's storage dtype."""
    g = torch.Generator(device="cpu")
    g.manual_seed((w.seed if seed is None else seed) + GRAD_SEED_OFFSET)
    return _draw(g, (w.B, w.H, w.Nq, w.d), ("normal", 1.0)).to(w.torch_dtype).contiguous()


def sha256(t: torch.Tensor) -> str:
    """sha256 of a CPU tensor's raw bytes (for recording which inputs ran)."""
    t = t.detach().cpu().contiguous()
    return hashlib.sha256(t.view(torch.uint8).numpy().tobytes()).hexdigest()
