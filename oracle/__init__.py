"""The oracle: plain, slow, CPU float64 exact attention.

TEST INFRASTRUCTURE ONLY. Nothing on the product path imports this package:
only the tests, the smoke check and the benchmark's CPU-baseline leg may use
it. It shares no code with the HIP kernels or their C-ABI.

Every function here is pinned: the forward (definition.py) by
tests/test_oracle.py (brute force on tiny inputs, closed forms, hand-derived
fixtures under tests/golden/, invariants of the definition, and the CPU
float64 scaled_dot_product_attention of PyTorch), the gradients (backward.py)
by tests/test_oracle_backward.py (central finite differences of the forward,
float64 autograd of a plain PyTorch attention, closed forms and invariants).
No function is "parity unpinned".
"""
from .definition import (  # noqa: F401
    to_f64,
    scores,
    apply_causal_mask,
    softmax_stats,
    probabilities,
    attention_head,
    attention,
    attention_rows,
)
from .backward import (  # noqa: F401
    attention_backward_head,
    attention_backward,
    attention_backward_sampled,
    row_delta,
)
