"""Plants one plausible mistake at a time into a copy of the oracle's source
and requires at least one pin in tests/oracle_pins.py to fail on it.

This shows the pins would notice a dropped term, a wrong sign or index, a
transposed operand or a wrong axis anywhere in the oracle. The mistakes live
only in an in-memory copy on the CPU; the oracle file is never modified.
"""
import os
import types

import pytest

from tests import oracle_pins as pins

SRC_PATH = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                        "oracle", "definition.py")

# (name, original text, planted mistake)
MUTANTS = [
    ("dropped_scale", "return scale * (q_h @ k_h.T)", "return (q_h @ k_h.T)"),
    ("scale_squared", "return scale * (q_h @ k_h.T)", "return scale * scale * (q_h @ k_h.T)"),
    ("q_times_q", "return scale * (q_h @ k_h.T)", "return scale * (q_h @ q_h.T)"),
    ("default_scale_1_over_d", "scale = 1.0 / math.sqrt(d)\n    O = np.empty",
     "scale = 1.0 / d\n    O = np.empty"),
    ("causal_reversed", "masked = cols[None, :] > row_ids[:, None]",
     "masked = cols[None, :] < row_ids[:, None]"),
    ("causal_off_by_one", "masked = cols[None, :] > row_ids[:, None]",
     "masked = cols[None, :] > row_ids[:, None] + 1"),
    ("causal_mask_diagonal", "masked = cols[None, :] > row_ids[:, None]",
     "masked = cols[None, :] >= row_ids[:, None]"),
    ("mask_to_zero", "out[masked] = -np.inf", "out[masked] = 0.0"),
    ("max_over_columns", "m = S.max(axis=1)", "m = S.max(axis=0)"),
    ("sum_over_columns", "l = P.sum(axis=1)", "l = P.sum(axis=0)"),
    ("exp2_instead_of_exp", "P = np.exp(S - m[:, None])", "P = np.exp2(S - m[:, None])"),
    ("missing_normalisation", "O = (P @ v_h) / l[:, None]", "O = (P @ v_h)"),
    ("values_from_keys", "O = (P @ v_h) / l[:, None]", "O = (P @ k_h) / l[:, None]"),
    ("lse_without_max", "lse = m + np.log(l)", "lse = np.log(l)"),
    ("lse_log2", "lse = m + np.log(l)", "lse = m + np.log2(l)"),
    ("lse_minus_max", "lse = m + np.log(l)", "lse = -m + np.log(l)"),
    ("row_block_offset_lost", "row_ids=np.arange(r0, r1))", "row_ids=np.arange(0, r1 - r0))"),
    ("rows_ignore_ids", "return attention_head(qh, k[b, h], v[b, h], scale, causal, row_ids=rows)",
     "return attention_head(qh, k[b, h], v[b, h], scale, causal)"),
    ("rows_not_selected", "qh = to_f64(q[b, h])[rows]", "qh = to_f64(q[b, h])[:len(rows)]"),
    ("probabilities_unnormalised", "return P / l[:, None]", "return P"),
]


def _load_mutant(orig: str, planted: str) -> types.ModuleType:
    with open(SRC_PATH, encoding="utf-8") as f:
        src = f.read()
    assert src.count(orig) == 1, f"mutation anchor not unique or missing: {orig!r}"
    mod = types.ModuleType("oracle_mutant")
    exec(compile(src.replace(orig, planted), "oracle_mutant", "exec"), mod.__dict__)
    return mod


def _failing_checks(mod):
    failed = []
    for check in pins.ALL_CHECKS:
        try:
            check(mod)
        except Exception:  # an exception counts as the pin noticing
            failed.append(check.__name__)
    return failed


def test_unmutated_copy_passes_all_pins():
    with open(SRC_PATH, encoding="utf-8") as f:
        src = f.read()
    mod = types.ModuleType("oracle_copy")
    exec(compile(src, "oracle_copy", "exec"), mod.__dict__)
    assert _failing_checks(mod) == []


@pytest.mark.parametrize("name,orig,planted", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(name, orig, planted):
    mod = _load_mutant(orig, planted)
    failed = _failing_checks(mod)
    assert failed, f"no pin noticed the planted mistake {name}"
