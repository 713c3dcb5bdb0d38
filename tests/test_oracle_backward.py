"""The gradient oracle against its pins, and planted mistakes against the pins.

The mistakes live only in an in-memory copy of oracle/backward.py on the CPU.
"""
import os
import types

import pytest

import oracle
from tests import oracle_bwd_pins as pins

SRC_PATH = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                        "oracle", "backward.py")


@pytest.mark.parametrize("check", pins.ALL_CHECKS, ids=[c.__name__ for c in pins.ALL_CHECKS])
def test_oracle_backward_pin(check):
    check(oracle.backward)


# The code line, not its restatement in the module docstring.
DS_LINE = "dS = P * (dP - D[:, None])\n    dQ"

MUTANTS = [
    ("dv_untransposed", "dV = P.T @ do_h", "dV = P @ do_h"),
    ("dv_from_scores", "dV = P.T @ do_h", "dV = E.T @ do_h"),
    ("dp_with_keys", "dP = do_h @ v_h.T", "dP = do_h @ k_h.T"),
    ("delta_over_columns", "    D = (P * dP).sum(axis=1)\n    dS", "    D = (P * dP).sum(axis=0)\n    dS"),
    ("delta_dropped", DS_LINE, "dS = P * dP\n    dQ"),
    ("delta_sign", DS_LINE, "dS = P * (dP + D[:, None])\n    dQ"),
    ("ds_without_p", DS_LINE, "dS = (dP - D[:, None])\n    dQ"),
    ("dq_no_scale", "dQ = scale * (dS @ k_h)", "dQ = (dS @ k_h)"),
    ("dq_from_values", "dQ = scale * (dS @ k_h)", "dQ = scale * (dS @ v_h)"),
    ("dk_no_scale", "dK = scale * (dS.T @ q_h)", "dK = (dS.T @ q_h)"),
    ("dk_from_do", "dK = scale * (dS.T @ q_h)", "dK = scale * (dS.T @ do_h)"),
    ("no_causal_mask", "        S = apply_causal_mask(S, np.asarray(row_ids))",
     "        S = S"),
    ("unnormalised_p", "    P = E / l[:, None]\n    dV", "    P = E\n    dV"),
    # the row-blocked sampled form
    ("sampled_dv_overwritten", "dV += P[:, keys].T @ do_h[r0:r1]", "dV = P[:, keys].T @ do_h[r0:r1]"),
    ("sampled_mask_block_local", "S = apply_causal_mask(S, np.arange(r0, r1))",
     "S = apply_causal_mask(S, np.arange(0, r1 - r0))"),
    ("sampled_row_selection", "sel = (rows >= r0) & (rows < r1)", "sel = (rows > r0) & (rows < r1)"),
    ("sampled_dk_no_scale", "dK += scale * (dS[:, keys].T @ q_h[r0:r1])", "dK += dS[:, keys].T @ q_h[r0:r1]"),
    ("row_delta_wrong_axis", "return (to_f64(o) * to_f64(do)).sum(axis=-1)",
     "return (to_f64(o) * to_f64(do)).sum(axis=-2)"),
    ("default_scale_wrong", "scale = 1.0 / math.sqrt(d)\n    dQ", "scale = 1.0 / d\n    dQ"),
]


def _load(src: str) -> types.ModuleType:
    src = src.replace("from .definition import", "from oracle.definition import")
    mod = types.ModuleType("oracle_backward_copy")
    exec(compile(src, "oracle_backward_copy", "exec"), mod.__dict__)
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
        assert _failing_checks(_load(f.read())) == []


@pytest.mark.parametrize("name,orig,planted", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(name, orig, planted):
    with open(SRC_PATH, encoding="utf-8") as f:
        src = f.read()
    assert src.count(orig) == 1, f"mutation anchor not unique or missing: {orig!r}"
    failed = _failing_checks(_load(src.replace(orig, planted)))
    assert failed, f"no pin noticed the planted mistake {name}"
