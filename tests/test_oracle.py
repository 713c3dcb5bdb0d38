"""The oracle against its pins (see tests/oracle_pins.py)."""
import pytest

import oracle.definition as ora
from tests import oracle_pins as pins


@pytest.mark.parametrize("check", pins.ALL_CHECKS, ids=lambda f: f.__name__)
def test_oracle_pin(check):
    check(ora)


def test_oracle_rejects_bad_shapes():
    import numpy as np

    with pytest.raises(ValueError):
        ora.attention(np.zeros((1, 1, 0, 4)), np.zeros((1, 1, 3, 4)), np.zeros((1, 1, 3, 4)))
    with pytest.raises(ValueError):
        ora.attention(np.zeros((1, 1, 2, 4)), np.zeros((1, 1, 3, 5)), np.zeros((1, 1, 3, 5)))


def test_oracle_large_logits_finite():
    """Logits near 400 in magnitude (the 19x19 tail workload's range) stay finite."""
    import numpy as np

    rng = np.random.default_rng(0)
    q = rng.standard_normal((1, 1, 8, 64)) * 8
    k = rng.standard_normal((1, 1, 8, 64)) * 8
    v = rng.uniform(-1, 1, (1, 1, 8, 64))
    O, L = ora.attention(q, k, v)
    assert np.all(np.isfinite(O)) and np.all(np.isfinite(L))
    assert np.max(np.abs(L)) > 50  # really in the large-logit regime
    assert np.all(np.abs(O) <= 1.0 + 1e-12)  # convex combination of rows in [-1, 1]
