"""Pins of the oracle's attention gradients (CPU only)."""
import numpy as np
import pytest

import oracle
import pins_bwd


@pytest.mark.parametrize("check", pins_bwd.ALL_BWD_CHECKS, ids=lambda c: c.__name__)
def test_bwd_pin(check):
    check(oracle)


def test_row_sampler_matches_the_full_gradient():
    rng = np.random.default_rng(9)
    q, k, v, do = (rng.normal(size=(1, 1, 200, 32)) for _ in range(4))
    for causal in (False, True):
        dq, _, _ = oracle.attention_bwd(q, k, v, do, 0.2, causal)
        rows = [0, 1, 77, 199]
        got = oracle.attention_bwd_rows(q[0, 0], k[0, 0], v[0, 0], do[0, 0], 0.2, causal, rows)
        assert np.abs(got - dq[0, 0, rows]).max() <= 1e-13
