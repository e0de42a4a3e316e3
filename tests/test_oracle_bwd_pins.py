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


def test_row_spans_reassemble_the_whole_head():
    """Spans that cover every query row once, at ragged boundaries and with
    blocks that cut across them, give the whole head's dQ rows and, summed,
    its dK and dV (the whole-head function is itself one span)."""
    rng = np.random.default_rng(10)
    q, k, v, do = (rng.normal(size=(203, 16)) for _ in range(4))
    for causal in (False, True):
        want = oracle.attention_bwd_head(q, k, v, do, 0.3, causal)
        bounds = [0, 1, 50, 64, 130, 203]
        dq = np.zeros_like(q)
        dk = np.zeros_like(k)
        dv = np.zeros_like(v)
        for r0, r1 in zip(bounds[:-1], bounds[1:]):
            sq, sk, sv = oracle.attention_bwd_span(q, k, v, do, 0.3, causal, r0, r1, row_block=24)
            assert sq.shape == (r1 - r0, 16) and sk.shape == sv.shape == ((r1 if causal else 203), 16)
            dq[r0:r1] = sq
            dk[:sk.shape[0]] += sk
            dv[:sv.shape[0]] += sv
        for got, ref in zip((dq, dk, dv), want):
            assert np.abs(got - ref).max() <= 1e-12 * max(1.0, np.abs(ref).max())
