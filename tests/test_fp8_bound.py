"""The E4M3 bound the FP8 GPU test holds the kernel to, checked on the CPU:
the oracle's FP8 attention (P rounded to E4M3 against the running maximum)
stays within it for any key blocking, and a wrong rounding does not."""
import numpy as np
import pytest

import workloads
from gpu_common import e4m3_p_bounds
from oracle import fp8 as ofp8


def _head(N, d, causal, seed):
    w = workloads.custom(1, 1, N, d, causal, seed=seed)
    q, k, v = workloads.make_inputs(w)
    signs = workloads.make_fp8_signs(w.seed, d)
    deq = []
    for x, rot in ((q, d == 128), (k, d == 128), (v, False)):
        c, _, s = ofp8.quantize_heads(x.float().numpy(), rot, signs if rot else 0)
        deq.append(ofp8.dequantize_heads(c, s)[0, 0])
    return w, deq


@pytest.mark.parametrize("N,d,causal", [(700, 128, True), (513, 64, False), (1000, 64, True)])
@pytest.mark.parametrize("tile", [16, 64, 256])
def test_oracle_fp8_attention_is_within_the_bound_for_any_blocking(N, d, causal, tile):
    w, (qd, kd, vd) = _head(N, d, causal, seed=7100 + N + d)
    rows = np.arange(N)
    o8, l8 = ofp8.attention_fp8_head_rows(qd, kd, vd, w.scale, causal, rows, tile=tile)
    ro, rl, bound, var = e4m3_p_bounds(qd, kd, vd, w.scale, causal, rows)
    diff = np.abs(o8 - ro)
    assert (diff <= bound + 1e-12).all()
    assert (diff * diff).sum() <= var.sum()
    assert np.abs(l8 - rl).max() <= 1e-12          # the LSE adds unrounded P


def test_a_coarser_rounding_of_p_breaks_the_bound():
    """P rounded to 2 mantissa bits instead of 3 (errors up to 2^-3 P): both
    the per-element bound and the mean square check catch it."""
    w, (qd, kd, vd) = _head(700, 128, True, seed=7200)
    rows = np.arange(700)
    s = w.scale * (qd @ kd.T)
    s = np.where(np.arange(700)[None, :] > rows[:, None], -np.inf, s)
    p = np.exp(s - s.max(axis=1, keepdims=True))
    e = np.floor(np.log2(np.maximum(p, 1e-300))).astype(int)
    coarse = np.where(p > 0, np.ldexp(np.round(np.ldexp(p, 2 - e)), e - 2), 0.0)
    o_bad = (coarse @ vd) / p.sum(axis=1, keepdims=True)
    ro, _, bound, var = e4m3_p_bounds(qd, kd, vd, w.scale, True, rows)
    diff = np.abs(o_bad - ro)
    assert (diff > bound).any()
    assert (diff * diff).sum() > var.sum()
