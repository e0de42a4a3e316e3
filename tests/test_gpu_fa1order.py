"""The K/V-outer (FA1) loop order ablation (fa_fwd_fa1order) against the
fp64 oracle with the forward's bar: both orders compute the same function
(GPU only)."""
import pytest
import torch

import io_aware_exact_13_amd as fa
import workloads
from gpu_common import O_MAX_ABS, O_MEAN_ABS, LSE_MAX_ABS, announce, compare_all_heads, compare_full, device

pytestmark = pytest.mark.gpu

CASES = [
    (1, 1, 256, 64, False),
    (1, 2, 333, 128, False),
    (2, 1, 700, 64, True),
    (1, 3, 513, 128, True),
    (1, 1, 1, 128, True),
    (1, 1, 65, 64, False),
]


@pytest.mark.parametrize("B,H,N,d,causal", CASES)
def test_fa1_order_matches_oracle(B, H, N, d, causal):
    dev = device()
    w = workloads.custom(B, H, N, d, causal, seed=4000 + N + d)
    q, k, v = workloads.make_inputs(w)
    announce(f"[fa1order] {w.name}")
    o, lse = fa.fwd_fa1order(q.to(dev), k.to(dev), v.to(dev), scale=w.scale, causal=causal)
    torch.cuda.synchronize()
    mo, me, ml = compare_full(q, k, v, w.scale, causal, o, lse)
    announce(f"    max|dO|={mo:.3e} mean|dO|={me:.3e} max|dLSE|={ml:.3e}")
    assert mo <= O_MAX_ABS and me <= O_MEAN_ABS and ml <= LSE_MAX_ABS


def test_fa1_order_agrees_with_fa2_order_at_size():
    dev = device()
    w = workloads.WORKLOADS["mid_b4h16_n4096_d128"]
    q, k, v = (t.to(dev) for t in workloads.make_inputs(w))
    o1, l1 = fa.fwd_fa1order(q, k, v, scale=w.scale, causal=w.causal)
    o2, l2 = fa.fwd(q, k, v, scale=w.scale, causal=w.causal)
    torch.cuda.synchronize()
    d_o = float((o1.float() - o2.float()).abs().max())
    d_l = float((l1 - l2).abs().max())
    announce(f"[fa1order] {w.name} vs fa_fwd: max|dO|={d_o:.3e} max|dLSE|={d_l:.3e}")
    assert d_o <= O_MAX_ABS and d_l <= LSE_MAX_ABS
    mo, me, ml, _ = compare_all_heads(*(t.cpu() for t in (q, k, v)), w.scale, w.causal, o1.cpu(), l1.cpu())
    announce(f"    every element vs the oracle: max|dO|={mo:.3e} mean|dO|={me:.3e} max|dLSE|={ml:.3e}")
    assert mo <= O_MAX_ABS and me <= O_MEAN_ABS and ml <= LSE_MAX_ABS
