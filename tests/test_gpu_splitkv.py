"""The split-KV forward (fa_fwd_splitkv) against the fp64 oracle, with the
forward's bar: it computes the same function as fa_fwd (GPU only)."""
import math

import numpy as np
import pytest
import torch

import io_aware_exact_13_amd as fa
import workloads
from gpu_common import (O_MAX_ABS, O_MEAN_ABS, LSE_MAX_ABS, announce, compare_all_heads, compare_full, device,
                        to64)

pytestmark = pytest.mark.gpu

CASES = [
    (1, 1, 256, 64, False, 4),
    (1, 2, 333, 128, False, 3),
    (2, 1, 1000, 64, True, 5),
    (1, 3, 700, 128, True, 2),
    (1, 1, 100, 64, True, 7),      # two key tiles, seven ranges: most ranges are empty
    (1, 1, 1, 128, False, 3),
    (1, 2, 513, 128, True, 1),
]


def run_split(q, k, v, scale, causal, n_splits):
    dev = device()
    o, lse = fa.fwd_splitkv(q.to(dev), k.to(dev), v.to(dev), scale=scale, causal=causal, n_splits=n_splits)
    torch.cuda.synchronize()
    return o, lse


def _random_cases(seed, count):
    rng = np.random.default_rng(seed)
    return [(int(rng.integers(1, 3)), int(rng.integers(1, 3)), int(rng.integers(1, 1600)),
             int(rng.choice([64, 128])), bool(rng.integers(0, 2)), int(rng.integers(1, 9)))
            for _ in range(count)]


@pytest.mark.parametrize("B,H,N,d,causal,n_splits", CASES + _random_cases(20261204, 8))
def test_small_shapes_match_oracle(B, H, N, d, causal, n_splits):
    w = workloads.custom(B, H, N, d, causal, seed=3000 + N + d + n_splits)
    q, k, v = workloads.make_inputs(w)
    announce(f"[splitkv] {w.name} n_splits={n_splits}")
    o, lse = run_split(q, k, v, w.scale, causal, n_splits)
    mo, me, ml = compare_full(q, k, v, w.scale, causal, o, lse)
    announce(f"    max|dO|={mo:.3e} mean|dO|={me:.3e} max|dLSE|={ml:.3e}")
    assert mo <= O_MAX_ABS and me <= O_MEAN_ABS and ml <= LSE_MAX_ABS


def test_one_gpu_share_of_the_16k_causal_workload():
    """The headline shape with 4 of its 32 heads (one GPU's share over 8 GPUs)
    at the planned split count: every element against the oracle, and every
    element against fa_fwd (the same function, another summation order)."""
    dev = device()
    w = workloads.custom(1, 4, 16384, 128, True, seed=3)
    q, k, v = workloads.make_inputs(w)
    n = fa.fa_fwd_splitkv_plan(1, 4, 16384, 128, 1)[0]
    announce(f"[splitkv-share] {w.name} n_splits={n}")
    o, lse = run_split(q, k, v, w.scale, True, n)
    mo, me, ml, _ = compare_all_heads(q, k, v, w.scale, True, o.cpu(), lse.cpu())
    announce(f"    every element: max|dO|={mo:.3e} mean|dO|={me:.3e} max|dLSE|={ml:.3e}")
    assert mo <= O_MAX_ABS and me <= O_MEAN_ABS and ml <= LSE_MAX_ABS
    o1, lse1 = fa.fwd(q.to(dev), k.to(dev), v.to(dev), scale=w.scale, causal=True)
    torch.cuda.synchronize()
    d_o = float((o.float() - o1.float()).abs().max())
    d_l = float((lse - lse1).abs().max())
    announce(f"    vs fa_fwd: max|dO|={d_o:.3e} max|dLSE|={d_l:.3e}")
    assert d_o <= O_MAX_ABS and d_l <= LSE_MAX_ABS


@pytest.mark.parametrize("B,H,N,d,causal", [(1, 1, 65536, 128, True), (1, 1, 32768, 64, False)])
def test_one_long_head_every_element(B, H, N, d, causal):
    """The case split-KV is for: one head, a long sequence, far fewer query
    blocks than CUs.  At the planned split count, every element against the
    oracle and the bitwise run-to-run check."""
    dev = device()
    w = workloads.custom(B, H, N, d, causal, seed=3300 + d)
    q, k, v = workloads.make_inputs(w)
    n = fa.fa_fwd_splitkv_plan(B, H, N, d, int(causal))[0]
    announce(f"[splitkv-long] {w.name} n_splits={n}")
    assert n > 1
    o, lse = run_split(q, k, v, w.scale, causal, n)
    o2, lse2 = run_split(q, k, v, w.scale, causal, n)
    assert torch.equal(o.view(torch.int16), o2.view(torch.int16)) and torch.equal(lse, lse2)
    mo, me, ml, _ = compare_all_heads(q, k, v, w.scale, causal, o.cpu(), lse.cpu())
    announce(f"    every element: max|dO|={mo:.3e} mean|dO|={me:.3e} max|dLSE|={ml:.3e}")
    assert mo <= O_MAX_ABS and me <= O_MEAN_ABS and ml <= LSE_MAX_ABS
    del dev


def test_splitkv_is_bitwise_deterministic():
    w = workloads.custom(1, 2, 900, 128, True, seed=91)
    q, k, v = workloads.make_inputs(w)
    a = run_split(q, k, v, w.scale, True, 3)
    b = run_split(q, k, v, w.scale, True, 3)
    assert torch.equal(a[0].view(torch.int16), b[0].view(torch.int16))
    assert torch.equal(a[1], b[1])


@pytest.mark.parametrize("B,H,N,d,causal,n_splits", [(1, 2, 300, 128, True, 5), (1, 2, 300, 64, True, 5),
                                                     (2, 1, 700, 64, True, 7), (1, 1, 130, 128, False, 4),
                                                     (1, 2, 100, 64, False, 7)])
def test_partials_of_rows_without_a_visible_key_are_exact_zeros(B, H, N, d, causal, n_splits):
    """A range that holds no key a row may see (more ranges than key tiles)
    must give that row exactly O_s = 0 and LSE_s = -inf (it drops out of the
    two-block merge of the online softmax); under the causal mask, ranges a
    short query block does not have (it gets fewer than n_splits) are neither
    written nor read; and no partial anywhere may hold a NaN (the running
    statistics of a row start at -inf and must not form (-inf) - (-inf))."""
    dev = device()
    w = workloads.custom(B, H, N, d, causal, seed=4000 + N + d)
    q, k, v = (t.to(dev) for t in workloads.make_inputs(w))
    o_part = torch.full((n_splits, B, H, N, d), 7.0, dtype=torch.float32, device=dev)
    lse_part = torch.full((n_splits, B, H, N), 7.0, dtype=torch.float32, device=dev)
    o, lse = fa.fwd_splitkv(q, k, v, scale=w.scale, causal=causal, n_splits=n_splits, o_part=o_part,
                            lse_part=lse_part)
    torch.cuda.synchronize()
    op, lp = o_part.cpu(), lse_part.cpu()
    assert not torch.isnan(op).any().item() and not torch.isnan(lp).any().item()
    br, kc = fa.fa_fwd_tile(B, H, N, d, int(causal))[:2]
    r = fa.fa_fwd_splitkv_ranges(B, H, N, d, int(causal), n_splits)   # > 0: block b has ceil((b + 1) / r)
    n_empty = n_unused = 0
    for i in range(N):
        q0 = (i // br) * br
        tiles = -(-(min(N, q0 + br) if causal else N) // kc)
        n_ranges = (i // br + r) // r if r > 0 else n_splits
        for s in range(n_splits):
            if s >= n_ranges:    # no such range: the workspace is left as it was
                n_unused += 1
                assert (op[s, :, :, i] == 7.0).all().item() and (lp[s, :, :, i] == 7.0).all().item()
                continue
            j0, j1 = s * tiles // n_ranges, (s + 1) * tiles // n_ranges
            visible = j0 < j1 and (not causal or j0 * kc <= i)
            if visible:
                assert torch.isfinite(op[s, :, :, i]).all().item() and torch.isfinite(lp[s, :, :, i]).all().item()
            else:
                n_empty += 1
                assert (op[s, :, :, i] == 0).all().item() and (lp[s, :, :, i] == -math.inf).all().item()
    announce(f"[splitkv-empty] {w.name} n_splits={n_splits}: {n_empty} (row, range) pairs with no visible key, "
             f"{n_unused} past the row's ranges")
    assert n_empty + n_unused > 0
    mo, me, ml = compare_full(*(t.cpu() for t in (q, k, v)), w.scale, causal, o, lse)
    assert mo <= O_MAX_ABS and me <= O_MEAN_ABS and ml <= LSE_MAX_ABS
