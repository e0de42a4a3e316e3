"""The seeded input generator: shapes, determinism, value structure (no GPU)."""
import math

import torch

import workloads


def test_five_workloads_have_the_stated_shapes():
    w = workloads.WORKLOADS
    assert [(x.B, x.H, x.N, x.d, x.causal) for x in w.values()] == [
        (1, 1, 256, 64, False), (4, 16, 4096, 128, False), (1, 32, 16384, 128, True),
        (16, 32, 2048, 64, False), (1, 8, 65536, 128, True)]
    assert [x.seed for x in w.values()] == [1, 2, 3, 4, 5]
    assert workloads.HEADLINE == "causal_b1h32_n16384_d128"
    assert all(x.scale == 1.0 / math.sqrt(x.d) for x in w.values())


def test_generator_is_deterministic_and_bf16():
    w = workloads.custom(2, 3, 100, 64, False, seed=11)
    a = workloads.make_inputs(w)
    b = workloads.make_inputs(w)
    for x, y in zip(a, b):
        assert x.dtype == torch.bfloat16 and x.shape == (2, 3, 100, 64) and x.is_contiguous()
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))
    assert workloads.sha256_of(a[0]) == workloads.sha256_of(b[0])
    c = workloads.make_inputs(w, seed=12)
    assert not torch.equal(a[0], c[0])


def test_peaky_keys_structure():
    w = workloads.custom(1, 2, 1000, 64, True, seed=5, peaky=True)
    q, k, v = workloads.make_inputs(w)
    # 1% of key rows per head are 8x larger than the rest (std ~4 vs ~0.5)
    for h in range(2):
        norms = k[0, h].float().pow(2).mean(dim=1).sqrt()
        hot = (norms > 2.0).sum().item()
        assert hot == 10
    assert 0.4 < q.float().std().item() < 0.6
    assert 0.4 < v.float().std().item() < 0.6


def test_peaky_workload_moves_the_reference_maximum():
    """The peaky causal workload must exercise the accumulator rescale: count
    the query rows (first 4096 of head 0, keys in 64-key blocks as the kernel
    walks them) whose running maximum grows after the first block, and those
    whose reference moves under a lag of up to 8 in log2 units (the kernel's
    rule).  Both counts are reported; the second must not be zero."""
    import numpy as np
    from streaming_model import reference_moves
    w = workloads.WORKLOADS["causal_peaky_b1h8_n65536_d128"]
    q, k, _ = workloads.make_inputs(w)
    n = 4096
    qh = q[0, 0, :n].double().numpy()
    kh = k[0, 0, :n].double().numpy()
    plain = reference_moves(qh, kh, w.scale, True, 64, 0.0)
    lazy = reference_moves(qh, kh, w.scale, True, 64, 8.0)
    print(f"\nrows with a growing maximum after the first tile: {int((plain > 0).sum())} of {n}; "
          f"rows whose lagging reference moves: {int((lazy > 0).sum())} ({int(lazy.sum())} moves)")
    assert (plain > 0).sum() > 0
    assert (lazy > 0).sum() > 0
