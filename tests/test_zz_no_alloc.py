"""fa_bwd_noalloc, the backward entry point that allocates nothing (its D
workspace is the library's own device array), against fa_bwd (GPU only).
It runs the same kernels, so its gradients must equal fa_bwd's bit for bit."""
import pytest
import torch

import io_aware_exact_13_amd as fa
import workloads
from gpu_common import announce, device

pytestmark = pytest.mark.gpu


def _inputs(B, H, N, d, causal, seed):
    dev = device()
    w = workloads.custom(B, H, N, d, causal, seed=seed)
    q, k, v = (t.to(dev) for t in workloads.make_inputs(w))
    dout = workloads.make_grad(w).to(dev)
    o, lse = fa.fwd(q, k, v, scale=w.scale, causal=causal)
    return w, q, k, v, o, lse, dout


def _check_equal_to_fa_bwd(B, H, N, d, causal, seed):
    w, q, k, v, o, lse, dout = _inputs(B, H, N, d, causal, seed)
    announce(f"[noalloc] {w.name}")
    ref = fa.bwd(q, k, v, o, lse, dout, scale=w.scale, causal=causal)
    got = tuple(torch.full_like(q, 5.0) for _ in range(3))
    fa.bwd_noalloc(q, k, v, o, lse, dout, *got, scale=w.scale, causal=causal)
    torch.cuda.synchronize()
    for name, a, b in zip(("dq", "dk", "dv"), ref, got):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), name


def test_two_calls_in_a_row_the_second_smaller_equal_fa_bwd():
    _check_equal_to_fa_bwd(2, 3, 1000, 128, True, seed=71)
    _check_equal_to_fa_bwd(1, 2, 333, 64, False, seed=72)


def test_largest_accepted_size_equals_fa_bwd():
    # B*H*N = FA_NOALLOC_ROWS exactly: the whole array is used
    _check_equal_to_fa_bwd(1, 32, fa.NOALLOC_ROWS // 32, 64, True, seed=73)


def test_beyond_the_limit_is_rejected_before_any_launch():
    w, q, k, v, o, lse, dout = _inputs(1, 1, 64, 64, False, seed=74)
    outs = [torch.full_like(q, 3.0) for _ in range(3)]
    ptrs = [t.data_ptr() for t in (q, k, v, o, lse, dout, *outs)]
    st = fa.fa_bwd_noalloc(*ptrs, 1, 1, fa.NOALLOC_ROWS + 1, 64, w.scale, 0, None)
    assert st == fa.FA_ERR_SCRATCH
    st = fa.fa_bwd_noalloc(*ptrs, 3, 1, fa.NOALLOC_ROWS // 2, 64, w.scale, 0, None)
    assert st == fa.FA_ERR_SCRATCH
    torch.cuda.synchronize()
    assert all((t == 3.0).all().item() for t in outs)
