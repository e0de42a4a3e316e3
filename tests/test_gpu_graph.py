"""The library's launches captured in a HIP graph (torch.cuda.CUDAGraph) and
replayed (GPU only).  Captured: fa_fwd, fa_fwd_splitkv with caller-given
workspaces, and fa_bwd_noalloc, the backward meant for callers that cannot
allocate (code under graph capture).  None of them allocates or clears
memory with a memset, so every replay must equal the eager calls bit for
bit; the replays are separated by the program's own eager work and
synchronisations, and one replay runs on new input contents."""
import pytest
import torch

import io_aware_exact_13_amd as fa
import workloads
from gpu_common import announce, device

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def _eager(q, k, v, dout, scale, causal, n_splits):
    o, lse = fa.fwd(q, k, v, scale=scale, causal=causal)
    os_, lses = fa.fwd_splitkv(q, k, v, scale=scale, causal=causal, n_splits=n_splits)
    dq, dk, dv = fa.bwd(q, k, v, o, lse, dout, scale=scale, causal=causal)
    torch.cuda.synchronize()
    return o, lse, os_, lses, dq, dk, dv


@pytest.mark.parametrize("B,H,N,d,causal,n_splits", [(1, 4, 1000, 128, True, 3), (2, 2, 777, 64, False, 4)])
def test_captured_launches_replay_like_eager_calls(B, H, N, d, causal, n_splits):
    dev = device()
    w = workloads.custom(B, H, N, d, causal, seed=8100 + N)
    q, k, v = (t.to(dev) for t in workloads.make_inputs(w))
    dout = workloads.make_grad(w).to(dev)
    w2 = workloads.custom(B, H, N, d, causal, seed=8200 + N)
    q2, k2, v2 = (t.to(dev) for t in workloads.make_inputs(w2))
    announce(f"[graph] {w.name} n_splits={n_splits}")

    ref = _eager(q, k, v, dout, w.scale, causal, n_splits)
    ref2 = _eager(q2, k2, v2, dout, w.scale, causal, n_splits)

    # static buffers the graph reads and writes
    sq, sk, sv = q.clone(), k.clone(), v.clone()
    f32 = dict(dtype=torch.float32, device=dev)
    o, os_ = torch.empty_like(q), torch.empty_like(q)
    lse, lses = torch.empty((B, H, N), **f32), torch.empty((B, H, N), **f32)
    o_part = torch.empty((n_splits, B, H, N, d), **f32)
    lse_part = torch.empty((n_splits, B, H, N), **f32)
    dq, dk, dv = (torch.empty_like(q) for _ in range(3))
    outs = (o, lse, os_, lses, dq, dk, dv)

    def calls():
        fa.fwd(sq, sk, sv, scale=w.scale, causal=causal, out=o, lse=lse)
        fa.fwd_splitkv(sq, sk, sv, scale=w.scale, causal=causal, n_splits=n_splits, out=os_, lse=lses,
                       o_part=o_part, lse_part=lse_part)
        fa.bwd_noalloc(sq, sk, sv, o, lse, dout, dq, dk, dv, scale=w.scale, causal=causal)

    # warm up on a side stream (the no-allocation entry point looks up its
    # device array on its first call on a device), then capture
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        calls()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        calls()
    torch.cuda.synchronize()

    for rep in range(4):
        new_inputs = rep == 2
        src = (q2, k2, v2) if new_inputs else (q, k, v)
        for dst, s in zip((sq, sk, sv), src):
            dst.copy_(s)
        for t in outs:
            t.fill_(7.0)
        # the program's own eager work between replays
        fa.fwd(q2, k2, v2, scale=w.scale, causal=causal)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        want = ref2 if new_inputs else ref
        names = ("o", "lse", "o_splitkv", "lse_splitkv", "dq", "dk", "dv")
        for name, a, b in zip(names, want, outs):
            assert torch.equal(_bits(a), _bits(b)), f"replay {rep}: {name}"
        announce(f"    replay {rep}{' (new inputs)' if new_inputs else ''}: bitwise equal to the eager calls")
