"""The HIP gradients (fa_bwd) against the fp64 oracle's (GPU only).

Bar (no tolerance is fixed for the gradients, so it is derived from the
arithmetic): the kernels round P and dS to bf16 (8 significant bits, relative
error <= 2^-8) before the MFMAs and round dQ, dK, dV to bf16 on the way out.
Each alone moves an element by up to 2^-8 of its size.  In a contraction
whose terms have random signs (dV = P^T dO, dK = scale dS^T Q, dQ = scale
dS K) the operand rounding errors add like the terms themselves, so the
relative error of a result is about the rms relative rounding error of one
operand, 2^-8 / sqrt(3) = 2.3e-3, plus the output rounding.  Per tensor the
test requires max|diff| <= 2^-5 max|ref| (8 units of 2^-8) and
mean|diff| <= 2^-7 mean|ref| (2 units, about 3.5 times the expected mean),
against the oracle evaluated on the same bf16 inputs and upstream gradient.
"""
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import io_aware_exact_13_amd as fa
import oracle
import workloads
from gpu_common import (LSE_MAX_ABS, O_MAX_ABS, O_MEAN_ABS, announce, compare_full, device, oracle_threads,
                        row_spans, spans_per_head, to64, variant_bwd)

pytestmark = pytest.mark.gpu

MAX_REL = 2.0 ** -5
MEAN_REL = 2.0 ** -7

SMALL = [
    (1, 1, 256, 64, False),
    (1, 1, 256, 128, True),
    (1, 2, 333, 128, False),
    (2, 1, 300, 64, True),
    (1, 2, 513, 128, True),
    (1, 1, 1, 64, False), (1, 1, 1, 128, True),
    (1, 1, 65, 128, False), (1, 1, 65, 64, True),
    (3, 1, 129, 128, True),
]
# Tile-count edge cases of the gradient loops: the dK/dV kernel walks
# 32-row query tiles and the dQ kernel 64-key tiles, interior tiles in pairs
# and the diagonal, tail and leftover tiles masked.  One, two, three and
# five tiles, exact multiples and ragged tails, several key blocks.
EDGE = [
    (1, 1, 32, 128, True), (1, 1, 32, 64, False),
    (1, 2, 64, 128, False), (2, 1, 96, 64, True),
    (1, 1, 160, 128, True), (1, 1, 192, 128, False),
    (1, 2, 320, 64, True), (1, 1, 384, 128, True),
    (2, 1, 1056, 128, True), (1, 1, 1056, 64, False),
    (1, 1, 1000, 128, False), (1, 2, 777, 64, True),
]


def run_fwd_bwd(q, k, v, do, scale, causal):
    dev = device()
    q, k, v, do = (t.to(dev) for t in (q, k, v, do))
    o, lse = fa.fwd(q, k, v, scale=scale, causal=causal)
    dq, dk, dv = fa.bwd(q, k, v, o, lse, do, scale=scale, causal=causal)
    torch.cuda.synchronize()
    return o, lse, dq, dk, dv


def check_tensor(name, got, ref, quiet=False):
    """Hold one gradient tensor to the bar; returns its two ratios."""
    diff = np.abs(got - ref)
    big = float(np.abs(ref).max())
    mean_ref = float(np.abs(ref).mean())
    r_max = float(diff.max()) / big if big > 0 else float(diff.max())
    r_mean = float(diff.mean()) / mean_ref if mean_ref > 0 else float(diff.mean())
    if not quiet:
        announce(f"    {name}: max|diff|/max|ref|={r_max:.3e}  mean|diff|/mean|ref|={r_mean:.3e}")
    assert np.isfinite(got).all(), name
    assert r_max <= MAX_REL and r_mean <= MEAN_REL, name
    return r_max, r_mean


def _random_shapes(seed, count):
    """Seeded ragged shapes away from the tile multiples the fixed lists favour."""
    rng = np.random.default_rng(seed)
    return [(int(rng.integers(1, 3)), int(rng.integers(1, 3)), int(rng.integers(2, 1500)),
             int(rng.choice([64, 128])), bool(rng.integers(0, 2))) for _ in range(count)]


@pytest.mark.parametrize("B,H,N,d,causal", SMALL + EDGE + _random_shapes(20261205, 8))
def test_small_shapes_match_oracle_gradients(B, H, N, d, causal):
    w = workloads.custom(B, H, N, d, causal, seed=2000 + N + d + int(causal))
    q, k, v = workloads.make_inputs(w)
    do = workloads.make_grad(w)
    announce(f"[bwd-small] {w.name}")
    _, _, dq, dk, dv = run_fwd_bwd(q, k, v, do, w.scale, causal)
    rq, rk, rv = oracle.attention_bwd(to64(q), to64(k), to64(v), to64(do), w.scale, causal)
    if N == 1:
        # one key: dV = dO exactly (P = 1 rounds to 1), while dQ and dK are
        # scale dS (K or Q) with dS = P (dP - D) the difference of two fp32
        # evaluations of one dot product: zero up to fp32 rounding
        assert np.array_equal(to64(dv), to64(do))
        assert float(dq.abs().max()) <= 1e-4 and float(dk.abs().max()) <= 1e-4
        return
    for name, got, ref in (("dQ", dq, rq), ("dK", dk, rk), ("dV", dv, rv)):
        check_tensor(name, to64(got), ref)


@pytest.mark.parametrize("name", ["causal_b1h32_n16384_d128", "mid_b4h16_n4096_d128", "short_b16h32_n2048_d64",
                                  "causal_peaky_b1h8_n65536_d128"])
def test_full_size_gradients_every_head(name):
    """Full sizes, every element: the oracle recomputes dQ, dK and dV of every
    head (all rows), each held to the bar per head, and the gradients are
    bitwise equal run to run."""
    w = workloads.WORKLOADS[name]
    announce(f"[bwd-full] {name}: generating inputs")
    q, k, v = workloads.make_inputs(w)
    do = workloads.make_grad(w)
    announce(f"[bwd-full] {name}: running fa_fwd + fa_bwd twice")
    _, _, dq, dk, dv = run_fwd_bwd(q, k, v, do, w.scale, w.causal)
    again = run_fwd_bwd(q, k, v, do, w.scale, w.causal)[2:]
    # bitwise equal run to run: a race would show here even inside the tolerance
    for x, y in zip((dq, dk, dv), again):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))
    del again
    for t in (dq, dk, dv):
        assert torch.isfinite(t).all()
    dq, dk, dv = dq.cpu(), dk.cpu(), dv.cpu()

    def part(bh, r0, r1):
        b, h = divmod(bh, w.H)
        return oracle.attention_bwd_span(to64(q[b, h]), to64(k[b, h]), to64(v[b, h]), to64(do[b, h]), w.scale,
                                         w.causal, r0, r1)

    worst = {"dQ": [0.0, 0.0], "dK": [0.0, 0.0], "dV": [0.0, 0.0]}
    n_heads = w.B * w.H

    def check_heads(futures, spans):
        for bh in range(n_heads):
            b, h = divmod(bh, w.H)
            rq, rk, rv = (np.zeros((w.N, w.d)) for _ in range(3))
            for (r0, r1), f in zip(spans, futures[bh]):
                sq, sk, sv = f.result()
                rq[r0:r1] = sq
                rk[:sk.shape[0]] += sk
                rv[:sv.shape[0]] += sv
            futures[bh] = None
            for tn, got, ref in (("dQ", dq[b, h], rq), ("dK", dk[b, h], rk), ("dV", dv[b, h], rv)):
                r_max, r_mean = check_tensor(f"{tn}[{b},{h}]", to64(got), ref, quiet=True)
                worst[tn] = [max(worst[tn][0], r_max), max(worst[tn][1], r_mean)]
            if bh % 16 == 15 or bh == n_heads - 1:
                announce(f"[bwd-full] {name}: {bh + 1} heads within the bar")

    with oracle_threads() as workers, ThreadPoolExecutor(workers) as ex:
        # each head's query rows in spans of similar work, one task each; a
        # head's dQ is its spans' rows, its dK and dV the sums of their shares
        spans = row_spans(w.N, w.causal, spans_per_head(n_heads, w.N, workers))
        futures = [[ex.submit(part, bh, r0, r1) for r0, r1 in spans] for bh in range(n_heads)]
        try:
            check_heads(futures, spans)
        finally:
            for fs in futures:
                for f in fs or ():
                    f.cancel()
    for tn, (r_max, r_mean) in worst.items():
        announce(f"    {tn}, worst head: max|diff|/max|ref|={r_max:.3e}  mean|diff|/mean|ref|={r_mean:.3e}")


def test_gradient_special_cases():
    dev = device()
    w = workloads.custom(1, 2, 200, 128, True, seed=77)
    q, k, v = workloads.make_inputs(w)
    do = workloads.make_grad(w)
    # V = 0: dP = 0 and O = 0, so dS = 0 and dQ, dK vanish exactly
    _, _, dq, dk, dv = run_fwd_bwd(q, k, torch.zeros_like(v), do, w.scale, True)
    assert torch.all(dq == 0) and torch.all(dk == 0)
    # Q = 0 without the mask: dK = scale dS^T Q vanishes exactly; dV rows are all the mean of dO
    _, _, dq, dk, dv = run_fwd_bwd(torch.zeros_like(q), k, v, do, w.scale, False)
    assert torch.all(dk == 0)
    mean_do = to64(do).mean(axis=2, keepdims=True)
    assert np.abs(to64(dv) - mean_do).max() <= 2.0 ** -7 * np.abs(mean_do).max() + 1e-6
    # causal row 0 sees one key with weight 1: its dQ row is (nearly) zero
    _, _, dq, _, _ = run_fwd_bwd(q, k, v, do, w.scale, True)
    assert float(dq[:, :, 0].abs().max()) <= 1e-3 * float(dq.abs().max())
    del dev


def test_gradients_are_bitwise_deterministic():
    w = workloads.custom(2, 2, 700, 128, True, seed=78)
    q, k, v = workloads.make_inputs(w)
    do = workloads.make_grad(w)
    a = run_fwd_bwd(q, k, v, do, w.scale, True)[2:]
    b = run_fwd_bwd(q, k, v, do, w.scale, True)[2:]
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))


@pytest.mark.parametrize("B,H,N,d,causal,workload", [
    (2, 3, 777, 128, True, None), (1, 3, 333, 64, False, None), (1, 2, 1000, 64, True, None),
    (3, 1, 1025, 128, True, None), (1, 2, 4096, 128, False, None), (0, 0, 0, 0, False, "causal_b1h32_n16384_d128")])
def test_extra_barrier_build_gradients_are_bitwise_equal(B, H, N, d, causal, workload):
    """The gradient kernels' race-check build waits for every memory
    operation and holds a workgroup barrier after each tile's LDS reads, so no
    wave can refill a double buffer another wave may still read.  Its
    gradients must equal the default build's bit for bit."""
    dev = device()
    w = workloads.WORKLOADS[workload] if workload else workloads.custom(B, H, N, d, causal, seed=6100 + N)
    announce(f"[bwd racecheck] {w.name}")
    q, k, v = (t.to(dev) for t in workloads.make_inputs(w))
    do = workloads.make_grad(w).to(dev)
    o, lse = fa.fwd(q, k, v, scale=w.scale, causal=w.causal)
    ref = fa.bwd(q, k, v, o, lse, do, scale=w.scale, causal=w.causal)
    got = variant_bwd("bwdracecheck", q, k, v, o, lse, do, w.scale, w.causal)
    for name, a, b in zip(("dq", "dk", "dv"), ref, got):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), name


def test_long_sequence_gradients():
    """A 32K-token causal head: dK and dV of the whole head and sampled dQ rows."""
    w = workloads.custom(1, 1, 32768, 128, True, seed=5100)
    q, k, v = workloads.make_inputs(w)
    do = workloads.make_grad(w)
    announce(f"[bwd-long] {w.name}: running fa_fwd + fa_bwd")
    _, _, dq, dk, dv = run_fwd_bwd(q, k, v, do, w.scale, True)
    announce(f"[bwd-long] {w.name}: oracle")
    rq, rk, rv = oracle.attention_bwd_head(to64(q[0, 0]), to64(k[0, 0]), to64(v[0, 0]), to64(do[0, 0]), w.scale,
                                           True)
    for tn, got, ref in (("dQ", dq[0, 0], rq), ("dK", dk[0, 0], rk), ("dV", dv[0, 0], rv)):
        check_tensor(tn, to64(got), ref)


def test_many_heads_forward_and_gradients_on_sampled_heads():
    """65536 heads of 160 rows (a ragged key tile each, causal): the largest
    grids of the forward and both gradient kernels, and head offsets past
    2^31 bytes into each 2.7 GB tensor.  Six heads (the first, the last and
    four others) against the oracle on every element: dQ, dK and dV to the
    gradients' bar; LSE and mean|dO| to the forward's bar outright, and O to
    1e-2 beyond its own bf16 rounding, since the first rows of a causal head
    average a few values of V, where |O| can pass 4 and half a bf16 ulp of the
    stored O (2^-6 there) is itself more than 1e-2."""
    w = workloads.custom(4, 16384, 160, 128, True, seed=5300)
    assert w.B * w.H * w.N * w.d * 2 > 2 ** 31
    announce(f"[many-heads] {w.name}: generating inputs")
    q, k, v = workloads.make_inputs(w)
    do = workloads.make_grad(w)
    announce(f"[many-heads] {w.name}: running fa_fwd + fa_bwd")
    o, lse, dq, dk, dv = run_fwd_bwd(q, k, v, do, w.scale, True)
    for t in (o, lse, dq, dk, dv):
        assert torch.isfinite(t.float()).all()
    rng = np.random.default_rng(5300)
    heads = [(0, 0), (w.B - 1, w.H - 1)] + [(int(rng.integers(w.B)), int(rng.integers(w.H))) for _ in range(4)]
    for b, h in heads:
        sl = (slice(b, b + 1), slice(h, h + 1))
        beyond, me, ml, mo = compare_full(q[sl], k[sl], v[sl], w.scale, True, o[sl].cpu(), lse[sl].cpu(),
                                          with_rounding=True)
        announce(f"    head ({b},{h}): max|dO|={mo:.3e} (beyond O's rounding {beyond:.3e}) mean|dO|={me:.3e} "
                 f"max|dLSE|={ml:.3e}")
        assert beyond <= O_MAX_ABS and me <= O_MEAN_ABS and ml <= LSE_MAX_ABS
        refs = oracle.attention_bwd_head(to64(q[b, h]), to64(k[b, h]), to64(v[b, h]), to64(do[b, h]), w.scale, True)
        for tn, got, ref in zip(("dQ", "dK", "dV"), (dq[b, h], dk[b, h], dv[b, h]), refs):
            check_tensor(f"{tn}[{b},{h}]", to64(got), ref)


@pytest.mark.parametrize("B,H,N,d,causal", [(2, 3, 333, 128, True), (1, 2, 300, 64, False)])
def test_autograd_attention_matches_the_direct_calls(B, H, N, d, causal):
    """fa.attention under autograd gives fa_fwd's O and, on backward, fa_bwd's
    gradients bit for bit, also when the upstream gradient reaches it as a
    non-contiguous view (the loss taken through a transpose)."""
    dev = device()
    w = workloads.custom(B, H, N, d, causal, seed=9100 + N)
    base = [t.to(dev) for t in workloads.make_inputs(w)]
    do = workloads.make_grad(w).to(dev)
    ro, rl = fa.fwd(*base, scale=w.scale, causal=causal)
    ref = fa.bwd(*base, ro, rl, do, scale=w.scale, causal=causal)
    for through_transpose in (False, True):
        q, k, v = (t.clone().requires_grad_() for t in base)
        o = fa.attention(q, k, v, causal=causal)
        if through_transpose:
            loss = (o.transpose(1, 2).float() * do.transpose(1, 2).float()).sum()
        else:
            loss = (o.float() * do.float()).sum()
        loss.backward()
        torch.cuda.synchronize()
        assert torch.equal(o.detach().view(torch.int16), ro.view(torch.int16))
        for name, got, want in zip(("dq", "dk", "dv"), (q.grad, k.grad, v.grad), ref):
            assert torch.equal(got.view(torch.int16), want.view(torch.int16)), (name, through_transpose)
