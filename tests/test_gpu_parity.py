"""The HIP path against the fp64 oracle, element by element (GPU only)."""
import json
import math
import os
import time

import numpy as np
import pytest
import torch

import io_aware_exact_13_amd as fa
import workloads
from gpu_common import (O_MAX_ABS, O_MEAN_ABS, LSE_MAX_ABS, announce, compare_all_heads, compare_full,
                        compare_rows, device, run_gpu, sample_picks, to64, variant_fwd, variant_fwd_splitkv)

pytestmark = pytest.mark.gpu


def log_parity(name, mo, me, ml, beyond):
    """Append one workload's figures to the JSON-lines file FA_PARITY_LOG names (if set)."""
    path = os.environ.get("FA_PARITY_LOG")
    if path:
        with open(path, "a") as f:
            f.write(json.dumps({"workload": name, "max_abs_dO": mo, "mean_abs_dO": me, "max_abs_dLSE": ml,
                                "max_dO_beyond_bf16_rounding": beyond}) + "\n")

# Small shapes the oracle finishes in seconds: several query blocks (128 rows)
# and key tiles (64 keys), ragged tails, both head dims, with and without mask.
SMALL = [
    (1, 1, 256, 64, False),
    (1, 1, 256, 64, True),
    (2, 3, 333, 128, False),
    (1, 2, 1000, 64, True),
    (1, 3, 700, 128, True),
    (2, 2, 513, 128, False),
    (1, 1, 1, 64, False), (1, 1, 1, 128, True),
    (1, 2, 7, 64, True), (1, 2, 7, 128, False),
    (1, 1, 65, 64, False), (1, 1, 65, 128, True),
    (1, 1, 129, 128, False), (1, 1, 129, 64, True),
    (3, 1, 1025, 128, True),
]


@pytest.mark.parametrize("B,H,N,d,causal", SMALL)
def test_small_shapes_match_oracle_everywhere(B, H, N, d, causal):
    w = workloads.custom(B, H, N, d, causal, seed=1000 + N + d + int(causal))
    q, k, v = workloads.make_inputs(w)
    announce(f"[parity-small] {w.name}")
    o, lse = run_gpu(q, k, v, w.scale, causal)
    mo, me, ml = compare_full(q, k, v, w.scale, causal, o, lse)
    announce(f"    max|dO|={mo:.3e} mean|dO|={me:.3e} max|dLSE|={ml:.3e}")
    assert mo <= O_MAX_ABS and me <= O_MEAN_ABS and ml <= LSE_MAX_ABS


def _random_shapes(seed, count):
    """Seeded ragged shapes away from the tile multiples the fixed list favours."""
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(count):
        B, H = int(rng.integers(1, 3)), int(rng.integers(1, 3))
        N = int(rng.integers(1, 1600))
        out.append((B, H, N, int(rng.choice([64, 128])), bool(rng.integers(0, 2))))
    return out


@pytest.mark.parametrize("B,H,N,d,causal", _random_shapes(20261203, 16))
def test_random_shapes_match_oracle_everywhere(B, H, N, d, causal):
    w = workloads.custom(B, H, N, d, causal, seed=5000 + N)
    q, k, v = workloads.make_inputs(w)
    announce(f"[parity-random] {w.name}")
    o, lse = run_gpu(q, k, v, w.scale, causal)
    mo, me, ml = compare_full(q, k, v, w.scale, causal, o, lse)
    announce(f"    max|dO|={mo:.3e} mean|dO|={me:.3e} max|dLSE|={ml:.3e}")
    assert mo <= O_MAX_ABS and me <= O_MEAN_ABS and ml <= LSE_MAX_ABS


def test_tiny_workload_full_compare():
    w = workloads.WORKLOADS["tiny_b1h1_n256_d64"]
    q, k, v = workloads.make_inputs(w)
    o, lse = run_gpu(q, k, v, w.scale, w.causal)
    mo, me, ml = compare_full(q, k, v, w.scale, w.causal, o, lse)
    announce(f"[parity] {w.name}: max|dO|={mo:.3e} mean|dO|={me:.3e} max|dLSE|={ml:.3e}")
    assert mo <= O_MAX_ABS and me <= O_MEAN_ABS and ml <= LSE_MAX_ABS


@pytest.mark.parametrize("name", [n for n in workloads.WORKLOAD_ORDER if n != "tiny_b1h1_n256_d64"])
def test_full_size_workloads_every_element(name):
    """Full sizes, in the launch the benchmark times: every element of O and
    LSE of every head against the oracle, held to the bar outright (mean over
    the whole tensor); the output is also bitwise equal run to run."""
    w = workloads.WORKLOADS[name]
    announce(f"[parity-full] {name}: generating inputs")
    q, k, v = workloads.make_inputs(w)
    announce(f"[parity-full] {name}: running fa_fwd twice")
    dev = device()
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    o, lse = run_gpu(qd, kd, vd, w.scale, w.causal)
    o2, l2 = run_gpu(qd, kd, vd, w.scale, w.causal)
    # bitwise equal run to run: a race between waves would show here even
    # where its error stayed inside the tolerance below
    assert torch.equal(o.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(lse.view(torch.int32), l2.view(torch.int32))
    del qd, kd, vd, o2, l2
    o, lse = o.cpu(), lse.cpu()
    announce(f"[parity-full] {name}: oracle over all {w.B * w.H} heads")
    t0 = time.perf_counter()
    mo, me, ml, beyond = compare_all_heads(q, k, v, w.scale, w.causal, o, lse)
    announce(f"[parity-full] {name}: max|dO|={mo:.3e} mean|dO|={me:.3e} max|dLSE|={ml:.3e} "
             f"(max|dO| beyond O's bf16 rounding {beyond:.3e}; oracle {time.perf_counter() - t0:.1f} s)")
    log_parity(name, mo, me, ml, beyond)
    assert mo <= O_MAX_ABS and me <= O_MEAN_ABS and ml <= LSE_MAX_ABS


def test_closed_forms_on_gpu():
    dev = device()
    for d in (64, 128):
        for causal in (False, True):
            N = 300
            w = workloads.custom(1, 2, N, d, causal, seed=77 + d)
            _, k, v = workloads.make_inputs(w)
            q = torch.zeros_like(k)
            o, lse = run_gpu(q, k, v, w.scale, causal)
            counts = np.arange(1, N + 1) if causal else np.full(N, N)
            v64 = to64(v)
            mean = np.cumsum(v64, axis=2) / counts[None, None, :, None] if causal \
                else np.broadcast_to(v64.mean(axis=2, keepdims=True), v64.shape)
            assert np.abs(to64(o) - mean).max() <= O_MAX_ABS
            assert np.abs(to64(lse) - np.log(counts)[None, None]).max() <= LSE_MAX_ABS
            if causal:
                # row 0 sees only key 0: P = 1 exactly, so O_0 is V_0 bit for bit
                q2, k2, v2 = workloads.make_inputs(w)
                o2, lse2 = run_gpu(q2, k2, v2, w.scale, True)
                assert torch.equal(o2[:, :, 0].cpu().view(torch.int16), v2[:, :, 0].view(torch.int16))
                s00 = w.scale * (q2[:, :, 0].double() * k2[:, :, 0].double()).sum(-1)
                assert (lse2[:, :, 0].cpu().double() - s00).abs().max().item() <= LSE_MAX_ABS
    # N = 1: O = V
    w = workloads.custom(2, 3, 1, 128, False, seed=5)
    q, k, v = workloads.make_inputs(w)
    o, _ = run_gpu(q, k, v, w.scale, False)
    assert torch.equal(o.cpu().view(torch.int16), v.view(torch.int16))


@pytest.mark.parametrize("B,H,N,d,causal", [(2, 4, 777, 128, True), (1, 3, 333, 64, False)])
def test_bitwise_deterministic_and_no_out_of_bounds_writes(B, H, N, d, causal):
    dev = device()
    w = workloads.custom(B, H, N, d, causal, seed=9)
    announce(f"[canary] {w.name}")
    q, k, v = (t.to(dev) for t in workloads.make_inputs(w))
    n_o, n_l = q.numel(), w.B * w.H * w.N
    pad = 4096
    o_buf = torch.full((n_o + 2 * pad,), -7.25, dtype=torch.bfloat16, device=dev)
    l_buf = torch.full((n_l + 2 * pad,), -7.25, dtype=torch.float32, device=dev)
    o = o_buf[pad:pad + n_o].view(q.shape)
    lse = l_buf[pad:pad + n_l].view(w.B, w.H, w.N)
    fa.fwd(q, k, v, scale=w.scale, causal=causal, out=o, lse=lse)
    o2, l2 = fa.fwd(q, k, v, scale=w.scale, causal=causal)
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(lse.view(torch.int32), l2.view(torch.int32))
    for buf in (o_buf, l_buf):
        assert (buf[:pad] == -7.25).all().item() and (buf[-pad:] == -7.25).all().item()


def test_runs_on_a_non_default_stream():
    dev = device()
    w = workloads.custom(1, 4, 640, 64, False, seed=13)
    q, k, v = (t.to(dev) for t in workloads.make_inputs(w))
    ref_o, ref_l = fa.fwd(q, k, v, scale=w.scale)
    s = torch.cuda.Stream(device=dev)
    s.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(s):
        o, lse = fa.fwd(q, k, v, scale=w.scale)
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), ref_o.view(torch.int16))
    assert torch.equal(lse, ref_l)


def test_non_default_scale_and_large_scores():
    """scale other than 1/sqrt(d); scores spread over tens of units make the
    softmax peaky and force the running maximum to move on many tiles.  With a
    dominant key O approaches a single V row, whose entries reach |v| >= 4,
    where half a bf16 ulp of the stored O is up to 2^-6: this case is held to
    1e-2 beyond the output's own bf16 rounding (the five workloads are held to
    1e-2 outright), and the raw difference is reported."""
    for scale, mult in ((0.5, 1.0), (0.02, 1.0), (1.0 / math.sqrt(128), 6.0)):
        w = workloads.custom(1, 2, 900, 128, True, seed=int(scale * 1000) + int(mult))
        q, k, v = workloads.make_inputs(w)
        q = (q.float() * mult).to(torch.bfloat16)
        o, lse = run_gpu(q, k, v, scale, True)
        beyond, me, ml, raw = compare_full(q, k, v, scale, True, o, lse, with_rounding=True)
        announce(f"[scale {scale} x{mult}] max|dO|={raw:.3e} (beyond O's rounding {beyond:.3e}) "
                 f"mean|dO|={me:.3e} max|dLSE|={ml:.3e}")
        assert beyond <= O_MAX_ABS and me <= O_MEAN_ABS and ml <= LSE_MAX_ABS


@pytest.mark.parametrize("B,H,N,d,causal", [(1, 1, 262144, 128, True), (1, 2, 131072, 64, False),
                                             (1, 1, 2097152, 128, True)])
def test_long_sequences_on_sampled_rows(B, H, N, d, causal):
    """Sequences 4x, 2x and 32x the longest workload's (the last: 2M tokens,
    512 MiB per tensor): 32-bit tile and row arithmetic, the causal block
    order and the reference-maximum path over thousands of key tiles.
    Sampled rows against the oracle."""
    w = workloads.custom(B, H, N, d, causal, seed=5000 + d)
    announce(f"[parity-long] {w.name}: generating inputs")
    q, k, v = workloads.make_inputs(w)
    announce(f"[parity-long] {w.name}: running fa_fwd")
    o, lse = run_gpu(q, k, v, w.scale, causal)
    assert torch.isfinite(o.float()).all() and torch.isfinite(lse).all()
    mo, me, ml = compare_rows(q, k, v, w.scale, causal, o.cpu(), lse.cpu(), sample_picks(w, n_heads=2, n_rand=24))
    announce(f"    max|dO|={mo:.3e} mean|dO|={me:.3e} max|dLSE|={ml:.3e}")
    assert mo <= O_MAX_ABS and me <= O_MEAN_ABS and ml <= LSE_MAX_ABS


@pytest.mark.parametrize("d", [64, 128])
def test_late_dominant_key_moves_the_reference(d):
    """Key 700 is 8 times query 750 (exact in bf16): every row that sees it
    gets a score far above its earlier tiles', so the kernel must move its
    reference maximum in the middle of the sequence (for d = 64 through the
    recomputation of the tile's P).  Where that key dominates a row, its
    weight must be exact (the reference moves to it) rather than a lagged
    2^delta rounded to bf16, or O would be off by up to 2^-8 |v|: O is held
    to 1e-2 beyond its own output rounding, LSE and mean|dO| outright."""
    w = workloads.custom(1, 2, 900, d, True, seed=600 + d)
    q, k, v = workloads.make_inputs(w)
    k[:, :, 700] = (q[:, :, 750].float() * 8).to(torch.bfloat16)
    for scale in (w.scale, 0.5):
        o, lse = run_gpu(q, k, v, scale, True)
        beyond, me, ml, raw = compare_full(q, k, v, scale, True, o, lse, with_rounding=True)
        announce(f"[late key d={d} scale {scale:.3f}] max|dO|={raw:.3e} (beyond O's rounding {beyond:.3e}) "
                 f"mean|dO|={me:.3e} max|dLSE|={ml:.3e}")
        assert beyond <= O_MAX_ABS and me <= O_MEAN_ABS and ml <= LSE_MAX_ABS


def test_caller_buffers_of_the_wrong_shape_dtype_or_layout_are_rejected():
    """Outputs and workspaces the caller passes reach the kernels as raw
    pointers; a buffer that does not match is refused before any launch and
    is left untouched."""
    dev = device()
    w = workloads.custom(1, 2, 300, 64, True, seed=21)
    q, k, v = (t.to(dev) for t in workloads.make_inputs(w))
    B, H, N, d = q.shape
    short_o = torch.full((B, H, N - 1, d), 3.0, dtype=torch.bfloat16, device=dev)
    f32_o = torch.zeros(q.shape, dtype=torch.float32, device=dev)
    strided_o = torch.zeros((B, H, d, N), dtype=torch.bfloat16, device=dev).transpose(2, 3)
    short_l = torch.full((B, H, N - 1), 3.0, dtype=torch.float32, device=dev)
    for kw in ({"out": short_o}, {"out": f32_o}, {"out": strided_o}, {"lse": short_l}):
        with pytest.raises(ValueError):
            fa.fwd(q, k, v, causal=True, **kw)
    o, lse = fa.fwd(q, k, v, causal=True)
    dout = torch.randn_like(o)
    for name in ("dq", "dk", "dv"):
        with pytest.raises(ValueError):
            fa.bwd(q, k, v, o, lse, dout, causal=True, **{name: short_o})
    with pytest.raises(ValueError):
        fa.bwd(q, k, v, o, lse, dout, causal=True, delta=short_l)
    with pytest.raises(ValueError):
        fa.fwd_splitkv(q, k, v, causal=True, n_splits=2,
                       o_part=torch.empty((1, B, H, N, d), dtype=torch.float32, device=dev))
    with pytest.raises(ValueError):
        fa.fwd_splitkv(q, k, v, causal=True, n_splits=2,
                       lse_part=torch.empty((2, B, H, N - 1), dtype=torch.float32, device=dev))
    with pytest.raises(ValueError):
        fa.fwd_fa1order(q, k, v, causal=True, o_acc=torch.empty(q.shape, dtype=torch.bfloat16, device=dev))
    with pytest.raises(ValueError):
        fa.fwd_fa1order(q, k, v, causal=True, m=short_l)
    with pytest.raises(ValueError):
        fa.quant_fp8(q, out=torch.empty((B, H, N - 1, d), dtype=torch.uint8, device=dev))
    with pytest.raises(ValueError):
        fa.quant_fp8(q, descale=torch.empty((B, H + 1), dtype=torch.float32, device=dev))
    q8, qd = fa.quant_fp8(q)
    with pytest.raises(ValueError):
        fa.fwd_fp8(q8, q8, q8, qd, qd, qd, causal=True, out=short_o)
    with pytest.raises(ValueError):
        fa.fwd(q, k.cpu(), v, causal=True)
    torch.cuda.synchronize()
    assert (short_o == 3.0).all().item() and (short_l == 3.0).all().item()


@pytest.mark.parametrize("B,H,N,d,causal,workload", [
    (2, 4, 777, 128, True, None), (1, 3, 333, 64, False, None), (1, 2, 1000, 64, True, None),
    (3, 1, 1025, 128, True, None), (0, 0, 0, 0, False, "mid_b4h16_n4096_d128")])
def test_extra_barrier_build_is_bitwise_equal(B, H, N, d, causal, workload):
    """The race-check build waits for every memory operation and holds a
    workgroup barrier after each step's LDS reads, so no wave can refill an
    LDS ring buffer another wave may still read.  Its results must equal the
    default build's bit for bit: a race on the rings (the on-chip tiles the
    tiled method reuses across the key loop) would show as a difference."""
    dev = device()
    w = workloads.WORKLOADS[workload] if workload else workloads.custom(B, H, N, d, causal, seed=31 + N)
    announce(f"[racecheck] {w.name}")
    q, k, v = (t.to(dev) for t in workloads.make_inputs(w))
    o, lse = fa.fwd(q, k, v, scale=w.scale, causal=w.causal)
    o2, l2 = variant_fwd("racecheck", q, k, v, w.scale, w.causal)
    assert torch.equal(o.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(lse.view(torch.int32), l2.view(torch.int32))
    # the split-KV kernel, compiled from the same source, the same way
    n_splits = 3
    o3, l3 = fa.fwd_splitkv(q, k, v, scale=w.scale, causal=w.causal, n_splits=n_splits)
    o4, l4 = variant_fwd_splitkv("racecheck", q, k, v, w.scale, w.causal, n_splits)
    assert torch.equal(o3.view(torch.int16), o4.view(torch.int16))
    assert torch.equal(l3.view(torch.int32), l4.view(torch.int32))


@pytest.mark.parametrize("B,H,N,causal", [(1, 1, 65, False), (2, 3, 513, True), (1, 2, 1000, True),
                                           (2, 2, 2048, False)])
def test_row_group_build_matches_oracle(B, H, N, causal):
    """The d = 128 build with two 32-row groups per wave and 32-key tiles
    (one wave per SIMD) against the oracle on every element, and bit for bit
    against its own extra-barrier build (no race on its LDS rings)."""
    dev = device()
    w = workloads.custom(B, H, N, 128, causal, seed=1300 + N + int(causal))
    q, k, v = workloads.make_inputs(w)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    o, lse = variant_fwd("g2", qd, kd, vd, w.scale, causal)
    o2, l2 = variant_fwd("g2racecheck", qd, kd, vd, w.scale, causal)
    assert torch.equal(o.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(lse.view(torch.int32), l2.view(torch.int32))
    mo, me, ml = compare_full(q, k, v, w.scale, causal, o, lse)
    announce(f"[row groups] {w.name}: max|dO|={mo:.3e} mean|dO|={me:.3e} max|dLSE|={ml:.3e}")
    assert mo <= O_MAX_ABS and me <= O_MEAN_ABS and ml <= LSE_MAX_ABS


@pytest.mark.parametrize("d", [64, 128])
def test_exact_running_max_build_keeps_a_late_dominant_key_exact(d):
    """The build whose reference maximum is the running row maximum itself
    (the online softmax as the pages write it: m_new = max(m, rowmax S)):
    the dominant key's weight is exp(0) = 1, exact in bf16, so on the
    late-dominant-key rows O is held to 1e-2 beyond its own output rounding
    alone, and LSE and mean|dO| outright."""
    dev = device()
    w = workloads.custom(1, 2, 900, d, True, seed=600 + d)
    q, k, v = workloads.make_inputs(w)
    k[:, :, 700] = (q[:, :, 750].float() * 8).to(torch.bfloat16)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    for scale in (w.scale, 0.5):
        o, lse = variant_fwd("exactmax", qd, kd, vd, scale, True)
        beyond, me, ml, raw = compare_full(q, k, v, scale, True, o, lse, with_rounding=True)
        announce(f"[exact max, late key d={d} scale {scale:.3f}] max|dO|={raw:.3e} "
                 f"(beyond O's rounding {beyond:.3e}) mean|dO|={me:.3e} max|dLSE|={ml:.3e}")
        assert beyond <= O_MAX_ABS and me <= O_MEAN_ABS and ml <= LSE_MAX_ABS


@pytest.mark.parametrize("B,H,N,d,causal", [(1, 3, 700, 128, True), (2, 2, 513, 64, False), (1, 2, 1000, 64, True)])
def test_exact_running_max_build_matches_oracle(B, H, N, d, causal):
    dev = device()
    w = workloads.custom(B, H, N, d, causal, seed=1000 + N + d + int(causal))
    q, k, v = workloads.make_inputs(w)
    o, lse = variant_fwd("exactmax", q.to(dev), k.to(dev), v.to(dev), w.scale, causal)
    mo, me, ml = compare_full(q, k, v, w.scale, causal, o, lse)
    announce(f"[exact max] {w.name}: max|dO|={mo:.3e} mean|dO|={me:.3e} max|dLSE|={ml:.3e}")
    assert mo <= O_MAX_ABS and me <= O_MEAN_ABS and ml <= LSE_MAX_ABS
