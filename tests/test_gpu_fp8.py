"""The FP8 path (fa_quant_fp8, fa_fwd_fp8) against the oracle (GPU only).

Quantisation: codes and descale factors are integers / fp32 values the
definition fixes, so they must agree bit for bit with oracle.fp8.quantize_heads.

Attention: the oracle is fed its own quantisation of the bf16 inputs (the
GPU gets the same codes), and computes the online softmax with P rounded to
E4M3 (oracle.fp8.attention_fp8) in fp64.  The GPU's P is fp32, so a P within
rounding noise of a midpoint between two codes may round the other way; the
bar per element is |dO| <= half a bf16 ulp of O + the move of one such flip
(gpu_common.fp8_flip_allowance) + 1e-6; the mean of what |dO| exceeds half a
bf16 ulp by (the error the bf16 output does not explain) <= 1e-4; and
|dLSE| <= 1e-3 (the LSE adds unrounded P on both sides).
"""
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import io_aware_exact_13_amd as fa
import oracle
import workloads
from gpu_common import (announce, bf16_half_ulp, device, e4m3_p_bounds, fp8_flip_allowance, oracle_threads, row_spans,
                        spans_per_head, to64, variant_fwd_fp8)
from oracle import fp8 as ofp8

pytestmark = pytest.mark.gpu

O_MEAN_EXCESS = 1e-4
LSE_MAX = 1e-3


def gpu_quant(x, rotate, signs):
    x8, desc = fa.quant_fp8(x.to(device()), rotate=rotate, sign_bits=signs)
    torch.cuda.synchronize()
    return x8.cpu().numpy(), desc.cpu().numpy()


def oracle_quant(q, k, v, rotate, signs):
    cq, _, dq = ofp8.quantize_heads(q.float().numpy(), rotate, signs)
    ck, _, dk = ofp8.quantize_heads(k.float().numpy(), rotate, signs)
    cv, _, dv = ofp8.quantize_heads(v.float().numpy(), False, 0)
    return (cq, dq), (ck, dk), (cv, dv)


def gpu_fwd_fp8(qq, kk, vv, scale, causal):
    dev = device()
    t = [torch.from_numpy(np.ascontiguousarray(c)).to(dev) for c, _ in (qq, kk, vv)]
    d = [torch.from_numpy(np.ascontiguousarray(s)).to(dev) for _, s in (qq, kk, vv)]
    o, lse = fa.fwd_fp8(*t, *d, scale=scale, causal=causal)
    torch.cuda.synchronize()
    return o, lse


def check_rows(qq, kk, vv, scale, causal, o, lse, picks):
    """Compare the GPU's O/LSE on (b, h, rows) picks with the oracle; returns
    (max excess over the per-element bar, mean excess of |dO| over half a
    bf16 ulp, max |dLSE|)."""
    worst, worst_l, tot, cnt = -np.inf, 0.0, 0.0, 0
    deq = [ofp8.dequantize_heads(c, s) for c, s in (qq, kk, vv)]
    for b, h, rows in picks:
        qd, kd, vd = (x[b, h] for x in deq)
        ro, rl = ofp8.attention_fp8_head_rows(qd, kd, vd, scale, causal, rows)
        go = to64(o[b, h, torch.as_tensor(rows)])
        gl = to64(lse[b, h, torch.as_tensor(rows)])
        diff = np.abs(go - ro)
        half = bf16_half_ulp(ro)
        bar = half + fp8_flip_allowance(qd, kd, vd, scale, causal, rows) + 1e-6
        worst = max(worst, float((diff - bar).max()))
        worst_l = max(worst_l, float(np.abs(gl - rl).max()))
        tot += float(np.maximum(diff - half, 0.0).sum())
        cnt += diff.size
    return worst, tot / cnt, worst_l


QUANT_CASES = [(1, 1, 1, 64), (1, 2, 333, 128), (2, 3, 100, 64), (1, 2, 4096, 128), (1, 1, 700, 64)]


@pytest.mark.parametrize("rotate", [False, True])
@pytest.mark.parametrize("B,H,N,d", QUANT_CASES)
def test_quantisation_is_bit_exact(B, H, N, d, rotate):
    w = workloads.custom(B, H, N, d, False, seed=6000 + N + d)
    q, k, v = workloads.make_inputs(w)
    q[0, 0] = 0                                    # an all-zero head: codes 0, descale 0
    signs = workloads.make_fp8_signs(w.seed, d)
    announce(f"[fp8-quant] {w.name} rotate={rotate}")
    for x in (q, k):
        g8, gd = gpu_quant(x, rotate, signs)
        c, _, ds = ofp8.quantize_heads(x.float().numpy(), rotate, signs)
        assert np.array_equal(g8, c), int((g8 != c).sum())
        assert np.array_equal(gd.view(np.uint32), ds.view(np.uint32))
        if x is q:                                 # zeros (the rotation may give -0, code 0x80)
            assert not (g8[0, 0] & 0x7F).any() and gd[0, 0] == 0


def test_quantisation_of_tiny_heads_is_bit_exact():
    """Heads of bf16 subnormals and of values near 2^-117: the amax floor keeps
    448 / amax finite; codes and factors match the oracle bit for bit."""
    w = workloads.custom(1, 3, 300, 128, False, seed=6150)
    q = workloads.make_inputs(w)[0].float()
    q[0, 0] *= 2.0 ** -133          # bf16 subnormals (and some flushed to zero)
    q[0, 1] *= 2.0 ** -118
    x = q.to(torch.bfloat16)
    signs = workloads.make_fp8_signs(w.seed, w.d)
    for rotate in (False, True):
        g8, gd = gpu_quant(x, rotate, signs)
        c, _, ds = ofp8.quantize_heads(x.float().numpy(), rotate, signs)
        assert np.array_equal(g8, c) and np.array_equal(gd.view(np.uint32), ds.view(np.uint32))
        assert np.isfinite(ofp8.e4m3_decode(g8)).all()


def test_quantisation_of_peaky_and_outlier_inputs_is_bit_exact():
    for w, maker in ((workloads.custom(1, 2, 2048, 128, True, seed=6101, peaky=True), workloads.make_inputs),
                     (workloads.custom(1, 2, 1024, 128, True, seed=6102), workloads.make_outlier_inputs),
                     (workloads.custom(2, 1, 513, 64, True, seed=6103), workloads.make_outlier_inputs)):
        q, k, v = maker(w)
        signs = workloads.make_fp8_signs(w.seed, w.d)
        for rotate in (False, True):
            for x in (q, k, v):
                g8, gd = gpu_quant(x, rotate, signs)
                c, _, ds = ofp8.quantize_heads(x.float().numpy(), rotate, signs)
                assert np.array_equal(g8, c) and np.array_equal(gd.view(np.uint32), ds.view(np.uint32))


ATT_CASES = [
    (1, 1, 256, 64, False), (1, 2, 333, 128, False), (2, 1, 1000, 64, True), (1, 3, 700, 128, True),
    (1, 1, 1, 128, False), (1, 1, 65, 64, True), (1, 2, 513, 128, True), (1, 1, 4096, 128, True),
    (1, 1, 2048, 64, False),
]


@pytest.mark.parametrize("B,H,N,d,causal", ATT_CASES)
def test_fp8_attention_matches_oracle(B, H, N, d, causal):
    w = workloads.custom(B, H, N, d, causal, seed=6200 + N + d + int(causal))
    q, k, v = workloads.make_inputs(w)
    rotate = d == 128
    qq, kk, vv = oracle_quant(q, k, v, rotate, workloads.make_fp8_signs(w.seed, d))
    announce(f"[fp8-att] {w.name} rotate={rotate}")
    o, lse = gpu_fwd_fp8(qq, kk, vv, w.scale, causal)
    picks = [(b, h, np.arange(N)) for b in range(B) for h in range(H)]
    worst, mean, dl = check_rows(qq, kk, vv, w.scale, causal, o, lse, picks)
    announce(f"    excess over bar {worst:.3e}  mean excess {mean:.3e}  max|dLSE| {dl:.3e}")
    assert worst <= 0 and mean <= O_MEAN_EXCESS and dl <= LSE_MAX


def check_rows_against_plain(qq, kk, vv, scale, causal, o, lse, picks):
    """The GPU's O/LSE on (b, h, rows) picks against the plain definition on
    the dequantised operands (no key blocking anywhere), with the E4M3
    rounding of P bounded from that definition alone (gpu_common.e4m3_p_bounds).
    Returns (max of |dO| - bar, observed / predicted mean square of dO, max |dLSE|)."""
    worst, worst_l, sq, pred = -np.inf, 0.0, 0.0, 0.0
    deq = [ofp8.dequantize_heads(c, s) for c, s in (qq, kk, vv)]
    for b, h, rows in picks:
        qd, kd, vd = (x[b, h] for x in deq)
        ro, rl, bound, var = e4m3_p_bounds(qd, kd, vd, scale, causal, rows)
        go = to64(o[b, h, torch.as_tensor(rows)])
        gl = to64(lse[b, h, torch.as_tensor(rows)])
        diff = np.abs(go - ro)
        half = bf16_half_ulp(ro)
        worst = max(worst, float((diff - (half + bound + 1e-5)).max()))
        worst_l = max(worst_l, float(np.abs(gl - rl).max()))
        sq += float((diff * diff).sum())
        pred += float((var + half * half / 3.0).sum())
    return worst, sq / pred, worst_l


PLAIN_CASES = [(1, 2, 513, 128, True), (1, 1, 4096, 128, True), (1, 1, 2048, 64, False), (2, 2, 333, 64, True)]


@pytest.mark.parametrize("B,H,N,d,causal", PLAIN_CASES)
def test_fp8_attention_within_the_e4m3_bound_of_the_plain_definition(B, H, N, d, causal):
    """A check that does not depend on how the kernel blocks the keys: O
    against the plain softmax attention of the dequantised operands, within
    the most that rounding P to E4M3 can move it (a change of the kernel's
    key blocking must still pass this, and a wrong rounding or a lost term
    must not), and the mean square difference at most what independent
    roundings with errors spread over their whole range would give."""
    w = workloads.custom(B, H, N, d, causal, seed=6400 + N + d + int(causal))
    q, k, v = workloads.make_inputs(w)
    rotate = d == 128
    qq, kk, vv = oracle_quant(q, k, v, rotate, workloads.make_fp8_signs(w.seed, d))
    announce(f"[fp8-plain] {w.name} rotate={rotate}")
    o, lse = gpu_fwd_fp8(qq, kk, vv, w.scale, causal)
    picks = [(b, h, np.arange(N)) for b in range(B) for h in range(H)]
    worst, ratio, dl = check_rows_against_plain(qq, kk, vv, w.scale, causal, o, lse, picks)
    announce(f"    |dO| - bound {worst:.3e}  mean square / predicted {ratio:.3f}  max|dLSE| {dl:.3e}")
    assert worst <= 0 and ratio <= 1.0 and dl <= LSE_MAX


def test_fp8_headline_shape_on_sampled_rows():
    """1 x 32 x 16384 x 128, causal: the GPU quantises all heads (two checked
    bit for bit against the oracle), the GPU forward runs on its codes, and
    sampled rows of those two heads are checked against the oracle run on the
    oracle's own codes."""
    dev = device()
    w = workloads.WORKLOADS[workloads.HEADLINE]
    q, k, v = workloads.make_inputs(w)
    signs = workloads.make_fp8_signs(w.seed, w.d)
    announce("[fp8-headline] quantising")
    q8, qd = fa.quant_fp8(q.to(dev), rotate=True, sign_bits=signs)
    k8, kd = fa.quant_fp8(k.to(dev), rotate=True, sign_bits=signs)
    v8, vd = fa.quant_fp8(v.to(dev), rotate=False)
    o, lse = fa.fwd_fp8(q8, k8, v8, qd, kd, vd, scale=w.scale, causal=True)
    o2, l2 = fa.fwd_fp8(q8, k8, v8, qd, kd, vd, scale=w.scale, causal=True)
    torch.cuda.synchronize()
    # bitwise equal run to run: a race would show here even inside the tolerance
    assert torch.equal(o.view(torch.int16), o2.view(torch.int16)) and torch.equal(lse.view(torch.int32), l2.view(torch.int32))
    del o2, l2
    assert torch.isfinite(o.float()).all() and torch.isfinite(lse).all()
    rng = np.random.default_rng(17)
    for h in (0, 31):
        announce(f"[fp8-headline] head {h}: oracle quantisation and rows")
        qq, kk, vv = oracle_quant(q[:, h:h + 1], k[:, h:h + 1], v[:, h:h + 1], True, signs)
        for (c, s), (g8, gs) in zip((qq, kk, vv), ((q8, qd), (k8, kd), (v8, vd))):
            assert np.array_equal(g8[:, h:h + 1].cpu().numpy(), c)
            assert np.array_equal(gs[:, h:h + 1].cpu().numpy().view(np.uint32), s.view(np.uint32))
        rows = np.array(sorted(set(range(40)) | set(range(w.N - 40, w.N)) |
                               set(rng.integers(0, w.N, 48).tolist()) | {255, 256, 8191, 8192}))
        worst, mean, dl = check_rows(qq, kk, vv, w.scale, True, o[:, h:h + 1], lse[:, h:h + 1], [(0, 0, rows)])
        announce(f"    excess over bar {worst:.3e}  mean excess {mean:.3e}  max|dLSE| {dl:.3e}")
        assert worst <= 0 and mean <= O_MEAN_EXCESS and dl <= LSE_MAX
        worst, ratio, dl = check_rows_against_plain(qq, kk, vv, w.scale, True, o[:, h:h + 1], lse[:, h:h + 1],
                                                     [(0, 0, rows)])
        announce(f"    plain definition: |dO| - bound {worst:.3e}  mean square / predicted {ratio:.3f}")
        assert worst <= 0 and ratio <= 1.0 and dl <= LSE_MAX


@pytest.mark.parametrize("name", ["causal_b1h32_n16384_d128", "mid_b4h16_n4096_d128", "short_b16h32_n2048_d64",
                                  "causal_peaky_b1h8_n65536_d128"])
def test_fp8_full_size_every_element_within_the_plain_bound(name):
    """Full-size workloads, every element of every head: the GPU's E4M3
    codes and factors equal the oracle's for every head, and the GPU's O and
    LSE on those codes lie within the E4M3 bound of the plain definition on
    the dequantised operands (the check that does not depend on the kernel's
    key blocking), with the mean square difference at most the predicted one
    over the whole tensor.  Rows go in blocks of 256, each (under the causal
    mask) against the keys the mask leaves it; the rest carry weight 0."""
    dev = device()
    w = workloads.WORKLOADS[name]
    q, k, v = workloads.make_inputs(w)
    signs = workloads.make_fp8_signs(w.seed, w.d)
    rotate = w.d == 128
    q8, qd = fa.quant_fp8(q.to(dev), rotate=rotate, sign_bits=signs)
    k8, kd = fa.quant_fp8(k.to(dev), rotate=rotate, sign_bits=signs)
    v8, vd = fa.quant_fp8(v.to(dev), rotate=False)
    o, lse = fa.fwd_fp8(q8, k8, v8, qd, kd, vd, scale=w.scale, causal=w.causal)
    torch.cuda.synchronize()
    o, lse = o.cpu(), lse.cpu()
    codes = [(x8.cpu().numpy(), xs.cpu().numpy()) for x8, xs in ((q8, qd), (k8, kd), (v8, vd))]

    def part(bh, s0, s1):
        """(codes equal, |dO| - bound, max |dLSE|, sum of dO^2, predicted sum)
        of query rows [s0, s1) of one head."""
        b, h = divmod(bh, w.H)
        sl = (slice(b, b + 1), slice(h, h + 1))
        qq, kk, vv = oracle_quant(q[sl], k[sl], v[sl], rotate, signs)
        same = all(np.array_equal(g8[sl], c) and np.array_equal(gs[sl].view(np.uint32), sc.view(np.uint32))
                   for (c, sc), (g8, gs) in zip((qq, kk, vv), codes))
        qd64, kd64, vd64 = (ofp8.dequantize_heads(c, sc)[0, 0] for c, sc in (qq, kk, vv))
        hw, hl, hsq, hpred = -np.inf, 0.0, 0.0, 0.0
        for r0 in range(s0, s1, 256):
            r1 = min(s1, r0 + 256)
            kmax = r1 if w.causal else w.N
            ro, rl, bound, var = e4m3_p_bounds(qd64, kd64[:kmax], vd64[:kmax], w.scale, w.causal,
                                               np.arange(r0, r1))
            diff = np.abs(to64(o[b, h, r0:r1]) - ro)
            half = bf16_half_ulp(ro)
            hw = max(hw, float((diff - (half + bound + 1e-5)).max()))
            hl = max(hl, float(np.abs(to64(lse[b, h, r0:r1]) - rl).max()))
            hsq += float((diff * diff).sum())
            hpred += float((var + half * half / 3.0).sum())
        return same, hw, hl, hsq, hpred

    worst, worst_l, sq, pred = -np.inf, 0.0, 0.0, 0.0
    n_heads = w.B * w.H
    with oracle_threads() as workers, ThreadPoolExecutor(workers) as ex:
        spans = row_spans(w.N, w.causal, spans_per_head(n_heads, w.N, workers))
        tasks = [(bh, s0, s1) for bh in range(n_heads) for s0, s1 in spans]
        for (bh, s0, _), (same, hw, hl, hsq, hpred) in zip(tasks, ex.map(lambda t: part(*t), tasks)):
            assert same, f"codes or factors of head {divmod(bh, w.H)}"
            worst, worst_l, sq, pred = max(worst, hw), max(worst_l, hl), sq + hsq, pred + hpred
            if s0 == spans[-1][0] and (bh % 16 == 15 or bh == n_heads - 1):
                announce(f"[fp8-all] {name}: {bh + 1} heads, |dO| - bound so far {worst:.3e}, "
                         f"max|dLSE| {worst_l:.3e}")
    announce(f"    all heads: |dO| - bound {worst:.3e}  mean square / predicted {sq / pred:.3f}  "
             f"max|dLSE| {worst_l:.3e}")
    assert worst <= 0 and sq / pred <= 1.0 and worst_l <= LSE_MAX


@pytest.mark.parametrize("name", ["causal_peaky_b1h8_n65536_d128", "short_b16h32_n2048_d64",
                                  "mid_b4h16_n4096_d128"])
def test_fp8_other_workloads_on_sampled_rows(name):
    """The other full-size workloads through the whole GPU path (quantise, then
    the forward); two heads' codes checked bit for bit and their sampled rows
    against the oracle on its own codes.  The 64K-token peaky case keeps the
    running maximum moving (1% of the keys are 8x larger)."""
    dev = device()
    w = workloads.WORKLOADS[name]
    q, k, v = workloads.make_inputs(w)
    signs = workloads.make_fp8_signs(w.seed, w.d)
    rotate = w.d == 128
    announce(f"[fp8-full] {name}: quantising and running the forward")
    q8, qd = fa.quant_fp8(q.to(dev), rotate=rotate, sign_bits=signs)
    k8, kd = fa.quant_fp8(k.to(dev), rotate=rotate, sign_bits=signs)
    v8, vd = fa.quant_fp8(v.to(dev), rotate=False)
    o, lse = fa.fwd_fp8(q8, k8, v8, qd, kd, vd, scale=w.scale, causal=w.causal)
    torch.cuda.synchronize()
    assert torch.isfinite(o.float()).all() and torch.isfinite(lse).all()
    rng = np.random.default_rng(23)
    for b, h in ((0, 0), (w.B - 1, w.H - 1)):
        announce(f"[fp8-full] {name}: head ({b},{h})")
        sl = (slice(b, b + 1), slice(h, h + 1))
        qq, kk, vv = oracle_quant(q[sl], k[sl], v[sl], rotate, signs)
        for (c, s), (g8, gs) in zip((qq, kk, vv), ((q8, qd), (k8, kd), (v8, vd))):
            assert np.array_equal(g8[sl].cpu().numpy(), c)
            assert np.array_equal(gs[sl].cpu().numpy().view(np.uint32), s.view(np.uint32))
        rows = np.array(sorted(set(range(24)) | set(range(w.N - 24, w.N)) |
                               set(rng.integers(0, w.N, 24).tolist())))
        worst, mean, dl = check_rows(qq, kk, vv, w.scale, w.causal, o[sl], lse[sl], [(0, 0, rows)])
        announce(f"    excess over bar {worst:.3e}  mean excess {mean:.3e}  max|dLSE| {dl:.3e}")
        assert worst <= 0 and mean <= O_MEAN_EXCESS and dl <= LSE_MAX


def test_fp8_special_cases():
    """A zero V head gives O = 0 exactly; a key equal to 10 x a query row
    dominates that row, whose O is then (up to the bf16 output) that key's
    dequantised V row; equal keys give the mean of V."""
    w = workloads.custom(1, 2, 300, 128, False, seed=6301)
    q, k, v = workloads.make_inputs(w)
    v[0, 1] = 0
    k[0, 0, 123] = (q[0, 0, 200].float() * 10).to(torch.bfloat16)
    qq, kk, vv = oracle_quant(q, k, v, False, 0)
    o, lse = gpu_fwd_fp8(qq, kk, vv, w.scale, False)
    assert torch.all(o[0, 1] == 0) and torch.isfinite(lse).all()
    vrow = ofp8.dequantize_heads(*vv)[0, 0, 123]
    got = to64(o[0, 0, 200])
    assert np.all(np.abs(got - vrow) <= bf16_half_ulp(vrow) + 1e-6)
    # all keys equal: every P is 1, O is the mean of the V rows
    k2 = k.clone()
    k2[:] = k[0, 0, 0]
    qq, kk, vv = oracle_quant(q, k2, v, False, 0)
    o, lse = gpu_fwd_fp8(qq, kk, vv, w.scale, False)
    mean_v = ofp8.dequantize_heads(*vv)[0, 0].mean(axis=0)
    assert np.all(np.abs(to64(o[0, 0]) - mean_v) <= bf16_half_ulp(mean_v) + 1e-5)


@pytest.mark.parametrize("B,H,N,d,causal,workload", [
    (2, 3, 777, 128, True, None), (1, 3, 333, 64, False, None), (1, 2, 1000, 64, True, None),
    (3, 1, 1025, 128, True, None), (0, 0, 0, 0, False, "causal_b1h32_n16384_d128")])
def test_fp8_extra_barrier_build_is_bitwise_equal(B, H, N, d, causal, workload):
    """The FP8 forward's race-check build waits for every memory operation
    and holds a workgroup barrier after each step's LDS reads, so no wave can
    refill a ring buffer another wave may still read.  Its results must
    equal the default build's bit for bit."""
    dev = device()
    w = workloads.WORKLOADS[workload] if workload else workloads.custom(B, H, N, d, causal, seed=6500 + N)
    announce(f"[fp8 racecheck] {w.name}")
    q, k, v = (t.to(dev) for t in workloads.make_inputs(w))
    signs = workloads.make_fp8_signs(w.seed, w.d)
    (q8, qd), (k8, kd), (v8, vd) = (fa.quant_fp8(x, rotate=r, sign_bits=signs if r else 0)
                                    for x, r in ((q, True), (k, True), (v, False)))
    o, lse = fa.fwd_fp8(q8, k8, v8, qd, kd, vd, scale=w.scale, causal=w.causal)
    o2, l2 = variant_fwd_fp8("fp8racecheck", q8, k8, v8, qd, kd, vd, w.scale, w.causal)
    assert torch.equal(o.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(lse.view(torch.int32), l2.view(torch.int32))


def test_fp8_is_bitwise_deterministic():
    w = workloads.custom(1, 2, 900, 128, True, seed=6401)
    q, k, v = workloads.make_inputs(w)
    signs = workloads.make_fp8_signs(w.seed)
    a = [gpu_quant(x, True, signs) for x in (q, k)]
    b = [gpu_quant(x, True, signs) for x in (q, k)]
    for (x8, xd), (y8, yd) in zip(a, b):
        assert np.array_equal(x8, y8) and np.array_equal(xd, yd)
    qq, kk, vv = oracle_quant(q, k, v, True, signs)
    o1, l1 = gpu_fwd_fp8(qq, kk, vv, w.scale, True)
    o2, l2 = gpu_fwd_fp8(qq, kk, vv, w.scale, True)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)


@pytest.mark.parametrize("B,H,N,d,causal", [(2, 3, 777, 128, True), (1, 2, 333, 64, False)])
def test_fp8_writes_nothing_outside_its_outputs(B, H, N, d, causal):
    """Canary bytes around O and LSE stay untouched on ragged heads (the last
    query block's rows past N are staged but never stored)."""
    dev = device()
    w = workloads.custom(B, H, N, d, causal, seed=6500 + N)
    q, k, v = (t.to(dev) for t in workloads.make_inputs(w))
    signs = workloads.make_fp8_signs(w.seed, d)
    (q8, qd), (k8, kd), (v8, vd) = (fa.quant_fp8(q, rotate=True, sign_bits=signs),
                                    fa.quant_fp8(k, rotate=True, sign_bits=signs), fa.quant_fp8(v))
    announce(f"[fp8-canary] {w.name}")
    n_o, n_l, pad = q.numel(), B * H * N, 4096
    o_buf = torch.full((n_o + 2 * pad,), -7.25, dtype=torch.bfloat16, device=dev)
    l_buf = torch.full((n_l + 2 * pad,), -7.25, dtype=torch.float32, device=dev)
    o = o_buf[pad:pad + n_o].view(q.shape)
    lse = l_buf[pad:pad + n_l].view(B, H, N)
    fa.fwd_fp8(q8, k8, v8, qd, kd, vd, scale=w.scale, causal=causal, out=o, lse=lse)
    o2, l2 = fa.fwd_fp8(q8, k8, v8, qd, kd, vd, scale=w.scale, causal=causal)
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(lse.view(torch.int32), l2.view(torch.int32))
    for buf in (o_buf, l_buf):
        assert (buf[:pad] == -7.25).all().item() and (buf[-pad:] == -7.25).all().item()


def test_rotation_lowers_the_fp8_error_end_to_end():
    """Whole GPU path (quantise + forward) against the fp64 attention of the
    bf16 inputs, on inputs with two outlier channels shared by Q and K: the
    rotated path's error is well below the unrotated one's."""
    dev = device()
    w = workloads.custom(1, 4, 2048, 128, True, seed=6501)
    q, k, v = workloads.make_outlier_inputs(w)
    signs = workloads.make_fp8_signs(w.seed)
    ref, _ = oracle.attention(to64(q), to64(k), to64(v), w.scale, True)
    errs = {}
    for rotate in (False, True):
        q8, qd = fa.quant_fp8(q.to(dev), rotate=rotate, sign_bits=signs)
        k8, kd = fa.quant_fp8(k.to(dev), rotate=rotate, sign_bits=signs)
        v8, vd = fa.quant_fp8(v.to(dev), rotate=False)
        o, _ = fa.fwd_fp8(q8, k8, v8, qd, kd, vd, scale=w.scale, causal=True)
        torch.cuda.synchronize()
        errs[rotate] = float(np.sqrt(np.mean((to64(o) - ref) ** 2)) / np.sqrt(np.mean(ref ** 2)))
    announce(f"[fp8-outliers] relative rms error: plain {errs[False]:.3e}  rotated {errs[True]:.3e}")
    assert errs[True] * 1.5 < errs[False]
