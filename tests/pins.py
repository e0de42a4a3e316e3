"""Checks that pin the CPU oracle to facts outside itself.

Each check takes the oracle module as an argument, so the same checks can be
run against deliberately broken copies of it (tests/test_oracle_mutations.py)
to show that a plausible slip in the oracle fails at least one of them.

Page keys: [P1] FlashAttention的Triton实现：IO-aware注意力机制底层原理;
[P2] 为什么Flash Attention能将注意力计算提速数倍而不损失精度;
[P3] GPU Kernel 入门：Triton / FlashAttention.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")

# Tiny shapes for the scalar brute force: (B, H, N, d).
TINY_SHAPES = [(1, 1, 1, 1), (1, 1, 3, 2), (1, 2, 5, 4), (2, 1, 16, 8), (1, 1, 7, 3)]


def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).normal(size=shape) * scale


# ---------------------------------------------------------------- T1
def check_worked_example(orc):
    """[P3] 动手, part 1: blockwise streaming softmax equals the whole-row softmax;
    the page prints a max difference of 1.11e-16 for its seeded 4 x 16 example."""
    with open(os.path.join(GOLDEN, "online_softmax_worked_example.json")) as f:
        g = json.load(f)
    rng = np.random.default_rng(g["seed"])
    scores = rng.normal(size=(g["rows"], g["cols"])) * g["score_multiplier"]
    full = orc.softmax_rows(scores)
    streamed = orc.online_softmax_rows(scores, g["block"])
    diff = float(np.abs(full - streamed).max())
    assert diff <= 1e-15, diff
    assert f"{diff:.2e}" == g["printed_max_abs_diff"], (diff, g["printed_max_abs_diff"])
    # and both are probability rows
    assert np.allclose(full.sum(axis=1), 1.0, atol=1e-15, rtol=0)
    return diff


# ---------------------------------------------------------------- T3
def check_rows_sum_to_one(orc):
    """[P1] 在线Softmax, 最终归一化: every row of P sums to 1; masked entries are 0."""
    for causal in (False, True):
        for (n, d, seed) in [(1, 4, 1), (9, 8, 2), (33, 16, 3), (64, 4, 4)]:
            q = _rand((n, d), seed)
            k = _rand((n, d), seed + 100)
            p = orc.probs_head(q, k, 1.0 / math.sqrt(d), causal)
            assert p.shape == (n, n)
            assert np.abs(p.sum(axis=1) - 1.0).max() <= 1e-12
            assert (p >= 0).all()
            if causal:
                assert (np.triu(p, 1) == 0).all()
                assert (np.diag(p) > 0).all()


# ---------------------------------------------------------------- T4
def brute_force(q, k, v, scale, causal):
    """Scalar per-element evaluation of the definition with math.exp / math.fsum."""
    B, H, N, d = q.shape
    o = np.zeros((B, H, N, v.shape[-1]))
    lse = np.zeros((B, H, N))
    for b in range(B):
        for h in range(H):
            for i in range(N):
                keys = range(i + 1) if causal else range(N)
                s = [scale * math.fsum(float(q[b, h, i, c]) * float(k[b, h, j, c]) for c in range(d))
                     for j in keys]
                mx = max(s)
                w = [math.exp(x - mx) for x in s]
                tot = math.fsum(w)
                for c in range(v.shape[-1]):
                    o[b, h, i, c] = math.fsum(w[t] * float(v[b, h, j, c])
                                              for t, j in enumerate(keys)) / tot
                lse[b, h, i] = mx + math.log(tot)
    return o, lse


def check_brute_force(orc):
    for idx, shape in enumerate(TINY_SHAPES):
        for causal in (False, True):
            q, k, v = (_rand(shape, 10 * idx + t, 1.5) for t in range(3))
            scale = 1.0 / math.sqrt(shape[-1])
            o, lse = orc.attention(q, k, v, scale, causal)
            ob, lb = brute_force(q, k, v, scale, causal)
            assert np.abs(o - ob).max() <= 1e-13, (shape, causal)
            assert np.abs(lse - lb).max() <= 1e-13, (shape, causal)


# ---------------------------------------------------------------- T5
def torch_reference(q, k, v, scale, causal):
    """torch CPU fp64 softmax / logsumexp: an independent library route."""
    qt, kt, vt = (torch.from_numpy(np.ascontiguousarray(x)) for x in (q, k, v))
    s = torch.matmul(qt, kt.transpose(-1, -2).contiguous()) * scale
    if causal:
        n = s.shape[-1]
        mask = torch.ones(n, n, dtype=torch.bool).triu(1)
        s = s.masked_fill(mask, float("-inf"))
    p = torch.softmax(s, dim=-1)
    return torch.matmul(p, vt).numpy(), torch.logsumexp(s, dim=-1).numpy()


def check_library_softmax(orc):
    for (shape, seed) in [((1, 1, 256, 64), 5), ((2, 3, 37, 16), 6), ((1, 2, 130, 128), 7)]:
        for causal in (False, True):
            q, k, v = (_rand(shape, seed * 3 + t) for t in range(3))
            scale = 1.0 / math.sqrt(shape[-1])
            o, lse = orc.attention(q, k, v, scale, causal)
            ot, lt = torch_reference(q, k, v, scale, causal)
            assert np.abs(o - ot).max() <= 1e-12
            assert np.abs(lse - lt).max() <= 1e-12


# ---------------------------------------------------------------- T6
def check_closed_forms(orc):
    N, d = 40, 8
    v = _rand((1, 1, N, d), 21)
    k = _rand((1, 1, N, d), 22)
    scale = 1.0 / math.sqrt(d)
    counts = np.arange(1, N + 1)
    # Q = 0: every visible key gets the same weight.
    q0 = np.zeros((1, 1, N, d))
    for causal in (False, True):
        o, lse = orc.attention(q0, k, v, scale, causal)
        if causal:
            mean = np.cumsum(v[0, 0], axis=0) / counts[:, None]
            assert np.abs(lse[0, 0] - np.log(counts)).max() <= 1e-12
        else:
            mean = np.broadcast_to(v[0, 0].mean(axis=0), (N, d))
            assert np.abs(lse[0, 0] - math.log(N)).max() <= 1e-12
        assert np.abs(o[0, 0] - mean).max() <= 1e-12
    # All key rows equal: same as Q = 0 for O, LSE = scale*q.k + ln|J|.
    q = _rand((1, 1, N, d), 23)
    k_eq = np.broadcast_to(k[0, 0, :1], (N, d))[None, None].copy()
    o, lse = orc.attention(q, k_eq, v, scale, False)
    assert np.abs(o[0, 0] - v[0, 0].mean(axis=0)).max() <= 1e-12
    assert np.abs(lse[0, 0] - (scale * q[0, 0] @ k[0, 0, 0] + math.log(N))).max() <= 1e-12
    # Causal row 0 sees only key 0: O_0 = V_0 exactly, LSE_0 = scale * q_0 . k_0.
    o, lse = orc.attention(q, k, v, scale, True)
    assert (o[0, 0, 0] == v[0, 0, 0]).all()
    assert abs(lse[0, 0, 0] - scale * float(q[0, 0, 0] @ k[0, 0, 0])) <= 1e-12
    # Causal row 1 sees keys 0 and 1: a two-term softmax written out.
    s0 = scale * float(q[0, 0, 1] @ k[0, 0, 0])
    s1 = scale * float(q[0, 0, 1] @ k[0, 0, 1])
    w1 = 1.0 / (1.0 + math.exp(s0 - s1))
    assert np.abs(o[0, 0, 1] - ((1 - w1) * v[0, 0, 0] + w1 * v[0, 0, 1])).max() <= 1e-12
    # N = 1: O = V.
    o1, l1 = orc.attention(q[:, :, :1], k[:, :, :1], v[:, :, :1], scale, False)
    assert (o1 == v[:, :, :1]).all()
    # One key wins by >= 50 on every row: O is that key's V row (to e^-50 * N).
    q_hot = np.zeros((1, 1, N, d))
    q_hot[..., 0] = 1.0
    k_hot = np.zeros((1, 1, N, d))
    k_hot[0, 0, 17, 0] = 60.0 / scale
    o, _ = orc.attention(q_hot, k_hot, v, scale, False)
    assert np.abs(o[0, 0] - v[0, 0, 17]).max() <= 1e-15 * N + 1e-20 + math.exp(-60) * N * 10
    # Non-square: query rows independent of d; a d=1 head with scores s_j = scale*q*k_j.
    qs = np.array([[[[0.5], [-2.0]]]])
    ks = np.array([[[[1.0], [3.0]]]])
    vs = np.array([[[[10.0], [20.0]]]])
    o, lse = orc.attention(qs, ks, vs, 0.7, False)
    for i, qi in enumerate((0.5, -2.0)):
        e = [math.exp(0.7 * qi * 1.0), math.exp(0.7 * qi * 3.0)]
        assert abs(o[0, 0, i, 0] - (10 * e[0] + 20 * e[1]) / sum(e)) <= 1e-12
        assert abs(lse[0, 0, i] - math.log(sum(e))) <= 1e-12


# ---------------------------------------------------------------- T7
def check_invariants(orc):
    B, H, N, d = 2, 2, 48, 16
    q, k, v, v2 = (_rand((B, H, N, d), 30 + t, 2.0) for t in range(4))
    scale = 1.0 / math.sqrt(d)
    for causal in (False, True):
        o, lse = orc.attention(q, k, v, scale, causal)
        # convex hull of the visible V rows
        for i in (0, 1, N // 2, N - 1):
            vis = v[:, :, : i + 1] if causal else v
            assert (o[:, :, i] >= vis.min(axis=2) - 1e-12).all()
            assert (o[:, :, i] <= vis.max(axis=2) + 1e-12).all()
        # linear in V
        o2, _ = orc.attention(q, k, v2, scale, causal)
        o3, _ = orc.attention(q, k, 2.0 * v - 3.0 * v2, scale, causal)
        assert np.abs(o3 - (2.0 * o - 3.0 * o2)).max() <= 1e-12
        # max s <= LSE <= max s + ln|J|
        s = scale * np.einsum("bhid,bhjd->bhij", q, k)
        if causal:
            s = np.where(np.tril(np.ones((N, N), dtype=bool)), s, -np.inf)
        smax = s.max(axis=-1)
        cnt = np.arange(1, N + 1) if causal else np.full(N, N)
        assert (lse >= smax - 1e-12).all()
        assert (lse <= smax + np.log(cnt) + 1e-12).all()
        # shifting every key by u adds scale*q_i.u to row i's scores: O unchanged,
        # LSE shifted by exactly that.
        u = _rand((d,), 77)
        o4, lse4 = orc.attention(q, k + u, v, scale, causal)
        assert np.abs(o4 - o).max() <= 1e-12
        assert np.abs(lse4 - (lse + scale * (q @ u))).max() <= 1e-11
    # key permutation (non-causal): permuting K and V rows together changes nothing
    perm = np.random.default_rng(5).permutation(N)
    o, lse = orc.attention(q, k, v, scale, False)
    op, lp = orc.attention(q, k[:, :, perm], v[:, :, perm], scale, False)
    assert np.abs(op - o).max() <= 1e-12 and np.abs(lp - lse).max() <= 1e-12


# ---------------------------------------------------------------- T2
def check_streaming_model(orc):
    """Blockwise merging equals the whole-row softmax, extended to P.V and LSE
    ([P2] 在线Softmax技巧; [P3] FlashAttention与在线softmax)."""
    from streaming_model import streamed_head
    for (n, d, seed) in [(1, 8, 1), (37, 16, 2), (128, 64, 3), (200, 128, 4)]:
        q, k, v = (_rand((n, d), seed * 5 + t, 1.5) for t in range(3))
        scale = 1.0 / math.sqrt(d)
        for causal in (False, True):
            o, lse = orc.attention_head_rows(q, k, v, scale, causal)
            for block in (1, 4, 64):
                so, sl, _ = streamed_head(q, k, v, scale, causal, block)
                assert np.abs(so - o).max() <= 1e-13, (n, d, causal, block)
                assert np.abs(sl - lse).max() <= 1e-13, (n, d, causal, block)


def check_sampled_rows(orc):
    """Row sampling returns exactly the rows of the whole-head computation."""
    q, k, v = (_rand((1, 2, 300, 8), 40 + t) for t in range(3))
    for causal in (False, True):
        o, lse = orc.attention(q, k, v, 0.3, causal)
        rows = np.array([0, 1, 255, 256, 299, 17])
        orow, lrow = orc.attention_rows(q, k, v, 0.3, causal, 0, 1, rows)
        assert np.abs(orow - o[0, 1, rows]).max() <= 1e-15
        assert np.abs(lrow - lse[0, 1, rows]).max() <= 1e-15


ALL_CHECKS = [check_worked_example, check_rows_sum_to_one, check_brute_force,
              check_library_softmax, check_closed_forms, check_invariants,
              check_streaming_model, check_sampled_rows]
