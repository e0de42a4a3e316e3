"""Checks that pin the CPU oracle's attention gradients to facts outside it.

Each check takes a module exposing attention_bwd (the oracle, or a broken
copy of it in tests/test_oracle_bwd_mutations.py).

The pages fix the backward pass only as recomputation of S and P from Q, K
and V ([P2] 为什么Flash Attention能将注意力计算提速数倍而不损失精度,
反向传播中的重计算策略); the numbers it must produce are the gradients of the
forward's output.  So the pins here are the definition of a gradient (central
finite differences of a scalar-loop forward written in this file), an
independent library's autograd, exact identities and special cases.
"""
from __future__ import annotations

import math

import numpy as np
import torch


def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).normal(size=shape) * scale


def loop_forward(q, k, v, scale, causal):
    """O for one head by scalar loops (math.exp, math.fsum)."""
    n, d = q.shape
    o = np.zeros((n, v.shape[1]))
    for i in range(n):
        keys = range(i + 1) if causal else range(k.shape[0])
        s = [scale * math.fsum(q[i, c] * k[j, c] for c in range(d)) for j in keys]
        m = max(s)
        e = [math.exp(x - m) for x in s]
        l = math.fsum(e)
        for c in range(v.shape[1]):
            o[i, c] = math.fsum(e[t] * v[j, c] for t, j in enumerate(keys)) / l
    return o


def finite_difference_grads(q, k, v, do, scale, causal, h=1e-5):
    """Central differences of L = sum(O * dO) with respect to every input element."""
    grads = []
    for which in range(3):
        args = [q.copy(), k.copy(), v.copy()]
        g = np.zeros_like(args[which])
        for idx in np.ndindex(*g.shape):
            plus = [a.copy() for a in args]
            minus = [a.copy() for a in args]
            plus[which][idx] += h
            minus[which][idx] -= h
            lp = float(np.sum(loop_forward(*plus, scale, causal) * do))
            lm = float(np.sum(loop_forward(*minus, scale, causal) * do))
            g[idx] = (lp - lm) / (2 * h)
        grads.append(g)
    return grads


def torch_grads(q, k, v, do, scale, causal):
    """torch CPU fp64 autograd of softmax(scale q k^T [mask]) v, an independent route."""
    qt, kt, vt = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    s = torch.matmul(qt, kt.transpose(-1, -2)) * scale
    if causal:
        n = s.shape[-1]
        s = s.masked_fill(torch.ones(n, n, dtype=torch.bool).triu(1), float("-inf"))
    o = torch.matmul(torch.softmax(s, dim=-1), vt)
    o.backward(torch.tensor(do, dtype=torch.float64))
    return qt.grad.numpy(), kt.grad.numpy(), vt.grad.numpy()


# ---------------------------------------------------------------- B1
def check_finite_differences(orc):
    for (n, d, seed) in [(5, 3, 1), (4, 2, 2), (6, 4, 3)]:
        for causal in (False, True):
            q, k, v, do = (_rand((n, d), seed * 10 + t, 0.8) for t in range(4))
            scale = 1.0 / math.sqrt(d)
            dq, dk, dv = orc.attention_bwd(q[None, None], k[None, None], v[None, None], do[None, None],
                                           scale, causal)
            fq, fk, fv = finite_difference_grads(q, k, v, do, scale, causal)
            for got, ref in ((dq[0, 0], fq), (dk[0, 0], fk), (dv[0, 0], fv)):
                assert np.abs(got - ref).max() <= 1e-7, (n, d, causal)


# ---------------------------------------------------------------- B2
def check_library_autograd(orc):
    for (shape, seed) in [((1, 1, 64, 16), 4), ((2, 2, 33, 8), 5), ((1, 1, 300, 64), 6)]:
        for causal in (False, True):
            q, k, v, do = (_rand(shape, seed * 10 + t) for t in range(4))
            scale = 1.0 / math.sqrt(shape[-1])
            got = orc.attention_bwd(q, k, v, do, scale, causal)
            ref = torch_grads(q, k, v, do, scale, causal)
            for g, r in zip(got, ref):
                assert np.abs(g - r).max() <= 1e-12 * max(1.0, np.abs(r).max()), (shape, causal)


# ---------------------------------------------------------------- B3
def check_identities(orc):
    """Rows of P sum to 1, so the key-sum of dV is the query-sum of dO; rows of
    dS sum to 0, so the key-sum of dK vanishes.  Both hold with the mask."""
    for causal in (False, True):
        q, k, v, do = (_rand((2, 3, 50, 16), 30 + t) for t in range(4))
        dq, dk, dv = orc.attention_bwd(q, k, v, do, 0.3, causal)
        assert np.abs(dv.sum(axis=2) - do.sum(axis=2)).max() <= 1e-12
        assert np.abs(dk.sum(axis=2)).max() <= 1e-12 * np.abs(dk).sum(axis=2).max()


# ---------------------------------------------------------------- B4
def check_special_cases(orc):
    n, d = 24, 8
    k, v, do = (_rand((1, 1, n, d), 40 + t) for t in range(3))
    q = _rand((1, 1, n, d), 43)
    # causal row 0 sees one key with weight 1: its softmax Jacobian is 0
    dq, _, _ = orc.attention_bwd(q, k, v, do, 0.5, True)
    assert np.all(dq[0, 0, 0] == 0.0)
    # Q = 0, no mask: uniform weights, every key's dV is the mean of dO; dK = 0
    dq, dk, dv = orc.attention_bwd(np.zeros_like(q), k, v, do, 0.5, False)
    assert np.abs(dv[0, 0] - do[0, 0].mean(axis=0)[None, :]).max() <= 1e-13
    assert np.all(dk == 0.0)
    # V = 0: dP = 0, so dQ = dK = 0
    dq, dk, dv = orc.attention_bwd(q, k, np.zeros_like(v), do, 0.5, True)
    assert np.all(dq == 0.0) and np.all(dk == 0.0)
    # N = 1: O = V, so dV = dO and the other two vanish
    dq, dk, dv = orc.attention_bwd(q[:, :, :1], k[:, :, :1], v[:, :, :1], do[:, :, :1], 0.5, False)
    assert np.all(dv == do[:, :, :1]) and np.all(dq == 0.0) and np.all(dk == 0.0)


ALL_BWD_CHECKS = [check_finite_differences, check_library_autograd, check_identities,
                  check_special_cases]
