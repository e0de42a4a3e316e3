"""Plain fp64 gradients of exact attention: S and P are formed in full.

TEST INFRASTRUCTURE ONLY (see the package docstring for the page keys).

The pages describe the backward pass of the tiled method only by what it
keeps: the forward stores O and the per-row statistics, and the backward
recomputes S and P from Q, K and V on chip instead of reading them back
([P2] 反向传播中的重计算策略).  The result it must reach is the plain one: the
gradients of the forward output O = softmax(scale Q K^T [mask]) V with
respect to Q, K and V, for an upstream gradient dO.  This module writes that
out by the chain rule, per batch b and head h:

    P      = softmax over the visible keys of S = scale Q K^T   (as in the forward oracle)
    dV     = P^T dO                       O = P V, so dO/dV contracts P over the query rows
    dP     = dO V^T
    D_i    = sum_j P_ij dP_ij             softmax Jacobian diag(p) - p p^T applied to dP
    dS_ij  = P_ij (dP_ij - D_i)           (0 on masked entries, where P_ij = 0)
    dQ     = scale dS K
    dK     = scale dS^T Q

Whole rows of S and P are formed before anything is taken from them.  Query
rows are processed in blocks only to bound memory: dQ rows are independent,
and the dK, dV sums over query rows are split across the blocks and added up
(a split of one sum, nothing else).  Under the mask the keys past a block's
last row are left out, which is the same as multiplying them by an exact 0.

Inputs are float64 arrays (bf16 values convert to fp64 exactly).
"""
from __future__ import annotations

import numpy as np

ROW_BLOCK = 256


def attention_bwd_span(q, k, v, do, scale, causal, r0, r1, row_block=ROW_BLOCK):
    """Query rows [r0, r1) of one head (q, k, v, do: [N, d] arrays): their dQ
    rows ([r1 - r0, d]) and their shares of dK and dV, the sums over these
    rows only ([n_keys, d], n_keys = r1 under the mask, where later keys get
    nothing from these rows, else N).  dQ rows are independent, so spans that
    cover every row once give the head's dQ, and their shares add up to its
    dK and dV."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    do = np.asarray(do, np.float64)
    n_span_keys = r1 if causal else k.shape[0]
    dq = np.zeros((r1 - r0, q.shape[1]))
    dk = np.zeros((n_span_keys, k.shape[1]))
    dv = np.zeros((n_span_keys, v.shape[1]))
    for b0 in range(r0, r1, row_block):
        row_ids = np.arange(b0, min(b0 + row_block, r1))
        n_keys = int(row_ids.max()) + 1 if causal else k.shape[0]
        kk = k[:n_keys]
        s = scale * (q[row_ids] @ kk.T)
        if causal:
            key_ids = np.arange(n_keys)
            s = np.where(key_ids[None, :] <= row_ids[:, None], s, -np.inf)
        m = s.max(axis=1)
        e = np.exp(s - m[:, None])
        p = e / e.sum(axis=1)[:, None]
        dv[:n_keys] += p.T @ do[row_ids]
        dp = do[row_ids] @ v[:n_keys].T
        d_row = (p * dp).sum(axis=1)
        ds = p * (dp - d_row[:, None])
        dq[row_ids - r0] = scale * (ds @ kk)
        dk[:n_keys] += scale * (ds.T @ q[row_ids])
    return dq, dk, dv


def attention_bwd_head(q, k, v, do, scale, causal, row_block=ROW_BLOCK):
    """(dQ, dK, dV) of one head: q, k, v, do are [N, d] arrays.  One span
    holding every query row."""
    return attention_bwd_span(q, k, v, do, scale, causal, 0, np.shape(q)[0], row_block)


def attention_bwd(q, k, v, do, scale, causal):
    """(dQ, dK, dV) for [B, H, N, d] arrays."""
    q = np.asarray(q, np.float64)
    dq = np.zeros_like(q)
    dk = np.zeros(np.shape(k), np.float64)
    dv = np.zeros(np.shape(v), np.float64)
    for b in range(q.shape[0]):
        for h in range(q.shape[1]):
            dq[b, h], dk[b, h], dv[b, h] = attention_bwd_head(q[b, h], k[b, h], v[b, h], do[b, h],
                                                              scale, causal)
    return dq, dk, dv


def attention_bwd_rows(q, k, v, do, scale, causal, rows):
    """dQ of the given query rows of one head only ([len(rows), d]); cheap
    enough for the largest shapes.  Same formulas as attention_bwd_head."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    do = np.asarray(do, np.float64)
    out = np.zeros((len(rows), q.shape[1]))
    for t, i in enumerate(rows):
        n_keys = i + 1 if causal else k.shape[0]
        kk = k[:n_keys]
        s = scale * (kk @ q[i])
        e = np.exp(s - s.max())
        p = e / e.sum()
        dp = v[:n_keys] @ do[i]
        ds = p * (dp - (p * dp).sum())
        out[t] = scale * (ds @ kk)
    return out
