"""Test-only fp64 model of the streamed (online-softmax) attention forward.

It walks the keys in blocks, keeping per query row the running maximum m, the
running exponential sum l and the unnormalised output acc; when m grows, l and
acc are multiplied by exp(m_old - m_new); after the last block O = acc / l and
the logsumexp is m + ln l.  ([P2] 为什么Flash Attention能将注意力计算提速数倍而不损失精度,
在线Softmax技巧 two-block merge; [P3] GPU Kernel 入门：Triton / FlashAttention,
FlashAttention与在线softmax.)  It is written separately from the oracle so that
agreement between the two pins the oracle's whole-row definition.
"""
from __future__ import annotations

import numpy as np


def streamed_head(q, k, v, scale, causal, block):
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    n = q.shape[0]
    m = np.full(n, -np.inf)
    l = np.zeros(n)
    acc = np.zeros((n, v.shape[1]))
    rows = np.arange(n)
    moved_after_first = np.zeros(n, dtype=bool)
    for j0 in range(0, k.shape[0], block):
        kb = k[j0:j0 + block]
        vb = v[j0:j0 + block]
        s = scale * (q @ kb.T)
        if causal:
            keys = np.arange(j0, j0 + kb.shape[0])
            s = np.where(keys[None, :] <= rows[:, None], s, -np.inf)
        blk_max = s.max(axis=1)
        m_new = np.maximum(m, blk_max)
        if j0 > 0:
            moved_after_first |= m_new > m
        safe = np.where(np.isfinite(m_new), m_new, 0.0)
        shrink = np.where(np.isfinite(m), np.exp(m - safe), 0.0)
        p = np.exp(s - safe[:, None])
        l = l * shrink + p.sum(axis=1)
        acc = acc * shrink[:, None] + p @ vb
        m = m_new
    return acc / l[:, None], m + np.log(l), moved_after_first


def reference_moves(q, k, scale, causal, block, slack_log2):
    """Count, per query row, how often a lazily held reference maximum moves
    after the first key block: the reference (in log2 units of the scaled
    score) is replaced by the block's row maximum only when that maximum
    exceeds it by more than `slack_log2`.  slack_log2 = 0 gives the moves of
    the plain running maximum.  Returns an int array of move counts per row.
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    n = q.shape[0]
    rows = np.arange(n)
    ref = np.full(n, -np.inf)
    moves = np.zeros(n, dtype=np.int64)
    for j0 in range(0, k.shape[0], block):
        kb = k[j0:j0 + block]
        s = scale * (q @ kb.T) / np.log(2.0)
        if causal:
            keys = np.arange(j0, j0 + kb.shape[0])
            s = np.where(keys[None, :] <= rows[:, None], s, -np.inf)
        blk_max = s.max(axis=1)
        grow = blk_max > ref + slack_log2
        if j0 > 0:
            moves += grow
        ref = np.where(grow, blk_max, ref)
    return moves
