"""Plain fp64 attention: S and P are formed in full, row by row.

TEST INFRASTRUCTURE ONLY (see the package docstring for the page keys).

What is computed, per batch b and head h, for query row i (0-based):

    visible keys J_i = {0..N-1}, or {0..i} under the lower-triangular mask
    s_ij   = scale * sum_c q_ic k_jc                 S = Q K^T         [P2 标准注意力机制的内存困局]
    m_i    = max_{j in J_i} s_ij                     safe softmax      [P2 在线Softmax技巧]
    l_i    = sum_{j in J_i} exp(s_ij - m_i)
    P_ij   = exp(s_ij - m_i) / l_i (j in J_i), else 0  final normalisation [P1 在线Softmax, 最终归一化]
    O_ic   = sum_j P_ij v_jc                         O = P V           [P2 标准注意力机制的内存困局]
    LSE_i  = m_i + ln(l_i)                           the per-row statistics the tiled method keeps
                                                     besides O [P2 分块计算(Tiling)]; stored as one
                                                     natural-log logsumexp

The tiled method reaches exactly this result (up to rounding order): [P2]
在线Softmax技巧 ends with the statement that the merged result equals the
standard one, and [P3] FlashAttention与在线softmax says the same.  So this
module is that definition written out, with whole rows of S and P formed
before their max and sum are taken.  Rows are processed in blocks only to
bound memory; rows are independent, so that changes nothing.  Under the mask
the keys past the block's last row are left out of the product, which is the
same as multiplying them by an exact 0.

Inputs are float64 arrays (bf16 values convert to fp64 exactly).
"""
from __future__ import annotations

import numpy as np

ROW_BLOCK = 256


def softmax_rows(x: np.ndarray) -> np.ndarray:
    """Safe softmax of every row: exp(x - max x) / sum exp(x - max x).  [P2 在线Softmax技巧]"""
    x = np.asarray(x, dtype=np.float64)
    e = np.exp(x - x.max(axis=-1, keepdims=True))
    return e / e.sum(axis=-1, keepdims=True)


def online_softmax_rows(x: np.ndarray, block: int) -> np.ndarray:
    """Softmax of every row computed by streaming over blocks of `block` columns.

    Follows the online normaliser: the running maximum m and the running sum
    l of exp(x - m) are updated per block, l and the unnormalised outputs
    already produced are multiplied by exp(m_old - m_new) when the maximum
    grows, and the outputs are divided by l once at the end
    ([P1 在线Softmax, 两种情况统一]; [P2 在线Softmax技巧, two-block merge];
    [P3 FlashAttention与在线softmax, the three running statistics]).
    Here the "output" of a row is its own row of unnormalised weights, as in
    the worked example of [P3 动手, 第一段].
    """
    x = np.asarray(x, dtype=np.float64)
    rows, cols = x.shape
    m = np.full(rows, -np.inf)
    l = np.zeros(rows)
    out = np.zeros((rows, cols))
    for start in range(0, cols, block):
        blk = x[:, start:start + block]
        m_new = np.maximum(m, blk.max(axis=1))
        shrink = np.exp(m - m_new)               # exp(m_old - m_new); 0 on the first block
        weights = np.exp(blk - m_new[:, None])
        l = shrink * l + weights.sum(axis=1)
        out = out * shrink[:, None]
        out[:, start:start + block] = weights
        m = m_new
    return out / l[:, None]


def _row_block(q_rows, k, v, scale, causal, row_ids, want_p=False):
    """O, LSE (and P) for the query rows `row_ids` of one head."""
    if causal:
        n_keys = int(row_ids.max()) + 1          # keys beyond the last row are all masked
        k = k[:n_keys]
        v = v[:n_keys]
    s = scale * (q_rows @ k.T)                   # full rows of S, fp64
    if causal:
        key_ids = np.arange(k.shape[0])
        s = np.where(key_ids[None, :] <= row_ids[:, None], s, -np.inf)
    m = s.max(axis=1)
    e = np.exp(s - m[:, None])                   # exp(-inf) is exactly 0 for masked keys
    l = e.sum(axis=1)
    p = e / l[:, None]
    o = p @ v
    lse = m + np.log(l)
    return (o, lse, p) if want_p else (o, lse)


def attention_head_rows(q, k, v, scale, causal, rows=None, row_block=ROW_BLOCK):
    """O [R, d] and LSE [R] for the given query rows of one head (all rows if None).

    q, k, v: float64 [N, d].
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    n = q.shape[0]
    rows = np.arange(n) if rows is None else np.asarray(rows, dtype=np.int64)
    o = np.empty((rows.size, v.shape[1]))
    lse = np.empty(rows.size)
    for start in range(0, rows.size, row_block):
        ids = rows[start:start + row_block]
        o[start:start + ids.size], lse[start:start + ids.size] = _row_block(
            q[ids], k, v, float(scale), bool(causal), ids)
    return o, lse


def probs_head(q, k, scale, causal):
    """The full probability matrix P [N, N] of one head (small N only)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    n = q.shape[0]
    rows = np.arange(n)
    dummy_v = np.zeros((k.shape[0], 1))
    _, _, p = _row_block(q, k, dummy_v, float(scale), bool(causal), rows, want_p=True)
    if causal:                                   # re-pad the sliced key range to N columns
        full = np.zeros((n, k.shape[0]))
        full[:, :p.shape[1]] = p
        p = full
    return p


def attention(q, k, v, scale, causal):
    """O [B, H, N, d] and LSE [B, H, N] for float64 inputs of shape [B, H, N, d]."""
    q = np.asarray(q, dtype=np.float64)
    B, H, N, d = q.shape
    o = np.empty((B, H, N, v.shape[-1]))
    lse = np.empty((B, H, N))
    for b in range(B):
        for h in range(H):
            o[b, h], lse[b, h] = attention_head_rows(q[b, h], k[b, h], v[b, h], scale, causal)
    return o, lse


def attention_rows(q, k, v, scale, causal, b, h, rows):
    """O and LSE of selected query rows of head (b, h); inputs [B, H, N, d]."""
    return attention_head_rows(q[b, h], k[b, h], v[b, h], scale, causal, rows)
