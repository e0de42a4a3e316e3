"""Work and traffic accounting for the attention forward (host-side, no GPU).

FLOPs count the two matrix products only, 2*N*N*d each per head, i.e.
4*B*H*N^2*d, halved under the lower-triangular mask.  The method removes no
arithmetic; it removes the N x N intermediates' trips to HBM
([P3] GPU Kernel 入门：Triton / FlashAttention, section 边界与取舍; [P2] 为什么Flash
Attention能将注意力计算提速数倍而不损失精度, section 核函数融合).

Compulsory HBM bytes are what any implementation must move: read Q, K, V
(bf16) once, write O (bf16) and the fp32 logsumexp once.  The materialised
variant adds the N x N score matrix written and read back, the quantity the
pages price at N=4096 ([P3] 动手, part 2).
"""
from __future__ import annotations

MIB = 1 << 20

# MI355X published peaks used as roofline denominators.
PEAK_BF16_DENSE_TFLOPS = 2516.6     # 256 CU x 4096 FLOP/clk/CU x 2.4 GHz
PEAK_FP8_DENSE_TFLOPS = 5033.2      # twice the bf16 rate (E4M3 / E5M2 MFMA)
PEAK_HBM_GBPS = 8000.0


def attention_flops(B: int, H: int, N: int, d: int, causal: bool) -> float:
    f = 4.0 * B * H * N * N * d
    return f / 2.0 if causal else f


def attention_bwd_flops(B: int, H: int, N: int, d: int, causal: bool) -> float:
    """Algorithmic FLOPs of the recomputation backward: five N x N x d
    products (S again, dP, dV, dQ, dK) against the forward's two, 2.5x."""
    return 2.5 * attention_flops(B, H, N, d, causal)


def compulsory_bytes(B: int, H: int, N: int, d: int, in_bytes: int = 2, out_bytes: int = 2,
                     lse_bytes: int = 4) -> int:
    return B * H * (3 * N * d * in_bytes + N * d * out_bytes + N * lse_bytes)


def score_matrix_bytes(N: int, elem_bytes: int) -> int:
    """Bytes of one N x N matrix (S or P) for one head."""
    return N * N * elem_bytes


def score_round_trip_bytes(N: int, elem_bytes: int) -> int:
    """The N x N score matrix written to HBM and read back once."""
    return 2 * score_matrix_bytes(N, elem_bytes)


def kv_tile_stream_bytes(B: int, H: int, N: int, d: int, block_rows: int, causal: bool,
                         elem_bytes: int = 2) -> float:
    """K and V bytes that all query blocks of the tiled forward read (any cache level)."""
    n_qb = -(-N // block_rows)
    per_block = 2.0 * N * d * elem_bytes
    total = B * H * n_qb * per_block
    return total * (n_qb + 1) / (2.0 * n_qb) if causal else total
