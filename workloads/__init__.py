"""Seeded synthetic inputs for the attention forward workloads.

This module holds shapes, seeds and random draws only: none of the attention
arithmetic.  Both the CPU oracle (via the tests) and the HIP path take their
inputs from here, so the two sides see the same bf16 bits.

Shapes follow the workloads of the pages on IO-aware exact attention
("FlashAttention的Triton实现" and "为什么Flash Attention能将注意力计算提速数倍…"):
per-head Q, K, V of shape N x d in HBM, d in {64, 128}, long sequences
(16K tokens as the headline case) with and without the lower-triangular mask.
The value distribution is N(0, 1) for every tensor; the last workload scales
everything by 0.5 and multiplies 1% of the key rows of every head by 8, so a
few keys dominate their rows and the running maximum keeps moving.
"""
from __future__ import annotations

import hashlib
import math
from dataclasses import dataclass, asdict

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    d: int
    causal: bool
    peaky: bool = False      # 0.5 x N(0,1), 1% of K rows x 8
    seed: int = 0

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    def as_dict(self) -> dict:
        dct = asdict(self)
        dct["scale"] = self.scale
        return dct


# The five workloads: a tiny single head, a mid-size batch, the 16K-token
# causal headline case, many short sequences at d=64, and a 64K-token causal
# case with peaky keys.  Seed k belongs to the k-th workload.
WORKLOADS = {
    "tiny_b1h1_n256_d64": Workload("tiny_b1h1_n256_d64", 1, 1, 256, 64, False, seed=1),
    "mid_b4h16_n4096_d128": Workload("mid_b4h16_n4096_d128", 4, 16, 4096, 128, False, seed=2),
    "causal_b1h32_n16384_d128": Workload("causal_b1h32_n16384_d128", 1, 32, 16384, 128, True, seed=3),
    "short_b16h32_n2048_d64": Workload("short_b16h32_n2048_d64", 16, 32, 2048, 64, False, seed=4),
    "causal_peaky_b1h8_n65536_d128": Workload("causal_peaky_b1h8_n65536_d128", 1, 8, 65536, 128, True,
                                              peaky=True, seed=5),
}
WORKLOAD_ORDER = list(WORKLOADS)
HEADLINE = "causal_b1h32_n16384_d128"


def custom(B: int, H: int, N: int, d: int, causal: bool, seed: int, peaky: bool = False) -> Workload:
    return Workload(f"b{B}h{H}n{N}d{d}{'c' if causal else ''}{'p' if peaky else ''}",
                    B, H, N, d, causal, peaky, seed)


def make_inputs(w: Workload, seed: int | None = None):
    """Return (q, k, v) as contiguous CPU bf16 tensors of shape [B, H, N, d].

    Draw order: Q, K, V from one CPU generator seeded with `seed` (default:
    the workload's own), each as float32 N(0,1), rounded to bf16 (round to
    nearest even) at the end.  For the peaky workload all three are halved and,
    per (b, h) in row-major order, the first floor(0.01 N) entries of a random
    permutation of the N key rows are multiplied by 8.  Both factors are powers
    of two, so doing them before the bf16 rounding changes no bits.
    """
    g = torch.Generator(device="cpu")
    g.manual_seed(w.seed if seed is None else seed)
    shape = (w.B, w.H, w.N, w.d)
    q = torch.randn(shape, dtype=torch.float32, generator=g)
    k = torch.randn(shape, dtype=torch.float32, generator=g)
    v = torch.randn(shape, dtype=torch.float32, generator=g)
    if w.peaky:
        q.mul_(0.5)
        k.mul_(0.5)
        v.mul_(0.5)
        n_hot = int(math.floor(0.01 * w.N))
        for b in range(w.B):
            for h in range(w.H):
                idx = torch.randperm(w.N, generator=g)[:n_hot]
                k[b, h, idx, :] *= 8.0
    return (q.to(torch.bfloat16).contiguous(), k.to(torch.bfloat16).contiguous(),
            v.to(torch.bfloat16).contiguous())


def sha256_of(t: torch.Tensor) -> str:
    """SHA-256 of a tensor's raw bytes (bf16 viewed as int16)."""
    raw = t.contiguous().view(torch.int16).numpy().tobytes() if t.dtype == torch.bfloat16 \
        else t.contiguous().numpy().tobytes()
    return hashlib.sha256(raw).hexdigest()


GRAD_SEED_OFFSET = 7919


def make_grad(w: Workload, seed: int | None = None):
    """The upstream gradient dO for the backward pass: a contiguous CPU bf16
    tensor [B, H, N, d] of N(0,1) draws (float32, then round to nearest even),
    from its own CPU generator seeded with the workload's seed plus 7919 (or
    `seed` plus 7919), so it is independent of Q, K and V."""
    g = torch.Generator(device="cpu")
    g.manual_seed((w.seed if seed is None else seed) + GRAD_SEED_OFFSET)
    x = torch.randn((w.B, w.H, w.N, w.d), generator=g, dtype=torch.float32)
    return x.to(torch.bfloat16).contiguous()



FP8_SIGN_SEED_OFFSET = 104729
OUTLIER_CHANNELS = (5, 77)
OUTLIER_FACTOR = 16.0


def make_fp8_signs(seed: int, d: int = 128) -> int:
    """The random sign mask of the FP8 path's Hadamard rotation, as an integer
    of d bits (bit c set: channel c negated), drawn from its own CPU generator
    seeded with seed + 104729."""
    g = torch.Generator(device="cpu")
    g.manual_seed(seed + FP8_SIGN_SEED_OFFSET)
    bits = torch.randint(0, 2, (d,), generator=g).tolist()
    return sum(int(b) << c for c, b in enumerate(bits))


def make_outlier_inputs(w: Workload, seed: int | None = None):
    """(q, k, v) as make_inputs, then in Q and K the channels OUTLIER_CHANNELS
    (those below d) multiplied by OUTLIER_FACTOR (a power of two, so no bf16
    bits change besides the exponent): a few large channels shared by Q and
    K, the situation the FP8 path's rotation is meant for."""
    q, k, v = make_inputs(w, seed)
    ch = [c for c in OUTLIER_CHANNELS if c < w.d]
    q = q.clone()
    k = k.clone()
    q[..., ch] *= OUTLIER_FACTOR
    k[..., ch] *= OUTLIER_FACTOR
    return q.contiguous(), k.contiguous(), v
