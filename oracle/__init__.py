"""CPU fp64 oracle for exact attention, forward and gradients -- TEST INFRASTRUCTURE.

Only the tests, the package's smoke check and the benchmark's CPU-baseline leg
may import this package.  The product path (the HIP library and its Python
binding) never calls it and shares no code with it.

Sources cited in this package (pages on IO-aware exact attention):
  [P1] "FlashAttention的Triton实现：IO-aware注意力机制底层原理" (jsqmd.com)
  [P2] "为什么Flash Attention能将注意力计算提速数倍而不损失精度：从GPU内存墙到IO感知算法的技术突围"
       (answer.freetools.me)
  [P3] "GPU Kernel 入门：Triton / FlashAttention" (ai.clawlihai.cn)

The FP8 forward (oracle/fp8.py: the E4M3 format, per-head quantisation with
incoherent processing, attention with P rounded to E4M3) is imported as
`oracle.fp8`.

Pinned by the CPU tests (tests/test_oracle_pins.py, tests/test_oracle_bwd_pins.py,
tests/test_oracle_fp8_pins.py):
the printed worked example of [P3] 动手, brute-force scalar evaluation, an
independent library softmax and autograd, central finite differences of the
forward, closed forms, invariants; for FP8 the format's definition, an
exhaustive nearest-value search, Hadamard algebra, exact scaling identities
and a hand-computed example.  No function here is "parity unpinned".
"""
from .attention import (softmax_rows, online_softmax_rows, attention_head_rows,
                        attention, attention_rows, probs_head)
from .attention_bwd import attention_bwd_head, attention_bwd, attention_bwd_rows, attention_bwd_span

__all__ = ["softmax_rows", "online_softmax_rows", "attention_head_rows", "attention",
           "attention_rows", "probs_head", "attention_bwd_head", "attention_bwd",
           "attention_bwd_rows", "attention_bwd_span"]
