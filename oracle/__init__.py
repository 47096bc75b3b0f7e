"""Reference oracle for the attention forward: plain, slow, fp64, CPU only.

This package is test infrastructure. Only the tests, the smoke check and the
benchmark's CPU-baseline leg import it; the GPU library never does, and it shares
no code, tables or helpers with the HIP path.

Sources (the three pages on IO-aware softmax attention):
  * "Flash Attention (FA1)" (languisher.top), section "Naive Attention 问题分析":
    safe softmax definition m(x) = max_i x_i, softmax = e^{x-m} / sum e^{x-m}.
  * "01 · 注意力为什么是 IO 瓶颈" (ai-reference-codex), section 3 table and
    section 5 pseudocode: the three textbook steps S = QK^T, P = softmax(S), O = PV.
  * "Flash Attention (FA1)", section "核心局部状态计算和更新公式推导", steps 1-5:
    the per-tile update of (m_i, l_i, O_i).
  * The same page's tiling section: T_r = ceil(N/B_r), T_c = ceil(N/B_c).
  * The same update (steps 2 and 4-5) applied to whole key chunks: the merge of
    partial results of the split over keys (attention_split_fp64).

backward.py holds the gradients of the forward (the chain rule through its three
steps; the pages give no backward formulas, see its docstring).

Every function is pinned by tests that do not re-type its formulas (closed forms,
invariants, brute force, library special cases); the two bf16 yardsticks
(attention_unfused_bf16, attention_backward_unfused_bf16) also by hand-derived values
on inputs whose every fp32 step is exact, so that each of their bf16 rounding points
decides the expected bits (tests/golden/yardstick_cases.json). No function here is
"parity unpinned".
"""
from .backward import attention_backward_fp64, attention_backward_unfused_bf16  # noqa: F401
from .attention import (  # noqa: F401
    attention_fp64,
    attention_online_fp64,
    attention_split_fp64,
    attention_brute_force,
    attention_unfused_bf16,
)
