"""Plain fp64 CPU oracle for exact attention (test infrastructure only).

This package is the checker, not the product. Only the tests, the smoke entry
point and the benchmark's CPU-baseline leg may import it; the GPU path never
does, and it imports nothing from the GPU path.

Pages cited (by title or address, and by section; their text is the authority
on what the method computes):

* [wiki]      aiboss88.com wiki, "什么是 FlashAttention？一种 IO 感知的精确注意力算法"
              -- what the method is; "exact, not approximate".
* [interview] meko1 LLM interview guide, "FlashAttention 深入" -- standard
              attention, online softmax, recompute backward.
* [scratch]   l189.com/news/1255901 (an article implementing Flash Attention
              from scratch in PyTorch; numbered sections) -- §1.1 standard
              attention, §2.2 online softmax and its worked example, §3.1
              blocked forward, §3.3 backward and the softmax Jacobian, §5.2
              numerical stability, §5.3 causal mask.
* [notes]     claire-chang.com/post/flashattention-introduction, section
              "flash_attn 的程式碼怎麼寫？" -- the ``flash_attn_qkvpacked_func``
              docstring: (batch, seqlen, nheads, headdim) layout, softmax_scale
              default 1/sqrt(headdim), causal flag, inclusive sliding window.
"""

from .attention import (  # noqa: F401
    visible_mask,
    attention_forward,
    attention_forward_rows,
    attention_backward,
    visible_pair_count,
)
from .online import online_softmax_trace, blocked_online_forward  # noqa: F401
