"""CPU oracle for fused scaled-dot-product attention (test infrastructure only).

This package is the checker, not the product.  Only the test suite, the smoke
check and the CPU-baseline leg of the benchmark may import it; the library in
``exact_attention_118_amd`` never does, and the two share no code.

It computes, in float64 and with the full score matrix S and probability matrix
P materialised, exactly what the fused kernels compute tile by tile:

* forward  -- O = softmax(scale * Q K^T + mask) V and the per-row natural-log
  logsumexp L (the CSDN post "Flash Attention1", "Flash Attention" section, the three-line formula;
  the 51CTO FlashAttention V1/V2 notes, "FlashAttention V2 相比 V1 有哪些改进": the backward pass keeps only L);
* backward -- dQ, dK, dV of f = sum(dO * O), recomputing P from the inputs
  (the Huawei Cloud post "FlashAttention", section 3 "Recomputation"; the 51CTO FlashAttention V1/V2 notes names the auxiliary row vector D).

Dropout's random bits come from Philox4x32-10 (``oracle.philox``), written
from its published definition and pinned by the generator authors' known-answer
vectors (tests/golden/philox4x32_kat.json).

Every function is pinned by CPU tests against facts that do not come from this
code: hand-derived closed forms (tests/golden), the page-1 online-softmax
walk-through re-implemented independently, finite differences, algebraic
identities of softmax, and torch's own attention on small shapes.
"""

from .attention import (  # noqa: F401
    attention_backward,
    attention_backward_batched,
    attention_forward,
    attention_forward_batched,
    attention_forward_rows,
    causal_visible,
    scores,
    softmax_with_lse,
)
from .philox import (  # noqa: F401
    dropout_bytes,
    dropout_multiplier,
    dropout_multiplier_batched,
    keep_threshold,
    philox4x32,
)
