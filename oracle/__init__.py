"""Oracle for the FlashMask forward pass -- TEST INFRASTRUCTURE ONLY.

A plain, slow, float64 CPU statement of what the method computes, used to
check the HIP path.  Only the tests, the package smoke check and the CPU
baseline leg of the benchmark may import it; the product path never does.

It shares no code with the HIP library: it expands the interval mask to a
dense boolean matrix and evaluates softmax attention row by row from its
definition, with no tiling and no online recurrence.

Sources (web pages, cited by title and section):

* "FlashMask技术：大模型训练中的高效注意力掩码优化" (the FlashMask article):
  §1 per-query key range [col_start[i], col_end[i]] replacing the dense
  N x N mask; §2.1 interval vectors; §2.2 three-way (skip / full / masked)
  tile decision that keeps results mathematically equivalent; §3.3 document
  packing intervals; §4.1 item 3 inclusive element compare fused into the
  score.
* "FlashAttention优化：高效训练长上下文GPT的技术突破" (the FlashAttention
  article): §2 item 2, softmax of scaled scores q_i.k_j/sqrt(d) with max
  subtraction.
* "FlashMask: Efficient and Rich Mask Extension of FlashAttention"
  (abstract): skipping masked work does not change accuracy; the method is
  used in training, which needs the gradients (``attention_bwd``: the chain
  rule through the forward definition).

Every function here is pinned by CPU tests against values fixed by the
pages or by mathematics (closed forms, invariants, brute force, library
routines); none is "parity unpinned".
"""
from .attention import attention, attention_weights, dense_mask, bf16_round
from .backward import attention_bwd
from .tiles import (SKIP, FULL, PARTIAL, classes_minmax, classes_minmax_multi, classes_dense,
                    nonskip_counts, unmasked_count)

__all__ = ["attention", "attention_weights", "attention_bwd", "dense_mask", "bf16_round",
           "SKIP", "FULL", "PARTIAL", "classes_minmax", "classes_minmax_multi", "classes_dense",
           "nonskip_counts", "unmasked_count"]
