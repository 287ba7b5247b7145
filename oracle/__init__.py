"""CPU oracle for masked softmax attention (forward, backward, tile classes, block index).

TEST INFRASTRUCTURE ONLY. Nothing on the product path imports, calls or links this
package: it is used by ``tests/``, by the entry-point smoke check and by the bench's
``cpu_baseline`` leg (timing the oracle on the host). It shares no code, constants
or helpers with the HIP implementation; both sides receive the same seeded inputs.

What it computes is the plain textbook definition, in fp64:
  * the boolean mask M[i, j] materialised from a per-element predicate for each of the
    mask kinds named on "LongCA-bench: 长上下文注意力基准测试" (xllm-io blog),
    section 三 "注意力掩码模式" (regular, heterogeneous and dynamic block masks);
  * S = scale * Q K^T with S[~M] = -inf, row softmax P, O = P V, LSE = log-sum-exp;
  * the explicit backward dQ, dK, dV of that definition;
  * tile classes (EMPTY / PARTIAL / FULL) and CSR/CSC tile lists by brute force over
    the materialised mask, and CSR/CSC lists of a block-sparse keep matrix;
  * the count U of visible (query, key) pairs, from which effective FLOPs follow.

Every function is pinned by tests in ``tests/test_oracle_*.py`` against closed forms,
invariants, finite differences, a library routine (PyTorch's CPU scaled-dot-product
attention in fp64) and hand-drawn mask fixtures under ``tests/golden/``.
"""
from .masks import mask_block, visible, visible_count, row_visible_counts  # noqa: F401
from .attention import attention_forward, attention_backward  # noqa: F401
from .tiles import tile_classes, tile_csr, tile_csc, keep_csr, keep_csc  # noqa: F401
