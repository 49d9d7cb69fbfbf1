"""CPU oracle for FlashSwin window attention (test infrastructure only).

This package is the checker, not the product.  Only the test suite, the smoke
check and the benchmark's CPU-baseline leg may import it; the GPU library and
its Python binding never do, and they share no code with it.

Sources cited throughout ([FS] below) is the paper card titled
"FLASHSWIN: Unlocking Large Windows and Dense Tokens in Swin Vision
Transformers with Memory Efficient Attention" (its Abstract, Figure 1,
Table S2 and Figure S4).

Two independent routes are provided:

* ``wattn_ref``   -- O1: the plain materialized definition in float64
  (roll, window partition, explicit RoPE rotation, full N x N score matrix,
  region mask, softmax, P.V) plus its analytic backward.
* ``wattn_online`` -- O2: an online-softmax variant that never rolls or
  partitions; every query finds its window and region by index arithmetic,
  RoPE is applied as a complex phase, keys are streamed in tiles with a
  running max and sum.  Its backward recomputes P from the saved LSE.

Parity status: the softmax-attention core, the shift/mask index math and the
backward are pinned by the CPU tests (brute force, closed forms, library
attention, finite differences, invariants).  The RoPE conventions (axis split,
pair layout, rotation sign) are fixed readings that the pages do not print;
they are pinned for internal consistency only ("parity unpinned" against the
pages for those conventions).
"""

from .wattn_ref import (  # noqa: F401
    check_args,
    check_bias,
    check_lowrank,
    lowrank_bias,
    region_labels,
    relative_bias,
    rope_rotate,
    wattn_fwd_ref,
    wattn_bwd_ref,
    window_scores_ref,
)
from .wattn_online import wattn_fwd_online, wattn_bwd_online  # noqa: F401
