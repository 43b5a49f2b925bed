"""Plain CPU oracle for the lightning-indexer forward pass.

TEST INFRASTRUCTURE ONLY.  The tests, the smoke check and the benchmark's
CPU-baseline leg are the only code allowed to import it.  The product path
(the HIP library and its Python binding) never calls into this package, and
this package never imports the product path: the two share no code.

Everything is NumPy float64, with bfloat16 rounding emulated from its
definition where the V4.1 page fixes rounding points.  ``indexer_grad``
holds the backward pass (gradients of the selected scores).
"""

from .indexer import (  # noqa: F401
    NEG_INF,
    bf16_bits_to_f64,
    f64_to_bf16_bits,
    rne_bf16,
    ulp_bf16,
    causal_ranges,
    indexer_logits_rows,
    indexer_logits,
    topk_select,
    topk_select_visible_bf16,
    topk_scores_gather,
    indexer_scores_v41_rows,
    indexer_scores_v41,
    indexer_scores_v41_bounds_rows,
)
from .indexer_grad import indexer_backward  # noqa: F401
