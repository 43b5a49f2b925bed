"""MI355X-native DeepSeek-V4 lightning indexer (forward and backward).

The arithmetic lives in hand-written gfx950 HIP kernels behind the C ABI of
liblix.so (include/lix.h); this package only binds it.
"""

from ._lib import LixError, load, status_string, LIB_PATH, LIX_FUSED_TOPK_MAX  # noqa: F401
from .ops import (  # noqa: F401
    indexer_logits,
    topk,
    fused_topk_supported,
    topk_streaming,
    streaming_workspace_bytes,
    select_topk,
    topk_from_logits,
    topk_scores,
    indexer_scores_at,
    indexer_backward,
    V4IndexerFunction,
    indexer_scores_v41,
    topk_bf16,
    v4_lighting_indexer,
)
