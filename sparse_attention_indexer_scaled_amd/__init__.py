"""MI355X (gfx950) lightning-indexer logits.

The op lives in the C-ABI HIP library ``libmqa_indexer.so`` (declared in
``include/mqa_indexer.h``); this package is its thin Python binding plus the
seeded input generator used by the tests and the benchmark.

    from sparse_attention_indexer_scaled_amd import mqa_logits_prefill, paged_mqa_logits_decode

The library is loaded on first use, so importing the package (for example only
for ``inputs``) works on a machine without a GPU.
"""

from ._native import (  # noqa: F401
    EXPORTED,
    LIB_PATH,
    MQAError,
    Tunables,
    is_supported,
    kcache_quantize_insert,
    last_error,
    load_library,
    mqa_logits_prefill,
    paged_mqa_logits_decode,
    paged_mqa_topk_decode,
    paged_mqa_topk_decode_noalloc,
    paged_mqa_topk_workspace_size,
    topk_indices,
    topk_indices_ws,
    topk_workspace_size,
)
