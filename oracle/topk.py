"""CPU oracle for the row-wise top-k over indexer logits -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, the package smoke check and the benchmark's ``cpu_baseline``
leg may import this module; the product path never does.

The pages name the consumer of the indexer logits -- a top-k with index_topk
2048 or 512 (aiter PR 5047 page, "Integration" and the serving notes; the issue
page about next_n tiling, "Setup") -- but do not define its order.  The reading
implemented here (and by the HIP kernel) is one total order:

  - an entry is listable unless it is -inf or NaN (positions outside a row's
    window are -inf once the fused fill has run);
  - listable entries rank by value, larger first; equal values (with -0.0
    equal to +0.0) rank by column, smaller first;
  - row r's output is the first min(k, #listable) columns of that order,
    then -1.

This is the definition written out with one library sort per row
(``numpy.lexsort``, stable on the secondary key); the values are the fp32
logits themselves, so both sides take every comparison in fp32.
"""

from __future__ import annotations

import numpy as np


def topk_indices(logits: np.ndarray, k: int) -> np.ndarray:
    """logits [rows, cols] float32 -> int32 [rows, k]."""
    x = np.asarray(logits)
    if x.dtype != np.float32 or x.ndim != 2:
        raise ValueError("logits must be a 2-D float32 array")
    if k < 1:
        raise ValueError("k must be >= 1")
    rows = x.shape[0]
    out = np.full((rows, k), -1, dtype=np.int32)
    for r in range(rows):
        v = x[r]
        cols = np.nonzero(~(np.isnan(v) | (v == -np.inf)))[0]
        # primary key: value, descending (negated; -0.0 and +0.0 compare equal);
        # secondary key: column, ascending
        order = cols[np.lexsort((cols, -v[cols]))][:k]
        out[r, :order.size] = order
    return out
