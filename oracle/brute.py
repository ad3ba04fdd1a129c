"""Exact rational brute force for tiny inputs -- TEST INFRASTRUCTURE ONLY.

Evaluates the indexer logits definition (aiter PR 5046 and PR 5047 pages,
"Motivation") in exact rational arithmetic with ``fractions.Fraction``.  fp8
codes, fp32 weights and fp32 scales are all dyadic rationals, so the result is
the exact real value of the definition, which pins the fp64 C oracle to within
its own rounding bound.

Deliberately independent of ``mqa_oracle.c``:

* fp8 codes are decoded with torch's own float8_e4m3fn -> float32 conversion
  (exact), not with the oracle's bit-field decoder;
* the paged gather is done here from raw byte offsets;
* windows are enumerated as explicit Python ranges.

Pure Python loops: use only for a few thousand (row, column) pairs.
"""

from __future__ import annotations

import math
from fractions import Fraction

import numpy as np
import torch


def fp8_values(codes: np.ndarray) -> np.ndarray:
    """float64 values of fp8 e4m3fn codes via torch's conversion."""
    t = torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8)).view(torch.float8_e4m3fn)
    return t.to(torch.float32).numpy().astype(np.float64)


def _fr(x) -> Fraction:
    x = float(x)
    if not math.isfinite(x):
        raise ValueError("non-finite input inside a window")
    return Fraction(x)


def logit_exact(qv, kv, scale, w):
    """Exact sum_h relu(<q_h, k>) * scale * w_h; qv [H,D], kv [D] float values."""
    H, D = qv.shape
    total = Fraction(0)
    s = _fr(scale)
    for h in range(H):
        dot = Fraction(0)
        for d in range(D):
            dot += _fr(qv[h, d]) * _fr(kv[d])
        if dot > 0:
            total += dot * s * _fr(w[h])
    return total


def logit_abs_terms(qv, kv, scale, w):
    """sum_h |relu(<q_h,k>) * scale * w_h| (exact) -- the size the oracle's
    rounding bound is relative to."""
    H, D = qv.shape
    total = Fraction(0)
    s = _fr(scale)
    for h in range(H):
        dot = sum((_fr(qv[h, d]) * _fr(kv[d]) for d in range(D)), Fraction(0))
        if dot > 0:
            total += abs(dot * s * _fr(w[h]))
    return total


def prefill(q, k, kv_scale, weights, ks, ke):
    """Exact prefill logits: dict {(m, n): Fraction} for in-window pairs plus the
    set of in-window pairs.  Window: max(ks,0) <= n < min(ke,N)."""
    qv = fp8_values(q)
    kvals = fp8_values(k)
    M, H, D = qv.shape
    N = kvals.shape[0]
    vals, mags = {}, {}
    for m in range(M):
        lo = max(int(ks[m]), 0)
        hi = min(int(ke[m]), N)
        for n in range(lo, hi):
            vals[(m, n)] = logit_exact(qv[m], kvals[n], kv_scale[n], weights[m])
            mags[(m, n)] = logit_abs_terms(qv[m], kvals[n], kv_scale[n], weights[m])
    return vals, mags


def decode(q, kv_cache, weights, context_lens, block_tables, max_model_len, block_size):
    """Exact paged-decode logits, gathering K and scale from raw cache bytes.

    Block i occupies bytes [i*bs*(D+4), (i+1)*bs*(D+4)): bs K rows of D bytes,
    then bs little-endian fp32 scales.  Row (b, j) covers 0 <= p <= ctx_b -
    next_n + j.
    """
    q = np.asarray(q)
    B, next_n, H, D = q.shape
    flat = np.ascontiguousarray(kv_cache, dtype=np.uint8).reshape(-1)
    blk_bytes = block_size * (D + 4)
    vals, mags = {}, {}
    for b in range(B):
        for j in range(next_n):
            row = b * next_n + j
            bound = int(context_lens[b]) - next_n + j
            qv = fp8_values(q[b, j])
            for p in range(0, min(bound, max_model_len - 1) + 1):
                blk = int(block_tables[b][p // block_size])
                slot = p % block_size
                base = blk * blk_bytes
                kbytes = flat[base + slot * D: base + slot * D + D]
                sbytes = flat[base + block_size * D + 4 * slot: base + block_size * D + 4 * slot + 4]
                scale = np.frombuffer(sbytes.tobytes(), dtype="<f4")[0]
                kv = fp8_values(kbytes)
                vals[(row, p)] = logit_exact(qv, kv, scale, weights[row])
                mags[(row, p)] = logit_abs_terms(qv, kv, scale, weights[row])
    return vals, mags
