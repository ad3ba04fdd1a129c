"""Essential work of one call: the bytes and flops a perfect kernel must spend.

The benchmark divides these by measured time to get achieved HBM TB/s and fp8
TFLOP/s.  They are counts, not the op's arithmetic.

Decode bytes follow the accounting the issue page on next_n tiling uses for its
B16 / next_n 6 / 131072-context workload ("This is not a bandwidth problem":
327 MB when every K token is read once, 1711 MB when each of the six rows
re-reads it): each cached token's 128 B of K plus its 4 B scale once, plus each
fp32 output element once.  We add the small terms (Q, weights, used table
entries, context lengths), which that figure leaves out.
"""

from __future__ import annotations

import numpy as np

HEADS = 32
HEAD_DIM = 128
KV_BLOCK = 64


def decode_kv_and_out_bytes(B, next_n, context_lens, max_model_len, D=HEAD_DIM):
    """The two dominant terms: K + scale per cached token, fp32 output per element."""
    ctx = np.asarray(context_lens, dtype=np.int64)
    return int(ctx.sum()) * (D + 4) + B * next_n * int(max_model_len) * 4


def decode_essential_bytes(B, next_n, context_lens, max_model_len, H=HEADS, D=HEAD_DIM,
                           block_size=KV_BLOCK):
    ctx = np.asarray(context_lens, dtype=np.int64)
    q = B * next_n * H * D
    w = B * next_n * H * 4
    tables = int(((ctx + block_size - 1) // block_size).sum()) * 4
    return decode_kv_and_out_bytes(B, next_n, ctx, max_model_len, D) + q + w + tables + B * 4


def decode_valid_pairs(next_n, context_lens, max_model_len):
    """(row, position) pairs inside a decode window: row j of sequence b covers
    p <= ctx_b - next_n + j."""
    ctx = np.asarray(context_lens, dtype=np.int64)
    tot = 0
    for j in range(next_n):
        tot += int(np.clip(np.minimum(ctx - next_n + j + 1, max_model_len), 0, None).sum())
    return tot


def prefill_valid_pairs(ks, ke, N):
    lo = np.maximum(np.asarray(ks, np.int64), 0)
    hi = np.minimum(np.asarray(ke, np.int64), N)
    return int(np.clip(hi - lo, 0, None).sum())


def prefill_essential_bytes(M, N, H=HEADS, D=HEAD_DIM):
    """Q, K, scales, weights, the two window arrays and the full fp32 output."""
    return M * H * D + N * D + N * 4 + M * H * 4 + 2 * M * 4 + M * N * 4


def flops_per_pair(H=HEADS, D=HEAD_DIM):
    """2 * H * D: the multiply-adds of the 32-head Q.K contraction per (row, column)."""
    return 2 * H * D
