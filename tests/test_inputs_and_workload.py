"""Host-side pieces: the input generator's cache packing, and the byte model the
benchmark uses (pinned to figures printed on the pages)."""

from __future__ import annotations

import numpy as np

from sparse_attention_indexer_scaled_amd import inputs, workload
from tests.util import read_kv


def test_byte_model_matches_pages_figures():
    g = read_kv("byte_model.txt")
    B, nn, ctx = int(g["B"][0]), int(g["next_n"][0]), int(g["ctx"][0])
    shared = workload.decode_kv_and_out_bytes(B, nn, [ctx] * B, ctx)
    assert round(shared / 1e6) == int(g["shared_k_mb"][0])
    per_row = shared + (nn - 1) * B * ctx * (128 + 4)
    assert round(per_row / 1e6) == int(g["per_row_k_mb"][0])


def test_valid_pairs_counts():
    # decode: B16 nn6 ctx 131072: rows see ctx-5 .. ctx columns
    assert workload.decode_valid_pairs(6, [131072] * 16, 131072) == 16 * sum(131072 - 5 + j for j in range(6))
    ks, ke = inputs.causal_windows(4096, 32768)
    assert workload.prefill_valid_pairs(ks, ke, 32768) == sum(28673 + m for m in range(4096))


def test_cache_pack_roundtrip():
    d = inputs.make_decode(3, 2, [1, 64, 130], 200, seed=9, poison=True)
    kview, sview = inputs.cache_views(d.kv_cache, 64, 128)
    for b in range(3):
        ctx = int(d.context_lens[b])
        for p in range(ctx):
            blk = d.block_tables[b, p // 64]
            assert np.array_equal(kview[blk, p % 64], d.k_seq[b][p])
            assert sview[blk, p % 64] == d.s_seq[b][p]
    # the pool is exactly the used blocks plus one poison block, each used once
    used = [int(x) for b in range(3) for x in d.block_tables[b, : (int(d.context_lens[b]) + 63) // 64]]
    assert sorted(used) == list(range(d.num_blocks - 1))
    # block stride keeps every K row 16-byte aligned
    assert (64 * (128 + 4)) % 16 == 0


def test_quantize_tokens_hits_fp8_max():
    x = np.random.default_rng(0).standard_normal((50, 128)).astype(np.float32)
    codes, scale = inputs.quantize_tokens(x)
    assert ((codes & 0x7F) == 0x7E).any(axis=1).all()  # each token reaches +-448
    assert not ((codes & 0x7F) == 0x7F).any()          # never NaN
    assert np.allclose(scale, np.abs(x).max(axis=1) / 448, rtol=1e-6)


def test_generator_is_seeded():
    a = inputs.make_decode(2, 2, None, 4096, seed=5, ctx_range=(100, 4000))
    b = inputs.make_decode(2, 2, None, 4096, seed=5, ctx_range=(100, 4000))
    assert np.array_equal(a.kv_cache, b.kv_cache) and np.array_equal(a.block_tables, b.block_tables)
    assert np.array_equal(a.q, b.q) and np.array_equal(a.weights, b.weights)


def test_decode_bytes_at_head_dim_64_by_hand():
    """Workload 21 (the headline shape at head dim 64), term by term: 68-byte
    tokens, every output element once, Q, weights, used table entries and
    context lengths."""
    B, nn, ctx, H, D = 16, 6, 131072, 32, 64
    want = (B * ctx * (64 + 4)          # K + scale per cached token
            + B * nn * ctx * 4          # fp32 logits, -inf fill included
            + B * nn * H * D            # fp8 Q
            + B * nn * H * 4            # fp32 weights
            + B * (ctx // 64) * 4       # used table entries
            + B * 4)                    # context lengths
    assert workload.decode_essential_bytes(B, nn, [ctx] * B, ctx, H=H, D=D) == want
    d = inputs.make_config(21)
    assert d.D == 64 and d.kv_cache.shape[1] == 64 * 68


def test_cache_pack_roundtrip_head_dim_64_per_token_blocks():
    """68-byte per-token records: token p's 64 K bytes, then its scale."""
    d = inputs.make_decode(2, 1, [5, 9], 16, seed=11, D=64, block_size=1)
    kview, sview = inputs.cache_views(d.kv_cache, 1, 64)
    assert d.kv_cache.shape[1] == 68
    for b in range(2):
        for p in range(int(d.context_lens[b])):
            blk = d.block_tables[b, p]
            assert np.array_equal(kview[blk, 0], d.k_seq[b][p]) and sview[blk, 0] == d.s_seq[b][p]
