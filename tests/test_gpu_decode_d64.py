"""GPU parity of the paged decode at head dim 64 (64-byte K rows, one fp8
MFMA per row, tile and head tile): 32, 64 and 128 heads, blocks of 1, 16, 64
and 128 tokens, slot-major and (blocks of 16 or more) preshuffled K.

An exact integer pin (bit for bit against the oracle), random inputs element by
element against the oracle, and bitwise invariance under launch tunables,
block size and K order.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

from sparse_attention_indexer_scaled_amd import Tunables, inputs, is_supported
from tests.gpu_util import assert_parity, lib, oracle_decode, run_decode, say

pytestmark = pytest.mark.gpu
D = 64


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    lib()
    assert is_supported(32, D, 64) and is_supported(128, D, 16) and is_supported(32, D, 1)


def _integer(d, rng):
    """Integer fp8 values in [-8, 8], power-of-two weights and scales: every
    logit is exact in fp32 whatever the accumulation order."""
    d.q = inputs.to_fp8_bytes(rng.integers(-8, 9, d.q.shape).astype(np.float32))
    d.weights = (rng.choice([-1, 1], d.weights.shape) *
                 2.0 ** -rng.integers(0, 4, d.weights.shape)).astype(np.float32)
    kview, sview = inputs.cache_views(d.kv_cache, d.block_size, D)
    used = d.num_blocks - 1  # the last block is the poison block
    kview[:used] = inputs.to_fp8_bytes(rng.integers(-8, 9, kview[:used].shape).astype(np.float32))
    sview[:used] = rng.choice([0.5, 1.0, 2.0], sview[:used].shape).astype(np.float32)
    return d


@pytest.mark.parametrize("H", [32, 64, 128])
@pytest.mark.parametrize("bs,pre", [(1, False), (16, False), (64, False), (128, False), (16, True),
                                    (64, True), (128, True)])
def test_integer_inputs_bit_exact(H, bs, pre):
    rng = np.random.default_rng(800 + H + bs)
    d = inputs.make_decode(3, 3, [700, 64, 131], 800, seed=800 + bs, H=H, D=D, block_size=bs,
                           poison=True)
    d = _integer(d, rng)
    if pre:
        d.kv_cache = inputs.preshuffle_blocks(d.kv_cache, bs, D)
        d.preshuffle = True
    say("decode d64 int H=%d bs=%d preshuffle=%s" % (H, bs, pre))
    ref, _, _ = oracle_decode(d)
    assert np.array_equal(run_decode(d), ref)


@pytest.mark.parametrize("next_n", [1, 2, 4, 5, 6, 8])
def test_integer_inputs_bit_exact_every_row_split(next_n):
    rng = np.random.default_rng(820 + next_n)
    d = inputs.make_decode(2, next_n, [1500, next_n - 1], 1536, seed=820 + next_n, D=D,
                           poison=True)
    d = _integer(d, rng)
    ref, _, _ = oracle_decode(d)
    for r in sorted({1, 2, 3, 4} & set(range(1, next_n + 1))):
        say("decode d64 int next_n=%d rows=%d" % (next_n, r))
        assert np.array_equal(run_decode(d, tun=Tunables(rows_per_block=r)), ref)


@pytest.mark.parametrize("H", [32, 64, 128])
@pytest.mark.parametrize("bs", [1, 16, 64, 128])
@pytest.mark.parametrize("B,next_n,ctx,mml", [(3, 2, [700, 130, 3000], 3072),
                                              (4, 1, [0, 15, 65, 4100], 4160),
                                              (2, 6, [2000, 7], 2001)])
def test_matches_oracle(H, bs, B, next_n, ctx, mml):
    d = inputs.make_decode(B, next_n, ctx, mml, seed=840 + H + bs + mml, H=H, D=D, block_size=bs,
                           poison=True)
    say("decode d64 H=%d bs=%d B=%d next_n=%d" % (H, bs, B, next_n))
    ref, mag, _ = oracle_decode(d)
    assert_parity(run_decode(d), ref, mag, f"decode_d64_H{H}_bs{bs}_B{B}_nn{next_n}")
    if next_n == 2:
        win = np.isfinite(ref)
        out = run_decode(d, clean=False)
        assert_parity(np.where(win, out, -np.inf), ref, mag, f"decode_d64_H{H}_bs{bs}_noclean")
        assert np.isnan(out[~win]).all(), "clean_logits=0 wrote outside the window"


@pytest.mark.parametrize("H", [32, 128])
def test_tunables_block_sizes_and_k_order_do_not_change_bits(H):
    kw = dict(B=3, next_n=6, context_lens=[2000, 150, 1300], max_model_len=2048, seed=860 + H,
              H=H, D=D)
    base = run_decode(inputs.make_decode(block_size=64, **kw))
    for bs in (1, 16, 64, 128):
        for pre in ((False,) if bs == 1 else (False, True)):
            d = inputs.make_decode(block_size=bs, preshuffle=pre, **kw)
            say("decode d64 H=%d bs=%d preshuffle=%s vs 64-token slot-major" % (H, bs, pre))
            assert np.array_equal(run_decode(d), base, equal_nan=True)
            for rows in ([1, 2] if H == 32 else [1]):
                for split in (1, 7, 64):
                    out = run_decode(d, tun=Tunables(rows_per_block=rows, split_kv=split))
                    assert np.array_equal(out, base, equal_nan=True)
