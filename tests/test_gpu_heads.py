"""GPU parity with 64 and 128 index heads (the head counts the pages sweep
besides 32): each query row's heads are processed as 32-head MFMA tiles whose
relu.weight sums add up before the cross-lane reduction.

As for 32 heads: an exact integer pin (bit for bit; inputs in [-8, 8] keep the
128-head sum inside fp32's 24-bit mantissa), random inputs element by element
against the oracle, and bitwise invariance under every launch tunable.  The
decode cases run in every cache block size (1, 16, 64 and 128 tokens).
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

from sparse_attention_indexer_scaled_amd import Tunables, inputs, is_supported
from tests.gpu_util import (assert_parity, lib, oracle_decode, oracle_prefill, run_decode,
                            run_prefill, say)

pytestmark = pytest.mark.gpu
HEADS = [64, 128]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    lib()
    assert is_supported(64, 128, 64) and is_supported(128, 128, 0)


def _int_weights(rng, shape):
    return (rng.choice([-1, 1], shape) * 2.0 ** -rng.integers(0, 4, shape)).astype(np.float32)


@pytest.mark.parametrize("H", HEADS)
def test_prefill_integer_inputs_bit_exact(H):
    rng = np.random.default_rng(700 + H)
    M, N = 13, 333
    p = inputs.make_prefill(M, N, seed=700 + H, H=H)
    p.q = inputs.to_fp8_bytes(rng.integers(-8, 9, (M, H, 128)).astype(np.float32))
    p.k = inputs.to_fp8_bytes(rng.integers(-8, 9, (N, 128)).astype(np.float32))
    p.weights = _int_weights(rng, (M, H))
    p.kv_scale = rng.choice([0.5, 1.0, 2.0], N).astype(np.float32)
    ref, _ = oracle_prefill(p)
    for bm in (1, 2, 4, 8):
        if bm * H > 256:
            continue
        say("prefill int H=%d block_m=%d" % (H, bm))
        assert np.array_equal(run_prefill(p, tun=Tunables(block_m=bm)), ref)


BLOCK_SIZES = [1, 16, 64, 128]


@pytest.mark.parametrize("H", HEADS)
@pytest.mark.parametrize("bs", BLOCK_SIZES)
@pytest.mark.parametrize("next_n", [1, 3, 6])
def test_decode_integer_inputs_bit_exact(H, bs, next_n):
    rng = np.random.default_rng(710 + H + next_n)
    d = inputs.make_decode(3, next_n, [700, 64, 131], 800, seed=710 + next_n, H=H, block_size=bs,
                           poison=True)
    d.q = inputs.to_fp8_bytes(rng.integers(-8, 9, d.q.shape).astype(np.float32))
    d.weights = _int_weights(rng, d.weights.shape)
    kview, sview = inputs.cache_views(d.kv_cache, bs, 128)
    used = d.num_blocks - 1  # the last block is the poison block
    kview[:used] = inputs.to_fp8_bytes(rng.integers(-8, 9, kview[:used].shape).astype(np.float32))
    sview[:used] = rng.choice([0.5, 1.0, 2.0], sview[:used].shape).astype(np.float32)
    say("decode int H=%d bs=%d next_n=%d" % (H, bs, next_n))
    ref, _, _ = oracle_decode(d)
    assert np.array_equal(run_decode(d), ref)


@pytest.mark.parametrize("H", HEADS)
@pytest.mark.parametrize("mode", ["causal", "misaligned", "multi_req"])
def test_prefill_matches_oracle(H, mode):
    p = inputs.make_prefill(70, 700, seed=720 + H, H=H, windows=mode)
    say("prefill H=%d mode=%s" % (H, mode))
    ref, mag = oracle_prefill(p)
    for clean in (True, False):
        out = run_prefill(p, clean=clean)
        if clean:
            assert_parity(out, ref, mag, f"prefill_H{H}_{mode}")
        else:
            win = np.isfinite(ref)
            assert_parity(np.where(win, out, -np.inf), ref, mag, f"prefill_H{H}_{mode}_noclean")


@pytest.mark.parametrize("H", HEADS)
@pytest.mark.parametrize("bs", BLOCK_SIZES)
@pytest.mark.parametrize("B,next_n,ctx,mml", [(3, 2, [700, 130, 3000], 3072),
                                              (2, 6, [2000, 7], 2001),
                                              (4, 1, [0, 15, 65, 4100], 4160),
                                              (2, 8, [129, 1025], 1100)])
def test_decode_matches_oracle(H, bs, B, next_n, ctx, mml):
    d = inputs.make_decode(B, next_n, ctx, mml, seed=730 + H + mml, H=H, block_size=bs,
                           poison=True)
    say("decode H=%d bs=%d B=%d next_n=%d" % (H, bs, B, next_n))
    ref, mag, _ = oracle_decode(d)
    out = run_decode(d)
    assert_parity(out, ref, mag, f"decode_H{H}_bs{bs}_B{B}_nn{next_n}")


@pytest.mark.parametrize("H", HEADS)
@pytest.mark.parametrize("bs", [1, 16, 128])
def test_decode_block_sizes_give_the_same_bits(H, bs):
    """The same draws in a cache of other block sizes give the 64-token
    output bit for bit: only the gather changes."""
    kw = dict(B=3, next_n=3, context_lens=[1500, 1, 700], max_model_len=1536, seed=760 + H, H=H)
    base = run_decode(inputs.make_decode(**kw))
    say("decode H=%d bs=%d vs 64-token blocks" % (H, bs))
    assert np.array_equal(run_decode(inputs.make_decode(block_size=bs, **kw)), base,
                          equal_nan=True)


@pytest.mark.parametrize("H", HEADS)
def test_tunables_do_not_change_bits(H):
    rows = [1, 2] if H == 64 else [1]
    for bs in (64, 16):
        d = inputs.make_decode(3, 6, [2000, 150, 1300], 2048, seed=740 + H, H=H, block_size=bs,
                               poison=True)
        base = run_decode(d)
        for r in rows:
            for split in (1, 5, 64):
                say("decode H=%d bs=%d rows=%d split=%d" % (H, bs, r, split))
                out = run_decode(d, tun=Tunables(rows_per_block=r, split_kv=split))
                assert np.array_equal(out, base, equal_nan=True)
    p = inputs.make_prefill(50, 600, seed=750 + H, H=H)
    pbase = run_prefill(p)
    for bm in (1, 2, 4):
        if bm * H > 256:
            continue
        for nw in (1, 3):
            assert np.array_equal(run_prefill(p, tun=Tunables(block_m=bm, num_warps=nw, split_n=2)),
                                  pbase, equal_nan=True)
