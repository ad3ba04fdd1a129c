"""GPU parity of the K-cache quantise-and-insert step with the oracle.

Integer/byte work: the whole cache after the call (codes, scales and every
untouched byte) must equal the oracle's bit for bit.  The scale is one
correctly rounded fp32 division on both sides, the codes an exact
round-to-nearest-even, so there is no tolerance.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

from oracle import kcache as oracle_kcache
from sparse_attention_indexer_scaled_amd import _native, inputs
from tests.gpu_util import dev, lib, run_decode, say, oracle_decode, assert_parity

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    lib()


def gpu_insert(c, preshuffle=False):
    cache = dev(c.kv_cache)
    k = dev(c.k)
    if c.bf16:
        k = k.to(torch.bfloat16)
    _native.kcache_quantize_insert(k, dev(c.slot_mapping), cache, kv_block_size=c.block_size,
                                   preshuffle=preshuffle)
    torch.cuda.synchronize()
    return cache.cpu().numpy()


@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("T,num_blocks", [(1, 1), (5, 2), (64, 1), (1000, 20), (4096, 70)])
def test_insert_matches_oracle(T, num_blocks, bf16):
    c = inputs.make_kcache_insert(T, num_blocks, seed=600 + T + bf16, bf16=bf16)
    say("kcache insert T=%d blocks=%d bf16=%d" % (T, num_blocks, bf16))
    got = gpu_insert(c)
    want = oracle_kcache.insert(c.kv_cache, c.k, c.slot_mapping, c.block_size)
    if not np.array_equal(got, want):
        diff = np.argwhere(got != want)
        raise AssertionError("%d bytes differ, first at %s" % (len(diff), diff[0].tolist()))


@pytest.mark.parametrize("bs", [1, 16, 128])
def test_insert_other_block_sizes(bs):
    c = inputs.make_kcache_insert(700, -(-700 // bs) + 3, seed=620 + bs, block_size=bs)
    say("kcache insert bs=%d" % bs)
    got = gpu_insert(c)
    want = oracle_kcache.insert(c.kv_cache, c.k, c.slot_mapping, bs)
    assert np.array_equal(got, want)


@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("bs", [16, 64, 128])
def test_insert_preshuffled_layout(bs, bf16):
    c = inputs.make_kcache_insert(900, -(-900 // bs) + 2, seed=640 + bs + bf16, block_size=bs,
                                  bf16=bf16)
    say("kcache insert preshuffled bs=%d bf16=%d" % (bs, bf16))
    got = gpu_insert(c, preshuffle=True)
    want = oracle_kcache.insert(c.kv_cache, c.k, c.slot_mapping, bs, preshuffle=True)
    if not np.array_equal(got, want):
        diff = np.argwhere(got != want)
        raise AssertionError("%d bytes differ, first at %s" % (len(diff), diff[0].tolist()))


@pytest.mark.parametrize("bs", [1, 16, 64])
def test_insert_skips_slots_past_the_cache(bs):
    """Slots at or past num_blocks * block_size are dropped like padding (the
    oracle's reading of the out-of-range rule); the whole cache is compared."""
    c = inputs.make_kcache_insert(300, -(-300 // bs) + 2, seed=660 + bs, block_size=bs)
    nslots = c.kv_cache.shape[0] * bs
    slots = c.slot_mapping.copy()
    slots[0:6] = [nslots, nslots + 1, nslots + bs, 2 * nslots, 1 << 40, (1 << 62) + 5]
    c = inputs.KcacheInsertInputs(c.k, slots, c.kv_cache, bs, c.bf16)
    say("kcache insert out-of-range slots bs=%d" % bs)
    got = gpu_insert(c)
    want = oracle_kcache.insert(c.kv_cache, c.k, c.slot_mapping, bs)
    if not np.array_equal(got, want):
        diff = np.argwhere(got != want)
        raise AssertionError("%d bytes differ, first at %s" % (len(diff), diff[0].tolist()))


def test_rounding_boundaries_on_gpu():
    """Rows whose quotients land on every e4m3fn rounding boundary: the row
    maximum is 448 so the scale is 1 and k / scale = k exactly."""
    import oracle
    table = oracle.e4m3fn_table()[:0x7F].astype(np.float32)
    mids = ((table[:-1].astype(np.float64) + table[1:]) / 2).astype(np.float32)
    vals = np.concatenate([table, mids, np.nextafter(mids, np.float32(0)),
                           np.nextafter(mids, np.float32(1e9))])
    vals = np.concatenate([vals, -vals])
    rows = -(-vals.size // 127)
    k = np.zeros((rows, 128), dtype=np.float32)
    k[:, 0] = 448.0
    flat = np.zeros(rows * 127, dtype=np.float32)
    flat[:vals.size] = vals
    k[:, 1:] = flat.reshape(rows, 127)
    c = inputs.KcacheInsertInputs(k, np.arange(rows, dtype=np.int64),
                                  np.zeros((-(-rows // 64), 64 * 132), dtype=np.uint8), 64, False)
    got = gpu_insert(c)
    want = oracle_kcache.insert(c.kv_cache, c.k, c.slot_mapping, 64)
    assert np.array_equal(got, want)


def test_insert_then_decode_end_to_end():
    """GPU insert then GPU decode, against oracle insert then oracle decode:
    each side consumes only its own outputs."""
    import dataclasses
    d = inputs.make_decode(2, 3, [700, 1500], 1600, seed=610)
    rng = np.random.default_rng(611)
    slots = np.concatenate([d.block_tables[b, np.arange(int(d.context_lens[b])) // 64] * 64
                            + np.arange(int(d.context_lens[b])) % 64 for b in range(d.B)])
    k = (rng.standard_normal((slots.size, 128)) * 3).astype(np.float32)
    empty = np.zeros_like(d.kv_cache)
    say("kcache insert feeding decode")
    c = inputs.KcacheInsertInputs(k, slots.astype(np.int64), empty, 64, False)
    gpu_cache = gpu_insert(c)
    oracle_cache = oracle_kcache.insert(empty, k, slots, 64)
    assert np.array_equal(gpu_cache, oracle_cache)
    out = run_decode(dataclasses.replace(d, kv_cache=gpu_cache))
    ref, mag, _ = oracle_decode(dataclasses.replace(d, kv_cache=oracle_cache))
    assert_parity(out, ref, mag, "decode after insert")


def test_preshuffled_insert_then_decode_end_to_end():
    """The same chain in the preshuffled (16,16) layout, 16-token blocks."""
    import dataclasses
    d = inputs.make_decode(2, 2, [333, 1000], 1024, seed=612, block_size=16, preshuffle=True)
    rng = np.random.default_rng(613)
    slots = np.concatenate([d.block_tables[b, np.arange(int(d.context_lens[b])) // 16] * 16
                            + np.arange(int(d.context_lens[b])) % 16 for b in range(d.B)])
    k = (rng.standard_normal((slots.size, 128)) * 2).astype(np.float32)
    empty = np.zeros_like(d.kv_cache)
    say("kcache insert (preshuffled) feeding decode")
    c = inputs.KcacheInsertInputs(k, slots.astype(np.int64), empty, 16, False)
    gpu_cache = gpu_insert(c, preshuffle=True)
    oracle_cache = oracle_kcache.insert(empty, k, slots, 16, preshuffle=True)
    assert np.array_equal(gpu_cache, oracle_cache)
    out = run_decode(dataclasses.replace(d, kv_cache=gpu_cache))
    ref, mag, _ = oracle_decode(dataclasses.replace(d, kv_cache=oracle_cache))
    assert_parity(out, ref, mag, "preshuffled decode after insert")


def test_zero_tokens_is_a_no_op():
    cache = torch.zeros((1, 64 * 132), dtype=torch.uint8, device="cuda")
    _native.kcache_quantize_insert(torch.empty((0, 128), device="cuda"),
                                   torch.empty((0,), dtype=torch.int64, device="cuda"), cache)
    torch.cuda.synchronize()
    assert int(cache.sum()) == 0


@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("bs,pre", [(1, False), (16, False), (64, False), (128, False),
                                    (16, True), (64, True), (128, True)])
def test_insert_head_dim_64(bs, pre, bf16):
    """Head dim 64: 64 code bytes per token (one per lane), the scale after the
    block's 64-byte rows; the whole cache equals the oracle's bit for bit."""
    c = inputs.make_kcache_insert(900, -(-900 // bs) + 2, seed=660 + bs + bf16, block_size=bs, D=64,
                                  bf16=bf16)
    say("kcache insert d64 bs=%d preshuffle=%s bf16=%d" % (bs, pre, bf16))
    got = gpu_insert(c, preshuffle=pre)
    want = oracle_kcache.insert(c.kv_cache, c.k, c.slot_mapping, bs, preshuffle=pre)
    if not np.array_equal(got, want):
        diff = np.argwhere(got != want)
        raise AssertionError("%d bytes differ, first at %s" % (len(diff), diff[0].tolist()))


def test_insert_then_decode_end_to_end_head_dim_64():
    """The insert-then-decode chain at head dim 64 (64-token blocks, 64 heads)."""
    import dataclasses
    d = inputs.make_decode(2, 3, [700, 1500], 1600, seed=614, H=64, D=64)
    rng = np.random.default_rng(615)
    slots = np.concatenate([d.block_tables[b, np.arange(int(d.context_lens[b])) // 64] * 64
                            + np.arange(int(d.context_lens[b])) % 64 for b in range(d.B)])
    k = (rng.standard_normal((slots.size, 64)) * 3).astype(np.float32)
    empty = np.zeros_like(d.kv_cache)
    say("kcache insert d64 feeding decode")
    c = inputs.KcacheInsertInputs(k, slots.astype(np.int64), empty, 64, False)
    gpu_cache = gpu_insert(c)
    oracle_cache = oracle_kcache.insert(empty, k, slots, 64)
    assert np.array_equal(gpu_cache, oracle_cache)
    out = run_decode(dataclasses.replace(d, kv_cache=gpu_cache))
    ref, mag, _ = oracle_decode(dataclasses.replace(d, kv_cache=oracle_cache))
    assert_parity(out, ref, mag, "decode d64 after insert")
