"""Pins of the K-cache quantise-and-insert oracle (oracle.kcache) against
things other than itself: a hand-worked example, torch's own fp32 -> e4m3fn
conversion (a library routine) over every rounding boundary, the seeded
generator's independent quantiser, and the decode oracle's own gather."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from oracle import kcache
from sparse_attention_indexer_scaled_amd import inputs
from tests.util import golden_path, read_kv


def _golden():
    g = read_kv("kcache_example.txt")
    k = np.array([[np.float32(t) for t in g["k0"]], [np.float32(t) for t in g["k1"]]],
                 dtype=np.float32)
    codes = np.array([[int(t, 16) for t in g["codes0"]], [int(t, 16) for t in g["codes1"]]],
                     dtype=np.uint8)
    scale = np.array([float(g["scale0"][0]), float(g["scale1"][0])], dtype=np.float32)
    return g, k, codes, scale


def test_hand_example_quantize():
    _, k, codes, scale = _golden()
    got_codes, got_scale = kcache.quantize_tokens(k)
    assert np.array_equal(got_codes, codes)
    assert np.array_equal(got_scale, scale)


def test_hand_example_insert():
    g, k, codes, _ = _golden()
    cache = np.arange(3 * 16, dtype=np.uint8).reshape(3, 16)
    slots = np.array([int(t) for t in g["slots"]], dtype=np.int64)
    out = kcache.insert(cache, k, slots, block_size=2)
    want = cache.copy()
    want[2, 4:8] = codes[0]
    want[2, 12:16] = [0x00, 0x00, 0x80, 0x3f]
    assert np.array_equal(out, want)


def test_hand_example_out_of_range_slot_is_skipped():
    g, k, codes, _ = _golden()
    cache = np.arange(3 * 16, dtype=np.uint8).reshape(3, 16)
    slots = np.array([int(t) for t in g["slots_oob"]], dtype=np.int64)
    out = kcache.insert(cache, k, slots, block_size=2)
    want = cache.copy()
    want[2, 0:4] = codes[1]
    want[2, 8:12] = [0x00, 0x00, 0x00, 0x3f]
    assert np.array_equal(out, want)


def test_slots_past_the_cache_write_nothing():
    rng = np.random.default_rng(15)
    cache = rng.integers(0, 256, (2, 16 * 132), dtype=np.uint8)
    k = rng.standard_normal((3, 128)).astype(np.float32)
    out = kcache.insert(cache, k, np.array([32, 33, 1 << 40], np.int64), 16)
    assert np.array_equal(out, cache)


def test_negative_extreme_sets_the_scale():
    """Worked by hand: the largest magnitude is -448, so amax = 448, the scale is
    448 / 448 = 1 and the codes are the format's own: -448 = -1.75 * 2^8 is sign 1,
    exponent field 15, mantissa 6 (0xFE); 1 = 2^0 is exponent field 7 (0x38); 0 is 0x00."""
    k = np.zeros((1, 128), np.float32)
    k[0, 0], k[0, 1] = -448.0, 1.0
    codes, scale = kcache.quantize_tokens(k)
    assert scale.tolist() == [1.0]
    assert codes[0, :3].tolist() == [0xFE, 0x38, 0x00] and not codes[0, 3:].any()


def test_all_zero_token():
    """A zero row takes the floor of the amax: codes 0 and the scale of amax 1e-12."""
    codes, scale = kcache.quantize_tokens(np.zeros((1, 64), np.float32))
    assert not codes.any()
    assert scale[0] == np.float32(np.float32(1e-12) / np.float32(448.0))


def _boundaries():
    """Every midpoint between adjacent e4m3fn values, one fp32 ulp either
    side, and the values themselves, both signs."""
    table = oracle.e4m3fn_table()[:0x7F].astype(np.float32)
    mids = ((table[:-1].astype(np.float64) + table[1:]) / 2).astype(np.float32)
    pts = np.concatenate([table, mids, np.nextafter(mids, np.float32(0)),
                          np.nextafter(mids, np.float32(1e9))])
    pts = pts[np.abs(pts) <= 448]
    return np.concatenate([pts, -pts]).astype(np.float32)


def test_rounding_matches_torch_at_every_boundary():
    x = _boundaries()
    want = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(kcache.e4m3fn_rne(x), want)


def test_rounding_matches_torch_on_random_values():
    rng = np.random.default_rng(11)
    x = np.concatenate([rng.uniform(-448, 448, 100000), rng.uniform(-0.03, 0.03, 100000)])
    x = x.astype(np.float32)
    want = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(kcache.e4m3fn_rne(x), want)


def test_matches_the_generators_quantiser():
    rng = np.random.default_rng(12)
    k = (rng.standard_normal((300, 128)) * rng.uniform(0.01, 100, (300, 1))).astype(np.float32)
    k[0] = 0.0
    codes, scale = kcache.quantize_tokens(k)
    gcodes, gscale = inputs.quantize_tokens(k)
    assert np.array_equal(scale, gscale)
    assert np.array_equal(codes, gcodes)


@pytest.mark.parametrize("D", [128, 64])
def test_inserted_cache_feeds_the_decode_oracle(D):
    """Tokens quantised into a shuffled set of slots read back, through the
    decode oracle's own gather, as the prefill oracle on the same codes."""
    rng = np.random.default_rng(13)
    bs, H = 64, 32
    T = 150
    nblocks = 4
    k = rng.standard_normal((T, D)).astype(np.float32)
    blocks = rng.permutation(nblocks)[:3]
    slots = np.concatenate([blocks[p // bs:p // bs + 1] * bs + p % bs for p in range(T)])
    cache = np.zeros((nblocks, bs * (D + 4)), dtype=np.uint8)
    cache = kcache.insert(cache, k, slots, bs)
    codes, scale = kcache.quantize_tokens(k)
    q = inputs.to_fp8_bytes(rng.standard_normal((1, 1, H, D)).astype(np.float32))
    w = rng.standard_normal((1, H)).astype(np.float32)
    table = np.zeros((1, 4), dtype=np.int32)
    table[0, :3] = blocks
    got = oracle.decode(q, cache, w, np.array([T], np.int32), table, T, bs)
    want = oracle.prefill(q[0], codes, scale, w, np.array([0], np.int32), np.array([T], np.int32))
    assert np.array_equal(got, want)


def test_padding_slots_write_nothing():
    rng = np.random.default_rng(14)
    cache = rng.integers(0, 256, (2, 64 * 132), dtype=np.uint8)
    k = rng.standard_normal((3, 128)).astype(np.float32)
    out = kcache.insert(cache, k, np.array([-1, -1, -5], np.int64), 64)
    assert np.array_equal(out, cache)


def test_preshuffled_insert_positions_worked_by_hand():
    """A token that is 448 at one position and 0 elsewhere quantises to scale 1
    and the code 0x7E there (the largest e4m3fn value); inserted into a
    preshuffled cache, that code lands at the hand-worked offset of
    tests/golden/preshuffle_layout.txt and nowhere else."""
    with open(golden_path("preshuffle_layout.txt")) as f:
        rows = [tuple(int(x) for x in l.split("#", 1)[0].split()) for l in f
                if l.split("#", 1)[0].strip()]
    for bs, D, offset, slot, byte in rows:
        k = np.zeros((1, D), np.float32)
        k[0, byte] = 448.0
        cache = np.zeros((2, bs * (D + 4)), np.uint8)
        out = kcache.insert(cache, k, np.array([bs + slot], np.int64), bs, preshuffle=True)
        assert not out[0].any()
        kpart = out[1, : bs * D]
        assert np.flatnonzero(kpart).tolist() == [offset] and kpart[offset] == 0x7E
        assert out[1, bs * D + 4 * slot: bs * D + 4 * slot + 4].view(np.float32)[0] == 1.0


@pytest.mark.parametrize("D", [128, 64])
@pytest.mark.parametrize("bs", [16, 64, 128])
def test_preshuffled_insert_is_the_permuted_plain_insert(bs, D):
    """The generator's block permutation (numpy reshape/transpose) applied to
    the slot-major insert gives the preshuffled insert, byte for byte."""
    d = inputs.make_kcache_insert(40, 4, seed=5, block_size=bs, D=D)
    plain = kcache.insert(d.kv_cache, d.k, d.slot_mapping, bs)
    tiled_prior = inputs.preshuffle_blocks(d.kv_cache, bs, D)
    tiled = kcache.insert(tiled_prior, d.k, d.slot_mapping, bs, preshuffle=True)
    assert np.array_equal(tiled, inputs.preshuffle_blocks(plain, bs, D))
