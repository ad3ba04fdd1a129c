"""Pins of the CPU oracle against things other than itself (runs without a GPU).

Each test names what fixes the expected value: the pages' definitions and
printed figures (golden files), exact rational brute force, numpy closed forms,
torch's fp8 conversion, and invariants of the mathematics.  Together they are
chosen so that a plausible slip in the oracle -- a dropped relu, a sign, a
transposed operand, a wrong head/weight pairing, an off-by-one window, a wrong
gather offset -- fails at least one of them.
"""

from __future__ import annotations

import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from oracle import brute
from sparse_attention_indexer_scaled_amd import inputs
from tests.util import floats, read_kv, golden_path

# ---------------------------------------------------------------------------
# fp8 e4m3fn decode
# ---------------------------------------------------------------------------


def test_fp8_table_matches_torch_conversion():
    """Library routine: torch's float8_e4m3fn -> float32 conversion is exact."""
    ours = oracle.e4m3fn_table()
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float32).double().numpy()
    nan_ours = np.isnan(ours)
    assert np.array_equal(nan_ours, np.isnan(ref))
    assert np.array_equal(ours[~nan_ours], ref[~nan_ours])
    # sign of zero too
    assert np.array_equal(np.signbit(ours[~nan_ours]), np.signbit(ref[~nan_ours]))


def test_fp8_closed_forms():
    """Values fixed by the format itself (bias 7, 3 mantissa bits, no inf)."""
    t = oracle.e4m3fn_table()
    assert t[0x38] == 1.0          # 0 0111 000
    assert t[0x7E] == 448.0        # largest finite
    assert t[0xFE] == -448.0
    assert t[0x01] == 2.0 ** -9    # smallest subnormal
    assert t[0x07] == 7 * 2.0 ** -9
    assert t[0x08] == 2.0 ** -6    # smallest normal
    assert t[0x40] == 2.0
    assert t[0x3C] == 1.5
    assert np.isnan(t[0x7F]) and np.isnan(t[0xFF])
    assert int(np.isnan(t).sum()) == 2
    assert t[0x80] == 0.0 and math.copysign(1.0, t[0x80]) == -1.0
    # every finite code is an integer multiple of 2^-9 with magnitude <= 448
    fin = t[np.isfinite(t)]
    assert np.all(np.abs(fin) <= 448.0)
    assert np.all((fin * 512.0) == np.round(fin * 512.0))


# ---------------------------------------------------------------------------
# the pages' windows, enumerated by hand
# ---------------------------------------------------------------------------


def _golden_windows():
    cases = []
    with open(golden_path("windows.txt")) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            lhs, rhs = line.split(":")
            parts = lhs.split()
            cases.append((parts[0], [int(x) for x in parts[1:]], [int(x) for x in rhs.split()]))
    return cases


@pytest.mark.parametrize("case", _golden_windows(), ids=lambda c: "%s-%s" % (c[0], c[1]))
def test_golden_windows(case):
    kind, args, valid = case
    rng = np.random.default_rng(7)
    if kind == "prefill":
        N, ks, ke = args
        q = inputs.to_fp8_bytes(rng.standard_normal((1, 2, 4)).astype(np.float32))
        k = inputs.to_fp8_bytes(rng.standard_normal((N, 4)).astype(np.float32))
        out = oracle.prefill(q, k, np.ones(N, np.float32), np.ones((1, 2), np.float32),
                             np.array([ks], np.int32), np.array([ke], np.int32))
        got = [n for n in range(N) if not np.isneginf(out[0, n])]
    else:
        mml, ctx, next_n, row = args
        d = inputs.make_decode(1, next_n, [ctx], mml, seed=3, H=2, D=4, block_size=2)
        out = oracle.decode(d.q, d.kv_cache, d.weights, d.context_lens, d.block_tables, mml, 2)
        got = [p for p in range(mml) if not np.isneginf(out[row, p])]
    assert got == valid


# ---------------------------------------------------------------------------
# hand-worked example
# ---------------------------------------------------------------------------


def test_hand_example_prefill_and_decode():
    g = read_kv("hand_example.txt")
    q = inputs.to_fp8_bytes(floats(g["q"]).reshape(2, 2, 2).astype(np.float32))
    k = inputs.to_fp8_bytes(floats(g["k"]).reshape(3, 2).astype(np.float32))
    sc = floats(g["kv_scale"]).astype(np.float32)
    w = floats(g["weights"]).reshape(2, 2).astype(np.float32)
    ks = np.array([int(x) for x in g["ks"]], np.int32)
    ke = np.array([int(x) for x in g["ke"]], np.int32)
    exp = floats(g["prefill_expected"]).reshape(2, 3)
    out = oracle.prefill(q, k, sc, w, ks, ke)
    assert np.array_equal(out, exp)
    # the same numbers through a paged cache: block size 2, shuffled table
    table = np.array([[int(x) for x in g["decode_table"]]], np.int32)
    bs, D = 2, 2
    cache = np.full((2, bs * (D + 4)), 0x7F, np.uint8)  # NaN bytes in unused slots
    kview, sview = inputs.cache_views(cache, bs, D)
    for p in range(3):
        kview[table[0, p // bs], p % bs] = k[p]
        sview[table[0, p // bs], p % bs] = sc[p]
    qd = q.reshape(1, 2, 2, 2)
    dec = oracle.decode(qd, cache, w, np.array([3], np.int32), table, 4, bs)
    assert np.array_equal(dec, floats(g["decode_expected"]).reshape(2, 4))


# ---------------------------------------------------------------------------
# exact rational brute force
# ---------------------------------------------------------------------------


def _check_exact(out, vals, mags, ulps=64):
    """|oracle - exact| <= ulps * 2^-53 * sum_h |term_h| for every in-window pair."""
    for key, v in vals.items():
        o = out[key]
        assert math.isfinite(o)
        err = abs(Fraction(o) - v)
        bound = Fraction(ulps) * Fraction(1, 2 ** 53) * mags[key]
        assert err <= bound, (key, o, float(v))


@pytest.mark.parametrize("H,D,M,N,mode", [
    (1, 1, 5, 7, "causal"),
    (2, 3, 6, 8, "misaligned"),
    (32, 128, 4, 6, "causal"),
    (32, 64, 4, 6, "causal"),
    (64, 64, 3, 5, "multi_req"),
    (3, 16, 8, 8, "empty"),
    (2, 8, 6, 9, "past_end"),
    (4, 8, 8, 12, "multi_req"),
])
def test_prefill_matches_exact_brute_force(H, D, M, N, mode):
    p = inputs.make_prefill(M, N, seed=11 + H + D, H=H, D=D, windows=mode)
    out = oracle.prefill(p.q, p.k, p.kv_scale, p.weights, p.ks, p.ke)
    vals, mags = brute.prefill(p.q, p.k, p.kv_scale, p.weights, p.ks, p.ke)
    _check_exact(out, vals, mags)
    # and nothing outside the window is finite
    fin = {(m, n) for m in range(M) for n in range(N) if np.isfinite(out[m, n])}
    assert fin == set(vals.keys())


@pytest.mark.parametrize("H,D,B,next_n,bs,ctx", [
    (2, 4, 2, 2, 4, [5, 9]),
    (32, 128, 1, 3, 64, [70]),
    (2, 64, 2, 2, 16, [20, 33]),
    (2, 64, 2, 1, 1, [9, 4]),
    (3, 8, 3, 3, 2, [0, 2, 7]),
    (1, 1, 2, 1, 8, [17, 3]),
])
def test_decode_matches_exact_brute_force(H, D, B, next_n, bs, ctx):
    mml = max(max(ctx), 1) + 3
    d = inputs.make_decode(B, next_n, ctx, mml, seed=5 + H, H=H, D=D, block_size=bs, poison=True)
    out = oracle.decode(d.q, d.kv_cache, d.weights, d.context_lens, d.block_tables, mml, bs)
    vals, mags = brute.decode(d.q, d.kv_cache, d.weights, d.context_lens, d.block_tables, mml, bs)
    _check_exact(out, vals, mags)
    fin = {(r, p) for r in range(B * next_n) for p in range(mml) if np.isfinite(out[r, p])}
    assert fin == set(vals.keys())


def test_integer_inputs_are_exact():
    """Integer fp8 values in [-16,16], power-of-two weights and scales: every
    intermediate is exact, so the oracle must equal the exact result exactly."""
    rng = np.random.default_rng(3)
    M, N, H, D = 4, 6, 32, 128
    q = inputs.to_fp8_bytes(rng.integers(-16, 17, (M, H, D)).astype(np.float32))
    k = inputs.to_fp8_bytes(rng.integers(-16, 17, (N, D)).astype(np.float32))
    w = (rng.choice([-1, 1], (M, H)) * 2.0 ** -rng.integers(0, 4, (M, H))).astype(np.float32)
    sc = rng.choice([0.5, 1.0, 2.0], N).astype(np.float32)
    ks, ke = inputs.causal_windows(M, N)
    out = oracle.prefill(q, k, sc, w, ks, ke)
    vals, _ = brute.prefill(q, k, sc, w, ks, ke)
    for key, v in vals.items():
        assert Fraction(out[key]) == v


# ---------------------------------------------------------------------------
# closed forms through library routines
# ---------------------------------------------------------------------------


def test_single_head_unit_weights_is_matmul():
    """H = 1, w = 1, scale = 1: logits = max(Q K^T, 0); with Q, K >= 0 it is
    exactly the matrix product (numpy fp64 matmul, exact at these sizes)."""
    rng = np.random.default_rng(1)
    M, N, D = 9, 13, 128
    qf = rng.standard_normal((M, 1, D)).astype(np.float32)
    kf = rng.standard_normal((N, D)).astype(np.float32)
    for nonneg in (True, False):
        q = inputs.to_fp8_bytes(np.abs(qf) if nonneg else qf)
        k = inputs.to_fp8_bytes(np.abs(kf) if nonneg else kf)
        ks = np.zeros(M, np.int32)
        ke = np.full(M, N, np.int32)
        out = oracle.prefill(q, k, np.ones(N, np.float32), np.ones((M, 1), np.float32), ks, ke)
        ref = brute.fp8_values(q)[:, 0, :] @ brute.fp8_values(k).T
        assert np.array_equal(out, np.maximum(ref, 0.0))
        if nonneg:
            assert np.array_equal(out, ref)


def test_relu_odd_and_even_parts():
    """relu(x) - relu(-x) = x and relu(x) + relu(-x) = |x|.  Negating Q (flip
    the fp8 sign bit) therefore gives closed forms through a batched matmul:
      L(Q) - L(-Q) = scale_n * sum_h w_h <Q_h, K_n>
      L(Q) + L(-Q) = scale_n * sum_h w_h |<Q_h, K_n>|"""
    p = inputs.make_prefill(7, 40, seed=21, H=32, D=128)
    ks = np.zeros(7, np.int32)
    ke = np.full(7, 40, np.int32)
    a = oracle.prefill(p.q, p.k, p.kv_scale, p.weights, ks, ke)
    b = oracle.prefill(p.q ^ np.uint8(0x80), p.k, p.kv_scale, p.weights, ks, ke)
    S = np.matmul(brute.fp8_values(p.q), brute.fp8_values(p.k).T)   # [M, H, N], exact
    w = p.weights.astype(np.float64)[:, :, None]
    sc = p.kv_scale.astype(np.float64)[None, :]
    odd = (w * S).sum(axis=1) * sc
    even = (w * np.abs(S)).sum(axis=1) * sc
    scale = (np.abs(w * S).sum(axis=1) * sc).max()
    assert np.max(np.abs((a - b) - odd)) <= 1e-13 * scale
    assert np.max(np.abs((a + b) - even)) <= 1e-13 * scale
    # the relu matters: the odd part is far from zero
    assert np.max(np.abs(odd)) > 1e-3 * scale


# ---------------------------------------------------------------------------
# invariants of the definition
# ---------------------------------------------------------------------------


def test_hoisted_scale_equals_unhoisted():
    p = inputs.make_prefill(16, 200, seed=31)
    a = oracle.prefill(p.q, p.k, p.kv_scale, p.weights, p.ks, p.ke, hoist=False)
    b = oracle.prefill(p.q, p.k, p.kv_scale, p.weights, p.ks, p.ke, hoist=True)
    fin = np.isfinite(a)
    assert np.array_equal(fin, np.isfinite(b))
    assert np.max(np.abs(a[fin] - b[fin])) <= 1e-14 * np.max(np.abs(a[fin]))


@pytest.mark.parametrize("D", [128, 64])
def test_paged_decode_equals_contiguous_prefill(D):
    """Row (b, j) of decode = prefill over that sequence's gathered K with
    ks = 0, ke = ctx_b - next_n + j + 1, and -inf out to max_model_len."""
    B, next_n, mml = 3, 4, 300
    d = inputs.make_decode(B, next_n, [250, 3, 129], mml, seed=41, D=D, poison=True)
    dec = oracle.decode(d.q, d.kv_cache, d.weights, d.context_lens, d.block_tables, mml, 64)
    for b in range(B):
        ctx = int(d.context_lens[b])
        for j in range(next_n):
            row = b * next_n + j
            k = d.k_seq[b] if ctx else np.zeros((1, D), np.uint8)
            sc = d.s_seq[b] if ctx else np.ones(1, np.float32)
            N = k.shape[0]
            pre = oracle.prefill(d.q[b, j][None], k, sc, d.weights[row][None],
                                 np.array([0], np.int32), np.array([ctx - next_n + j + 1], np.int32))
            ref = np.full(mml, -np.inf)
            ref[:N] = pre[0]
            assert np.array_equal(dec[row], ref)


def test_zero_weights_give_zero():
    p = inputs.make_prefill(8, 64, seed=51)
    out = oracle.prefill(p.q, p.k, p.kv_scale, np.zeros_like(p.weights), p.ks, p.ke)
    fin = np.isfinite(out)
    assert fin.any() and np.all(out[fin] == 0.0)


def test_rows_are_independent():
    """Evaluating a subset of rows gives the same rows as the full call."""
    p = inputs.make_prefill(12, 90, seed=61, windows="multi_req")
    full = oracle.prefill(p.q, p.k, p.kv_scale, p.weights, p.ks, p.ke)
    sel = np.array([0, 5, 11])
    part = oracle.prefill(p.q[sel], p.k, p.kv_scale, p.weights[sel], p.ks[sel], p.ke[sel])
    assert np.array_equal(part, full[sel])


def test_head_permutation_pairs_weights_with_heads():
    """Permuting heads of Q and weights together changes nothing (up to the
    head-sum order); permuting Q's heads alone does."""
    p = inputs.make_prefill(6, 50, seed=71)
    perm = np.random.default_rng(0).permutation(32)
    a = oracle.prefill(p.q, p.k, p.kv_scale, p.weights, p.ks, p.ke)
    b = oracle.prefill(p.q[:, perm], p.k, p.kv_scale, p.weights[:, perm], p.ks, p.ke)
    c = oracle.prefill(p.q[:, perm], p.k, p.kv_scale, p.weights, p.ks, p.ke)
    fin = np.isfinite(a)
    tol = 1e-13 * np.max(np.abs(a[fin]))
    assert np.max(np.abs(a[fin] - b[fin])) <= tol
    assert np.max(np.abs(a[fin] - c[fin])) > 1e3 * tol


def test_scale_is_per_column_and_weight_per_row():
    """Doubling kv_scale[n0] doubles column n0 exactly and nothing else;
    doubling weights[m0, :] doubles row m0 exactly and nothing else."""
    p = inputs.make_prefill(6, 40, seed=81)
    ks = np.zeros(6, np.int32)
    ke = np.full(6, 40, np.int32)
    a = oracle.prefill(p.q, p.k, p.kv_scale, p.weights, ks, ke)
    sc = p.kv_scale.copy()
    sc[17] *= 2
    b = oracle.prefill(p.q, p.k, sc, p.weights, ks, ke)
    assert np.array_equal(b[:, 17], 2 * a[:, 17])
    assert np.array_equal(np.delete(b, 17, axis=1), np.delete(a, 17, axis=1))
    w = p.weights.copy()
    w[4] *= 2
    c = oracle.prefill(p.q, p.k, p.kv_scale, w, ks, ke)
    assert np.array_equal(c[4], 2 * a[4])
    assert np.array_equal(np.delete(c, 4, axis=0), np.delete(a, 4, axis=0))


def test_clean_false_leaves_outside_untouched():
    p = inputs.make_prefill(8, 70, seed=91, windows="empty")
    pre = np.full((8, 70), np.nan)
    out = oracle.prefill(p.q, p.k, p.kv_scale, p.weights, p.ks, p.ke, clean=False, out=pre)
    ref = oracle.prefill(p.q, p.k, p.kv_scale, p.weights, p.ks, p.ke)
    inside = ~np.isneginf(ref)
    assert np.array_equal(out[inside], ref[inside])
    assert np.all(np.isnan(out[~inside]))


def test_unowned_cache_slots_do_not_leak():
    """Poisoned (NaN) slots past the context and poisoned padding blocks never
    reach an in-window output."""
    d = inputs.make_decode(2, 2, [65, 130], 200, seed=101, poison=True)
    out = oracle.decode(d.q, d.kv_cache, d.weights, d.context_lens, d.block_tables, 200, 64)
    assert not np.isnan(out).any()


# ---------------------------------------------------------------------------
# the preshuffled (16,16) cache layout (reading of the aiter PR 5047 page,
# "Technical Details"; positions worked out by hand in the golden file)
# ---------------------------------------------------------------------------


def _layout_rows():
    rows = []
    with open(golden_path("preshuffle_layout.txt")) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                rows.append(tuple(int(x) for x in line.split()))
    return rows


def _one_hot_decode(bs, D, offset, byte, preshuffle):
    """Decode oracle over one block whose only nonzero K byte (1.0) sits at
    `offset`, with one head whose query is 1.0 at `byte`: the logit is 1 at
    the slot that byte belongs to and 0 at every other slot."""
    cache = np.zeros((1, bs * (D + 4)), dtype=np.uint8)
    cache[0, offset] = 0x38
    cache[0, bs * D:] = np.frombuffer(np.ones(bs, np.float32).tobytes(), dtype=np.uint8)
    q = np.zeros((1, 1, 1, D), dtype=np.uint8)
    q[0, 0, 0, byte] = 0x38
    w = np.ones((1, 1), dtype=np.float32)
    return oracle.decode(q, cache, w, np.array([bs], np.int32), np.zeros((1, 1), np.int32), bs,
                         bs, preshuffle=preshuffle)[0]


@pytest.mark.parametrize("row", _layout_rows(), ids=lambda r: "bs%d-off%d" % (r[0], r[2]))
def test_preshuffle_positions_worked_by_hand(row):
    bs, D, offset, slot, byte = row
    out = _one_hot_decode(bs, D, offset, byte, preshuffle=True)
    want = np.zeros(bs)
    want[slot] = 1.0
    assert np.array_equal(out, want)
    # the slot-major layout puts that byte at slot * D + byte instead
    out = _one_hot_decode(bs, D, slot * D + byte, byte, preshuffle=False)
    assert np.array_equal(out, want)


@pytest.mark.parametrize("row", _layout_rows(), ids=lambda r: "bs%d-off%d" % (r[0], r[2]))
def test_generator_preshuffle_matches_hand_positions(row):
    bs, D, offset, slot, byte = row
    plain = np.zeros((1, bs * (D + 4)), dtype=np.uint8)
    plain[0, slot * D + byte] = 1
    tiled = inputs.preshuffle_blocks(plain, bs, D)
    assert int(np.flatnonzero(tiled[0])[0]) == offset and int(tiled.sum()) == 1


@pytest.mark.parametrize("D", [128, 64])
@pytest.mark.parametrize("bs", [16, 64, 128])
def test_preshuffled_decode_equals_plain_decode(bs, D):
    """Invariant: the layout moves bytes, not values, so the oracle's logits on
    the preshuffled cache equal those on the slot-major cache of the same
    draws, bit for bit (ragged contexts, shuffled table, NaN-poisoned slots)."""
    kw = dict(B=3, next_n=3, context_lens=[5, bs + 7, 2 * bs], max_model_len=2 * bs + 8, seed=77,
              H=4, D=D, block_size=bs, poison=True)
    a = inputs.make_decode(**kw)
    b = inputs.make_decode(preshuffle=True, **kw)
    assert not np.array_equal(a.kv_cache, b.kv_cache)
    ra = oracle.decode(a.q, a.kv_cache, a.weights, a.context_lens, a.block_tables,
                       a.max_model_len, bs)
    rb = oracle.decode(b.q, b.kv_cache, b.weights, b.context_lens, b.block_tables,
                       b.max_model_len, bs, preshuffle=True)
    assert np.array_equal(ra, rb)
    # and reading the tiled bytes as if slot-major gives something else
    rc = oracle.decode(b.q, b.kv_cache, b.weights, b.context_lens, b.block_tables,
                       b.max_model_len, bs)
    assert not np.array_equal(np.nan_to_num(ra), np.nan_to_num(rc))


def test_preshuffle_needs_whole_tiles():
    q = np.zeros((1, 1, 1, 128), np.uint8)
    cache = np.zeros((1, 8 * 132), np.uint8)
    with pytest.raises(ValueError):
        oracle.decode(q, cache, np.ones((1, 1), np.float32), np.array([8], np.int32),
                      np.zeros((1, 1), np.int32), 8, 8, preshuffle=True)


# Hand-worked byte offsets of the preshuffled order at head dim 64 (16 rows of
# 64 bytes per tile group: a group is 1024 bytes, granule u of its 16 rows
# takes bytes 256 u .. 256 u + 255, row by row):
#   slot 0, byte 0   -> 0
#   slot 3, byte 17  -> granule 1, row 3: 256 + 48 + 1 = 305
#   slot 15, byte 63 -> granule 3, row 15: 768 + 240 + 15 = 1023
#   slot 17, byte 5  -> group 1 (1024), granule 0, row 1: 1024 + 16 + 5 = 1045
#   slot 33, byte 40 -> group 2 (2048), granule 2, row 1: 2048 + 512 + 16 + 8 = 2584
D64_TILED_POSITIONS = [(0, 0, 0), (3, 17, 305), (15, 63, 1023), (17, 5, 1045), (33, 40, 2584)]


@pytest.mark.parametrize("slot,byte,pos", D64_TILED_POSITIONS)
def test_preshuffle_positions_head_dim_64(slot, byte, pos):
    """The generator's preshuffled order at head dim 64 puts byte `byte` of
    slot `slot` at the hand-worked position, and the oracle reads it back from
    there: a one-hot K byte gives a logit only at that slot."""
    bs, D = 64, 64
    cache = np.zeros((1, bs * (D + 4)), np.uint8)
    k = cache[:, : bs * D].reshape(1, bs, D)
    k[0, slot, byte] = 0x38  # 1.0
    tiled = inputs.preshuffle_blocks(cache, bs, D)
    assert tiled[0, pos] == 0x38 and int(np.count_nonzero(tiled[0, : bs * D])) == 1
    tiled[0, bs * D:] = np.ones(bs, np.float32).view(np.uint8)  # unit scales
    q = np.zeros((1, 1, 1, D), np.uint8)
    q[0, 0, 0, byte] = 0x38
    out = oracle.decode(q, tiled, np.ones((1, 1), np.float32), np.array([bs], np.int32),
                        np.zeros((1, 1), np.int32), bs, bs, preshuffle=True)
    assert out[0, slot] == 1.0 and np.count_nonzero(out[0]) == 1
