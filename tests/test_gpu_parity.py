"""GPU parity: the HIP library (through its C ABI) against the CPU oracle on the
same seeded bytes.  Small and mid sizes are compared element by element in
full; they span several 64-token steps, ragged tails, every window mode, both
clean_logits settings, every next_n in 1..8 and every rows-per-wave
instantiation.  The full-size workloads are in test_gpu_workloads.py.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

from sparse_attention_indexer_scaled_amd import Tunables, inputs
from tests.gpu_util import (assert_parity, lib, oracle_decode, oracle_prefill, run_decode,
                            run_prefill, say)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    lib()
    from sparse_attention_indexer_scaled_amd import is_supported
    assert is_supported(32, 128, 0) and is_supported(32, 128, 64)


# ---------------------------------------------------------------------------
# exact integer pin: every intermediate is an exact fp32 value, so the GPU
# must equal the oracle bit for bit whatever its accumulation order.  This pins
# the fp8 format, the operand byte placement, the head <-> weight pairing and
# the lane layout of the cross-head reduction.
# ---------------------------------------------------------------------------


def _int_prefill(M, N, seed):
    rng = np.random.default_rng(seed)
    p = inputs.make_prefill(M, N, seed)
    p.q = inputs.to_fp8_bytes(rng.integers(-16, 17, (M, 32, 128)).astype(np.float32))
    p.k = inputs.to_fp8_bytes(rng.integers(-16, 17, (N, 128)).astype(np.float32))
    p.weights = (rng.choice([-1, 1], (M, 32)) * 2.0 ** -rng.integers(0, 4, (M, 32))).astype(np.float32)
    p.kv_scale = rng.choice([0.5, 1.0, 2.0], N).astype(np.float32)
    return p


@pytest.mark.parametrize("block_m", [1, 2, 4, 8, "ring"])
def test_prefill_integer_inputs_bit_exact(block_m):
    """Every rows-per-wave instantiation of the per-wave kernel, and the
    shared-K ring ("ring")."""
    p = _int_prefill(21, 333, seed=5 if block_m == "ring" else block_m)
    say("prefill int M=21 N=333 block_m=%s" % block_m)
    tun = Tunables(ring_depth=4) if block_m == "ring" else Tunables(block_m=block_m)
    out = run_prefill(p, tun=tun)
    ref, _ = oracle_prefill(p)
    if not np.array_equal(out, ref):
        bad = np.argwhere(out != ref)
        say("first mismatches (m, n, gpu, ref): %s" % [(int(m), int(n), float(out[m, n]), float(ref[m, n])) for m, n in bad[:8]])
    assert np.array_equal(out, ref)


@pytest.mark.parametrize("next_n", [1, 2, 3, 5, 8])
def test_decode_integer_inputs_bit_exact(next_n):
    rng = np.random.default_rng(next_n)
    d = inputs.make_decode(3, next_n, [700, 64, 131], 800, seed=next_n, poison=True)
    d.q = inputs.to_fp8_bytes(rng.integers(-16, 17, d.q.shape).astype(np.float32))
    d.weights = (rng.choice([-1, 1], d.weights.shape) * 2.0 ** -rng.integers(0, 4, d.weights.shape)).astype(np.float32)
    kview, sview = inputs.cache_views(d.kv_cache, 64, 128)
    used = d.num_blocks - 1  # the last block is the poison block
    kview[:used] = inputs.to_fp8_bytes(rng.integers(-16, 17, kview[:used].shape).astype(np.float32))
    sview[:used] = rng.choice([0.5, 1.0, 2.0], sview[:used].shape).astype(np.float32)
    say("decode int next_n=%d" % next_n)
    out = run_decode(d)
    ref, _, _ = oracle_decode(d)
    assert np.array_equal(out, ref)


# ---------------------------------------------------------------------------
# random inputs (the workloads' distributions), element by element
# ---------------------------------------------------------------------------

PREFILL_CASES = [
    # (M, N, window mode)
    (64, 512, "causal"),
    (37, 517, "causal"),
    (70, 700, "cp"),
    (33, 300, "misaligned"),
    (40, 260, "empty"),
    (29, 200, "past_end"),
    (64, 640, "multi_req"),
    (5, 3, "causal"),
    (1, 1, "causal"),
    (3, 2000, "causal"),
]


@pytest.mark.parametrize("M,N,mode", PREFILL_CASES, ids=[f"{m}x{n}-{w}" for m, n, w in PREFILL_CASES])
@pytest.mark.parametrize("clean", [1, 0])
def test_prefill_matches_oracle(M, N, mode, clean):
    p = inputs.make_prefill(M, N, seed=100 + M + N, windows=mode)
    say("prefill M=%d N=%d mode=%s clean=%d" % (M, N, mode, clean))
    out = run_prefill(p, clean=bool(clean))
    ref, mag = oracle_prefill(p)
    if clean:
        assert_parity(out, ref, mag, f"prefill_{M}x{N}_{mode}")
    else:
        win = np.isfinite(ref)
        assert np.isnan(out[~win]).all(), "clean_logits=0 wrote outside the window"
        out_w = np.where(win, out, -np.inf)
        assert_parity(out_w, ref, mag, f"prefill_{M}x{N}_{mode}_noclean")


@pytest.mark.parametrize("M,N,mode", PREFILL_CASES, ids=[f"{m}x{n}-{w}" for m, n, w in PREFILL_CASES])
def test_prefill_ring_matches_oracle(M, N, mode):
    """The shared-K ring forced on the same cases (the heuristic gives these
    small problems the per-wave kernel): one workgroup for M = 1, waves
    without rows, a single clamped step for N < 64."""
    p = inputs.make_prefill(M, N, seed=100 + M + N, windows=mode)
    ref, mag = oracle_prefill(p)
    for clean in (True, False):
        say("prefill ring M=%d N=%d mode=%s clean=%d" % (M, N, mode, clean))
        out = run_prefill(p, clean=clean, tun=Tunables(ring_depth=4))
        if clean:
            assert_parity(out, ref, mag, f"prefill_ring_{M}x{N}_{mode}")
        else:
            win = np.isfinite(ref)
            assert np.isnan(out[~win]).all(), "clean_logits=0 wrote outside the window"
            assert_parity(np.where(win, out, -np.inf), ref, mag, f"prefill_ring_{M}x{N}_{mode}_noclean")
        assert np.array_equal(out, run_prefill(p, clean=clean), equal_nan=True)


DECODE_CASES = [
    # (B, next_n, context lens, max_model_len)
    (2, 1, [1000, 333], 1024),
    (3, 2, [64, 65, 63], 200),
    (2, 3, [1, 2], 130),          # contexts shorter than next_n
    (4, 4, [0, 3, 700, 4096], 4096),
    (2, 5, [513, 1111], 1200),
    (2, 6, [2000, 7], 2001),      # max_model_len not a multiple of 64
    (1, 7, [300], 333),
    (2, 8, [129, 1025], 1100),
]


@pytest.mark.parametrize("B,next_n,ctx,mml", DECODE_CASES,
                         ids=[f"B{b}-nn{n}-mml{m}" for b, n, _, m in DECODE_CASES])
@pytest.mark.parametrize("clean", [1, 0])
def test_decode_matches_oracle(B, next_n, ctx, mml, clean):
    d = inputs.make_decode(B, next_n, ctx, mml, seed=200 + next_n, poison=True)
    say("decode B=%d next_n=%d ctx=%s mml=%d clean=%d" % (B, next_n, ctx, mml, clean))
    out = run_decode(d, clean=bool(clean))
    ref, mag, _ = oracle_decode(d)
    if clean:
        assert_parity(out, ref, mag, f"decode_B{B}_nn{next_n}")
    else:
        win = np.isfinite(ref)
        assert np.isnan(out[~win]).all(), "clean_logits=0 wrote outside the window"
        assert_parity(np.where(win, out, -np.inf), ref, mag, f"decode_B{B}_nn{next_n}_noclean")


def _row_instantiations():
    """(next_n, rows_per_block) pairs reaching every (rows per wave, waves per
    workgroup) kernel instantiation once."""
    seen, out = set(), []
    for nn in range(1, 9):
        for rows in range(1, min(4, nn) + 1):
            key = (rows, -(-nn // rows))
            if key not in seen:
                seen.add(key)
                out.append((nn, rows))
    return out


@pytest.mark.parametrize("next_n,rows", _row_instantiations())
def test_decode_every_row_grouping(next_n, rows):
    """Every rows-per-wave x waves-per-workgroup instantiation, including row
    groups that do not divide next_n (the last wave of the workgroup is short)."""
    d = inputs.make_decode(2, next_n, [900, 77], 1000, seed=300 + 10 * next_n + rows, poison=True)
    say("decode next_n=%d rows_per_block=%d" % (next_n, rows))
    out = run_decode(d, tun=Tunables(rows_per_block=rows))
    ref, mag, _ = oracle_decode(d)
    assert_parity(out, ref, mag, f"decode_nn{next_n}_rows{rows}")


@pytest.mark.parametrize("depth", [2, 3, 5, 7])
def test_decode_every_ring_depth(depth):
    """LDS ring depths other than the default, with splits that leave some
    workgroups fewer steps than the ring holds."""
    d = inputs.make_decode(3, 5, [700, 130, 3000], 3072, seed=310 + depth, poison=True)
    say("decode ring_depth=%d" % depth)
    for split in (1, 7):
        out = run_decode(d, tun=Tunables(ring_depth=depth, split_kv=split))
        ref, mag, _ = oracle_decode(d)
        assert_parity(out, ref, mag, f"decode_depth{depth}_split{split}")


BLOCK_SIZE_CASES = [
    (3, 2, [700, 130, 3000], 3072),
    (2, 6, [2000, 7], 2001),
    (4, 1, [0, 15, 17, 4100], 4160),
    (2, 3, [1, 2], 130),
]


@pytest.mark.parametrize("bs", [1, 16, 128])
@pytest.mark.parametrize("B,next_n,ctx,mml", BLOCK_SIZE_CASES,
                         ids=[f"B{b}-nn{n}-mml{m}" for b, n, _, m in BLOCK_SIZE_CASES])
def test_decode_other_block_sizes(bs, B, next_n, ctx, mml):
    """Per-token, 16- and 128-token cache blocks (a step spans 64 blocks, four
    blocks, or half of one); contexts that end mid-block, shorter than a step,
    or empty."""
    d = inputs.make_decode(B, next_n, ctx, mml, seed=330 + bs + mml, block_size=bs, poison=True)
    say("decode bs=%d B=%d next_n=%d ctx=%s mml=%d" % (bs, B, next_n, ctx, mml))
    ref, mag, _ = oracle_decode(d)
    for tun in (None, Tunables(split_kv=3), Tunables(rows_per_block=1, split_kv=1)):
        out = run_decode(d, tun=tun)
        assert_parity(out, ref, mag, f"decode_bs{bs}_B{B}_nn{next_n}")


@pytest.mark.parametrize("D", [128, 64])
@pytest.mark.parametrize("next_n", [4, 5, 7, 8])
def test_per_token_blocks_many_waves(next_n, D):
    """Per-token blocks with one row per wave, so next_n waves split each
    step's K chunks: 4-8 waves, where a wave requests one or two chunks and,
    when the wave count does not divide the chunk count, the last chunks'
    waves request one fewer."""
    d = inputs.make_decode(2, next_n, [1500, 70], 1536, seed=335 + next_n + D, D=D, block_size=1,
                           poison=True)
    say("decode bs=1 D=%d next_n=%d rows_per_block=1" % (D, next_n))
    ref, mag, _ = oracle_decode(d)
    for tun in (Tunables(rows_per_block=1), Tunables(rows_per_block=1, split_kv=5)):
        out = run_decode(d, tun=tun)
        assert_parity(out, ref, mag, f"decode_bs1_D{D}_nn{next_n}_rows1")


@pytest.mark.parametrize("bs", [1, 16, 128])
def test_block_size_does_not_change_bits(bs):
    """The same tokens paged through 1-, 16- or 128-token blocks give the
    64-token layout's output bit for bit (the gather is the only step that
    changes)."""
    d64 = inputs.make_decode(3, 4, [900, 64, 2500], 2560, seed=340)
    d = inputs.make_decode(3, 4, [900, 64, 2500], 2560, seed=340, block_size=bs)
    assert all(np.array_equal(a, b) for a, b in zip(d64.k_seq, d.k_seq))
    assert np.array_equal(run_decode(d64), run_decode(d), equal_nan=True)


@pytest.mark.parametrize("bs", [16, 64, 128])
@pytest.mark.parametrize("B,next_n,ctx,mml", BLOCK_SIZE_CASES,
                         ids=[f"B{b}-nn{n}-mml{m}" for b, n, _, m in BLOCK_SIZE_CASES])
def test_decode_preshuffled_layout(bs, B, next_n, ctx, mml):
    """Blocks whose K rows are in the preshuffled (16,16) order, against the
    oracle's own reading of that order; ragged, short and empty contexts,
    NaN-poisoned unused slots."""
    d = inputs.make_decode(B, next_n, ctx, mml, seed=350 + bs + mml, block_size=bs, poison=True,
                           preshuffle=True)
    say("decode preshuffled bs=%d B=%d next_n=%d ctx=%s mml=%d" % (bs, B, next_n, ctx, mml))
    ref, mag, _ = oracle_decode(d)
    tuns = [None, Tunables(split_kv=3), Tunables(rows_per_block=1, split_kv=1)]
    if bs == 64:
        tuns += [Tunables(ring_depth=2), Tunables(ring_depth=6, split_kv=2)]
    for tun in tuns:
        out = run_decode(d, tun=tun)
        assert_parity(out, ref, mag, f"decode_preshuffled_bs{bs}_B{B}_nn{next_n}")


@pytest.mark.parametrize("H", [32, 64, 128])
@pytest.mark.parametrize("bs", [16, 64, 128])
def test_preshuffled_layout_does_not_change_bits(bs, H):
    """The same draws stored slot-major and preshuffled give the same output
    bit for bit: the layout changes only where the loads read from."""
    kw = dict(B=3, next_n=4, context_lens=[900, 64, 2500], max_model_len=2560, seed=341, H=H,
              block_size=bs)
    plain = inputs.make_decode(**kw)
    tiled = inputs.make_decode(preshuffle=True, **kw)
    say("decode preshuffled vs slot-major bs=%d H=%d" % (bs, H))
    assert not np.array_equal(plain.kv_cache, tiled.kv_cache)
    assert np.array_equal(run_decode(plain), run_decode(tiled), equal_nan=True)


# ---------------------------------------------------------------------------
# GPU self-invariants (bitwise)
# ---------------------------------------------------------------------------


def test_prefill_tunables_do_not_change_bits():
    p = inputs.make_prefill(45, 1500, seed=401, windows="multi_req")
    base = run_prefill(p)
    for tun in [Tunables(block_m=1), Tunables(block_m=2, split_n=3), Tunables(block_m=8, num_warps=1),
                Tunables(split_n=7, num_warps=2, reverse_rows=1), Tunables(reverse_rows=-1),
                Tunables(block_m=4, split_n=40, num_warps=3),
                # the shared-K ring: 45 rows leave the last workgroup's last
                # wave one row; 40 splits leave some parts without a step
                Tunables(ring_depth=2), Tunables(ring_depth=4, split_n=3),
                Tunables(ring_depth=7, split_n=1, reverse_rows=1), Tunables(ring_depth=5, split_n=40),
                Tunables(ring_depth=1, split_n=2)]:
        say("prefill tunables %s" % [getattr(tun, f) for f, _ in Tunables._fields_])
        assert np.array_equal(run_prefill(p, tun=tun), base, equal_nan=True)


@pytest.mark.parametrize("mode", ["causal", "cp", "misaligned", "empty", "past_end", "multi_req"])
def test_prefill_ring_equals_per_wave_kernel(mode):
    """The shared-K ring (the default at 32 heads, head dim 128) against the
    per-wave kernel, bit for bit, with and without the -inf fill: a row count
    that is no multiple of the 16-row workgroup and columns that end inside a
    step."""
    p = inputs.make_prefill(1000, 3000, seed=405, windows=mode)
    for clean in (True, False):
        want = run_prefill(p, clean=clean, tun=Tunables(ring_depth=1))
        for tun in (None, Tunables(ring_depth=3, split_n=5)):
            say("prefill ring mode=%s clean=%d" % (mode, clean))
            assert np.array_equal(run_prefill(p, clean=clean, tun=tun), want, equal_nan=True)


@pytest.mark.parametrize("H", [64, 128])
@pytest.mark.parametrize("mode", ["causal", "multi_req", "empty"])
def test_prefill_ring_64_and_128_heads_equals_per_wave_kernel(mode, H):
    """The shared-K ring at 64 heads (4 waves of 2 rows) and 128 heads (4
    waves of 1 row) against the per-wave kernel, bit for bit."""
    p = inputs.make_prefill(1000, 3000, seed=406, H=H, windows=mode)
    for clean in (True, False):
        want = run_prefill(p, clean=clean, tun=Tunables(ring_depth=1))
        for tun in (None, Tunables(ring_depth=4), Tunables(ring_depth=3, split_n=5, reverse_rows=1)):
            say("prefill ring %d heads mode=%s clean=%d" % (H, mode, clean))
            assert np.array_equal(run_prefill(p, clean=clean, tun=tun), want, equal_nan=True)


def test_decode_tunables_do_not_change_bits():
    d = inputs.make_decode(3, 6, [2000, 150, 1300], 2048, seed=402, poison=True)
    base = run_decode(d)
    for tun in [Tunables(rows_per_block=1), Tunables(rows_per_block=4, split_kv=1),
                Tunables(rows_per_block=3, split_kv=9, ring_depth=2), Tunables(split_kv=64),
                Tunables(rows_per_block=2, ring_depth=7), Tunables(rows_per_block=4, split_kv=3, ring_depth=3),
                Tunables(rows_per_block=2, split_kv=5)]:
        say("decode tunables %s" % [getattr(tun, f) for f, _ in Tunables._fields_])
        assert np.array_equal(run_decode(d, tun=tun), base, equal_nan=True)


def test_decode_block_pool_permutation_invariance():
    """Moving the physical blocks around (and updating the table) must not
    change a single bit: the kernel reads K through the table, not by walking
    the cache."""
    d = inputs.make_decode(3, 2, [500, 64, 1000], 1024, seed=403)
    base = run_decode(d)
    perm = np.random.default_rng(0).permutation(d.num_blocks)
    inv = np.argsort(perm)
    d.kv_cache = d.kv_cache[perm]          # new block i holds old block perm[i]
    d.block_tables = inv[d.block_tables].astype(np.int32)
    assert np.array_equal(run_decode(d), base)


def test_power_of_two_homogeneity():
    """Doubling kv_scale or the weights doubles every finite output exactly."""
    p = inputs.make_prefill(17, 400, seed=404)
    base = run_prefill(p)
    p2 = inputs.make_prefill(17, 400, seed=404)
    p2.kv_scale = p2.kv_scale * np.float32(2)
    assert np.array_equal(run_prefill(p2), np.where(np.isfinite(base), 2 * base, base))
    p3 = inputs.make_prefill(17, 400, seed=404)
    p3.weights = p3.weights * np.float32(0.5)
    assert np.array_equal(run_prefill(p3), np.where(np.isfinite(base), 0.5 * base, base))


def test_paged_decode_equals_contiguous_prefill_on_gpu():
    """Row (b, j) of decode equals the prefill kernel over that sequence's K with
    ks = 0, ke = ctx - next_n + j + 1 (within the fp32 bound; the two kernels
    may order their sums differently)."""
    d = inputs.make_decode(2, 3, [777, 130], 800, seed=405, poison=True)
    dec = run_decode(d)
    for b in range(2):
        ctx = int(d.context_lens[b])
        p = inputs.PrefillInputs(d.q[b], d.k_seq[b], d.s_seq[b], d.weights[b * 3:(b + 1) * 3],
                                 np.zeros(3, np.int32), (ctx - 3 + np.arange(3) + 1).astype(np.int32))
        pre = run_prefill(p)
        ref = np.full((3, 800), -np.inf)
        ref[:, :ctx] = pre
        _, mag_full, _ = oracle_decode(d, seqs=[b])
        assert_parity(dec[b * 3:(b + 1) * 3], ref, mag_full, f"paged_vs_contig_{b}")


def test_empty_problems_are_noops():
    from sparse_attention_indexer_scaled_amd import mqa_logits_prefill, paged_mqa_logits_decode
    z8 = torch.zeros((0, 32, 128), dtype=torch.uint8, device="cuda")
    k = torch.zeros((5, 128), dtype=torch.uint8, device="cuda")
    out = mqa_logits_prefill(z8, k, torch.ones(5, device="cuda"), torch.zeros((0, 32), device="cuda"),
                             torch.zeros(0, dtype=torch.int32, device="cuda"),
                             torch.zeros(0, dtype=torch.int32, device="cuda"))
    assert out.shape == (0, 5)
    q = torch.zeros((0, 1, 32, 128), dtype=torch.uint8, device="cuda")
    cache = torch.zeros((1, 64 * 132), dtype=torch.uint8, device="cuda")
    out = paged_mqa_logits_decode(q, cache, torch.zeros((0, 32), device="cuda"),
                                  torch.zeros(0, dtype=torch.int32, device="cuda"),
                                  torch.zeros((0, 1), dtype=torch.int32, device="cuda"), 64)
    assert out.shape == (0, 64)
    torch.cuda.synchronize()


# ---------------------------------------------------------------------------
# large sizes
# ---------------------------------------------------------------------------


def test_decode_max_model_len_one_million():
    """max_model_len 1048576 (the long-context setting the issue page about
    next_n tiling measures with) and contexts far shorter: the -inf fill
    covers almost every row, every window is exact."""
    d = inputs.make_decode(2, 2, [131072, 5000], 1048576, seed=420, poison=True)
    say("decode mml=1048576")
    out = run_decode(d)
    ref, mag, _ = oracle_decode(d)
    assert_parity(out, ref, mag, "decode_mml1M")


def test_prefill_long_rows_few_queries():
    """A handful of query rows over 131072 columns (large N, tiny M)."""
    p = inputs.make_prefill(8, 131072, seed=421, windows="causal")
    say("prefill M8 N131072")
    out = run_prefill(p)
    ref, mag = oracle_prefill(p)
    assert_parity(out, ref, mag, "prefill_M8_N131072")
