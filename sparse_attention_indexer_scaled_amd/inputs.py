"""Seeded synthetic inputs for the lightning-indexer logits op.

This module only *produces* inputs.  It holds none of the op's arithmetic (no
dot products, no ReLU, no head sum, no masking), so the GPU path and the CPU
oracle can both consume its bytes without sharing any of the method's code.

What it does:

* draws Q, K and the per-row head weights from a numpy PCG64 generator;
* quantises K per token to fp8 e4m3fn with an fp32 dequant scale
  ``scale = max(amax, 1e-12) / 448`` (the producer side of the co-packed
  cache described on the aiter PR 5047 page, "Motivation": K is stored as fp8
  next to a per-token dequant scale);
* casts to fp8 e4m3fn with torch's CPU conversion (round to nearest even),
  after clamping to the format's finite range [-448, 448];
* builds prefill windows (``cu_seqlen_ks`` / ``cu_seqlen_ke``, aiter PR 5046
  page, "Motivation") and paged-decode block tables;
* packs K and its scale into the paged cache layout documented in
  ``include/mqa_indexer.h``: block ``i`` is ``block_size * (D + 4)`` bytes, the
  first ``block_size * D`` bytes are the K rows of its slots (slot-major), the
  last ``block_size * 4`` bytes are their fp32 scales.

Draw order per input set (fixed, so a seed names one input exactly):
context lengths (decode only), Q, K, weights, block permutation.
"""

from __future__ import annotations

import dataclasses
import math
from typing import Optional, Sequence

import numpy as np
import torch

FP8_MAX = 448.0
HEADS = 32
HEAD_DIM = 128
KV_BLOCK = 64
TABLE_PAD = 0  # padding entry written into unused block-table lanes

# ---------------------------------------------------------------------------
# fp8 encoding (input preparation only)
# ---------------------------------------------------------------------------


def to_fp8_bytes(x: np.ndarray) -> np.ndarray:
    """Encode float32 values as fp8 e4m3fn codes (uint8), round-to-nearest-even.

    Values are clamped to [-448, 448] first: torch's conversion maps anything
    past the largest finite code to NaN instead of saturating.
    """
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    t = t.clamp_(-FP8_MAX, FP8_MAX)
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def quantize_tokens(x: np.ndarray):
    """Per-token fp8 quantisation of K rows ``x[..., D]``.

    Returns ``(codes uint8[..., D], scale float32[...])`` with
    ``scale = max(amax, 1e-12) / 448`` so each token's largest element lands on
    +-448.
    """
    x = np.asarray(x, dtype=np.float32)
    amax = np.abs(x).max(axis=-1)
    scale = (np.maximum(amax, np.float32(1e-12)) / np.float32(FP8_MAX)).astype(np.float32)
    codes = to_fp8_bytes(x / scale[..., None])
    return codes, scale


# ---------------------------------------------------------------------------
# prefill
# ---------------------------------------------------------------------------


@dataclasses.dataclass
class PrefillInputs:
    q: np.ndarray        # uint8 [M, H, D]   fp8 e4m3fn codes
    k: np.ndarray        # uint8 [N, D]
    kv_scale: np.ndarray  # float32 [N]
    weights: np.ndarray  # float32 [M, H]
    ks: np.ndarray       # int32 [M]
    ke: np.ndarray       # int32 [M]

    @property
    def M(self):
        return self.q.shape[0]

    @property
    def N(self):
        return self.k.shape[0]

    @property
    def H(self):
        return self.q.shape[1]

    @property
    def D(self):
        return self.q.shape[2]


def causal_windows(M: int, N: int):
    """One request per chunk: ks = 0 and ke[m] = N - M + m + 1 (a causal triangle)."""
    ks = np.zeros(M, dtype=np.int32)
    ke = (N - M + np.arange(M, dtype=np.int64) + 1).astype(np.int32)
    return ks, ke


def window_mode(mode: str, M: int, N: int, rng: np.random.Generator):
    """Window patterns named after the prefill page's test modes (aiter PR 5046,
    "Test Plan": causal, cp, misaligned, empty, past_end, multi_req).

    The page names the modes but not their exact construction; these are our
    readings, each a legal, adversarial window set.
    """
    if mode == "causal":
        return causal_windows(M, N)
    if mode == "cp":
        # context-parallel style: this chunk holds a middle slice of a longer
        # request, so every row starts at 0 and ends somewhere mid-buffer.
        off = N // 3
        ks = np.zeros(M, dtype=np.int32)
        ke = np.minimum(off + np.arange(M) + 1, N).astype(np.int32)
        return ks, ke
    if mode == "misaligned":
        # starts and ends away from any 32- or 64-column boundary
        base = 5
        ks = np.full(M, base, dtype=np.int32) + (np.arange(M) % 3).astype(np.int32)
        ke = np.minimum(ks + 7 + 13 * np.arange(M), N).astype(np.int32)
        ke = np.maximum(ke, ks)
        return ks, ke.astype(np.int32)
    if mode == "empty":
        # rows whose window is empty: ke < 0, ke < ks, ke == ks, mixed with
        # ordinary rows
        ks, ke = causal_windows(M, N)
        ks = ks.copy()
        ke = ke.copy()
        ke[0::4] = -3
        ks[1::4] = ke[1::4] + 2
        ks[2::4] = ke[2::4]
        return ks.astype(np.int32), ke.astype(np.int32)
    if mode == "past_end":
        # bounds beyond the K buffer: ks past N on some rows, ke past N on all
        ks = rng.integers(0, N, size=M).astype(np.int32)
        ks[0::3] = N + 7
        ke = (N + 1 + rng.integers(0, 64, size=M)).astype(np.int32)
        return ks, ke
    if mode == "multi_req":
        # four requests packed into one chunk; ks jumps at each boundary and
        # row blocks straddle requests
        nreq = 4
        rows = np.array_split(np.arange(M), nreq)
        cols = np.linspace(0, N, nreq + 1).astype(np.int64)
        ks = np.zeros(M, dtype=np.int64)
        ke = np.zeros(M, dtype=np.int64)
        for r, idx in enumerate(rows):
            if len(idx) == 0:
                continue
            c0, c1 = cols[r], cols[r + 1]
            ks[idx] = c0
            ke[idx] = np.minimum(c1 - len(idx) + np.arange(len(idx)) + 1, c1)
            ke[idx] = np.maximum(ke[idx], c0)
        return ks.astype(np.int32), ke.astype(np.int32)
    raise ValueError(f"unknown window mode {mode!r}")


def make_prefill(M: int, N: int, seed: int, H: int = HEADS, D: int = HEAD_DIM,
                 windows: str = "causal", ks=None, ke=None) -> PrefillInputs:
    rng = np.random.Generator(np.random.PCG64(seed))
    q = to_fp8_bytes(rng.standard_normal((M, H, D), dtype=np.float32))
    k, kv_scale = quantize_tokens(rng.standard_normal((N, D), dtype=np.float32))
    w = (rng.standard_normal((M, H), dtype=np.float32) / np.float32(math.sqrt(H))).astype(np.float32)
    if ks is None:
        ks, ke = window_mode(windows, M, N, rng)
    return PrefillInputs(q, k, kv_scale, w, np.asarray(ks, np.int32), np.asarray(ke, np.int32))


# ---------------------------------------------------------------------------
# paged decode
# ---------------------------------------------------------------------------


@dataclasses.dataclass
class DecodeInputs:
    q: np.ndarray             # uint8 [B, next_n, H, D]
    kv_cache: np.ndarray      # uint8 [num_blocks, block_size * (D + 4)]
    weights: np.ndarray       # float32 [B * next_n, H]
    context_lens: np.ndarray  # int32 [B]
    block_tables: np.ndarray  # int32 [B, max_blocks_per_seq]
    max_model_len: int
    block_size: int
    # the same K and scales, unpaged: k_seq[b] is uint8 [ctx_b, D]
    k_seq: list
    s_seq: list
    # K rows of each block in the (16,16)-tiled order (see preshuffle_blocks)
    preshuffle: bool = False

    @property
    def B(self):
        return self.q.shape[0]

    @property
    def next_n(self):
        return self.q.shape[1]

    @property
    def H(self):
        return self.q.shape[2]

    @property
    def D(self):
        return self.q.shape[3]

    @property
    def num_blocks(self):
        return self.kv_cache.shape[0]


def cache_views(cache: np.ndarray, block_size: int, D: int):
    """(K view uint8 [nb, bs, D], scale view float32 [nb, bs]) of a packed cache."""
    nb = cache.shape[0]
    kview = cache[:, : block_size * D].reshape(nb, block_size, D)
    sview = cache[:, block_size * D:].view(np.float32).reshape(nb, block_size)
    return kview, sview


def preshuffle_blocks(cache: np.ndarray, block_size: int, D: int) -> np.ndarray:
    """The same blocks with their K rows rearranged into the preshuffled (16,16)
    order: a block's slots in groups of 16; within a group, 16-byte column
    granule u of all 16 slots (slot by slot) before granule u + 1.  Scales are
    unchanged.  A pure byte permutation."""
    nb = cache.shape[0]
    out = cache.copy()
    k = cache[:, : block_size * D].reshape(nb, block_size // 16, 16, D // 16, 16)
    out[:, : block_size * D] = k.transpose(0, 1, 3, 2, 4).reshape(nb, block_size * D)
    return out


def make_decode(B: int, next_n: int, context_lens, max_model_len: int, seed: int,
                H: int = HEADS, D: int = HEAD_DIM, block_size: int = KV_BLOCK,
                ctx_range: Optional[Sequence[int]] = None, poison: bool = False,
                extra_table_cols: int = 0, preshuffle: bool = False) -> DecodeInputs:
    """Build one paged-decode input set.

    ``context_lens``: an int (uniform), a sequence of B ints, or None together
    with ``ctx_range=(lo, hi)`` to draw each length uniformly from [lo, hi].

    The physical pool holds exactly sum(ceil(ctx_b / block_size)) blocks in a
    seeded random order, plus (with ``poison``) one extra block of NaN bytes
    that every unused table lane points to.  Slots past a sequence's context
    hold NaN bytes (K code 0x7F, scale NaN) with ``poison``, zeros otherwise.
    ``preshuffle`` stores each block's K rows in the (16,16)-tiled order; the
    draws are the same, so the logical K is the same as without it.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    if context_lens is None:
        lo, hi = ctx_range
        ctx = rng.integers(lo, hi, size=B, endpoint=True).astype(np.int32)
    elif np.isscalar(context_lens):
        ctx = np.full(B, int(context_lens), dtype=np.int32)
    else:
        ctx = np.asarray(context_lens, dtype=np.int32)
    assert ctx.shape == (B,)
    assert (ctx >= 0).all() and (ctx <= max_model_len).all()

    q = to_fp8_bytes(rng.standard_normal((B, next_n, H, D), dtype=np.float32))
    k_seq, s_seq = [], []
    for b in range(B):
        kb, sb = quantize_tokens(rng.standard_normal((int(ctx[b]), D), dtype=np.float32))
        k_seq.append(kb)
        s_seq.append(sb)
    w = (rng.standard_normal((B * next_n, H), dtype=np.float32) / np.float32(math.sqrt(H))).astype(np.float32)

    nblk = (ctx.astype(np.int64) + block_size - 1) // block_size
    used = int(nblk.sum())
    perm = rng.permutation(used).astype(np.int64)
    max_blocks_per_seq = (max_model_len + block_size - 1) // block_size + extra_table_cols
    num_blocks = used + (1 if poison else 0)
    pad = used if poison else TABLE_PAD
    tables = np.full((B, max_blocks_per_seq), pad, dtype=np.int32)
    stride = block_size * (D + 4)
    cache = np.full((num_blocks, stride), 0x7F if poison else 0, dtype=np.uint8)
    kview, sview = cache_views(cache, block_size, D)
    if poison:
        sview[:] = np.float32("nan")
    off = 0
    for b in range(B):
        n = int(nblk[b])
        phys = perm[off: off + n]
        off += n
        tables[b, :n] = phys
        c = int(ctx[b])
        if c == 0:
            continue
        p = np.arange(c)
        kview[phys[p // block_size], p % block_size] = k_seq[b]
        sview[phys[p // block_size], p % block_size] = s_seq[b]
    if preshuffle:
        cache = preshuffle_blocks(cache, block_size, D)
    return DecodeInputs(q, cache, w, ctx, tables, int(max_model_len), block_size, k_seq, s_seq,
                        preshuffle)


# ---------------------------------------------------------------------------
# named workloads
# ---------------------------------------------------------------------------

CONFIGS = {
    0: dict(kind="prefill", name="prefill_M64_N512", M=64, N=512),
    1: dict(kind="decode", name="decode_B16_nn1_ctx8192", B=16, next_n=1, ctx=8192, mml=8192),
    2: dict(kind="decode", name="decode_B16_nn6_ctx131072", B=16, next_n=6, ctx=131072, mml=131072),
    3: dict(kind="prefill", name="prefill_M4096_N32768", M=4096, N=32768),
    4: dict(kind="decode", name="decode_B64_nn4_ragged1K-128K", B=64, next_n=4, ctx=None,
            ctx_range=(1024, 131072), mml=131072),
    # the headline decode shape in the other cache layouts (16-token blocks,
    # and per-token blocks: the plain co-packed cache)
    9: dict(kind="decode", name="decode_B16_nn6_ctx131072_bs16", B=16, next_n=6, ctx=131072,
            mml=131072, block_size=16),
    10: dict(kind="decode", name="decode_B16_nn6_ctx131072_bs1", B=16, next_n=6, ctx=131072,
             mml=131072, block_size=1),
    # the headline decode shape and the long prefill chunk with 64 and 128
    # index heads (the same K bytes, more contraction per byte)
    11: dict(kind="decode", name="decode_B16_nn6_ctx131072_h64", B=16, next_n=6, ctx=131072,
             mml=131072, H=64),
    12: dict(kind="decode", name="decode_B16_nn6_ctx131072_h128", B=16, next_n=6, ctx=131072,
             mml=131072, H=128),
    13: dict(kind="prefill", name="prefill_M4096_N32768_h64", M=4096, N=32768, H=64),
    # the headline decode shape in the preshuffled (16,16) 64-token cache
    14: dict(kind="decode", name="decode_B16_nn6_ctx131072_preshuffle", B=16, next_n=6,
             ctx=131072, mml=131072, preshuffle=True),
    # the long prefill chunk at head dim 64
    15: dict(kind="prefill", name="prefill_M4096_N32768_d64", M=4096, N=32768, D=64),
    # the headline decode shape in 128-token blocks at 32, 64 and 128 heads
    # (the block size the next_n-tiling issue page quotes its head sweep on)
    18: dict(kind="decode", name="decode_B16_nn6_ctx131072_bs128", B=16, next_n=6, ctx=131072,
             mml=131072, block_size=128),
    19: dict(kind="decode", name="decode_B16_nn6_ctx131072_h64_bs128", B=16, next_n=6,
             ctx=131072, mml=131072, H=64, block_size=128),
    20: dict(kind="decode", name="decode_B16_nn6_ctx131072_h128_bs128", B=16, next_n=6,
             ctx=131072, mml=131072, H=128, block_size=128),
    # the headline decode shape at head dim 64 (64-byte K rows)
    21: dict(kind="decode", name="decode_B16_nn6_ctx131072_d64", B=16, next_n=6, ctx=131072,
             mml=131072, D=64),
    # the long-context decode at next_n 1: the read stream with the least
    # compute per byte (the shape of the issue page's ~5.4 TB/s figure)
    22: dict(kind="decode", name="decode_B16_nn1_ctx131072", B=16, next_n=1, ctx=131072,
             mml=131072),
    # the long prefill chunk with 128 index heads
    25: dict(kind="prefill", name="prefill_M4096_N32768_h128", M=4096, N=32768, H=128),
}


def _pages_decode(B, next_n, kv_len, block_size):
    """A decode shape of the fp8 paged MQA logits PR page's performance table
    ("Test Result": 32 heads, head dim 128, ragged contexts): each context
    drawn uniformly from kv_len +/- 30 %, max_model_len the largest possible
    draw rounded up to 64 tokens; 64-token blocks preshuffled, as the table
    has them.  Context figures only: those of another kernel."""
    lo, hi = int(0.7 * kv_len), int(1.3 * kv_len)
    return dict(kind="decode", name="pages_B%d_nn%d_L%d_bs%d" % (B, next_n, kv_len, block_size),
                B=B, next_n=next_n, ctx=None, ctx_range=(lo, hi), mml=(hi + 63) // 64 * 64,
                block_size=block_size, preshuffle=block_size == 64)


# The shapes of that table with its HIP kernel's time in us: index ->
# (workload, page's HIP us).
PAGES_TABLE = {
    30: (_pages_decode(1, 2, 32768, 1), 5.4),
    31: (_pages_decode(1, 6, 131072, 1), 14.3),
    32: (_pages_decode(4, 2, 32768, 1), 10.2),
    33: (_pages_decode(4, 6, 131072, 1), 40.2),
    34: (_pages_decode(16, 2, 32768, 1), 29.2),
    35: (_pages_decode(16, 6, 32768, 1), 46.9),
    36: (_pages_decode(16, 6, 131072, 1), 212.7),
    37: (_pages_decode(64, 2, 131072, 1), 594.0),
    38: (_pages_decode(64, 6, 131072, 1), 982.8),
    39: (_pages_decode(1, 2, 32768, 64), 4.3),
    40: (_pages_decode(4, 6, 131072, 64), 27.6),
    41: (_pages_decode(16, 6, 32768, 64), 32.7),
    42: (_pages_decode(16, 6, 131072, 64), 141.2),
    43: (_pages_decode(64, 6, 8192, 64), 32.5),
    44: (_pages_decode(64, 6, 131072, 64), 551.7),
}
CONFIGS.update({i: w for i, (w, _) in PAGES_TABLE.items()})


def make_config(idx: int, poison: bool = False):
    """The named workloads, seed = 1000 + index."""
    c = CONFIGS[idx]
    seed = 1000 + idx
    if c["kind"] == "prefill":
        return make_prefill(c["M"], c["N"], seed, H=c.get("H", HEADS), D=c.get("D", HEAD_DIM))
    return make_decode(c["B"], c["next_n"], c["ctx"], c["mml"], seed,
                       ctx_range=c.get("ctx_range"), poison=poison,
                       block_size=c.get("block_size", KV_BLOCK), H=c.get("H", HEADS),
                       D=c.get("D", HEAD_DIM), preshuffle=c.get("preshuffle", False))


# Row families for the top-k over logits: shapes a logits row takes (a masked
# window, many equal values, the special values the selection must skip or
# rank) rather than values the op would produce; the benchmark feeds the top-k
# real decode logits instead.
TOPK_FAMILIES = ("normal", "small_ints", "constant", "masked_half", "specials", "narrow",
                 "mostly_equal", "two_values", "zeros_heavy", "zeros_half")


def topk_rows(cols: int, seed: int) -> np.ndarray:
    """float32 [len(TOPK_FAMILIES), cols], one row per family, seeded."""
    rng = np.random.Generator(np.random.PCG64(seed))
    out = np.empty((len(TOPK_FAMILIES), cols), dtype=np.float32)
    out[0] = rng.standard_normal(cols)
    out[1] = rng.integers(-3, 4, cols)
    out[2] = 1.5
    x = rng.standard_normal(cols).astype(np.float32)
    x[rng.random(cols) < 0.5] = -np.inf
    out[3] = x
    x = rng.standard_normal(cols).astype(np.float32)
    x[rng.random(cols) < 0.1] = np.nan
    x[rng.random(cols) < 0.1] = 0.0
    x[rng.random(cols) < 0.1] = -0.0
    x[rng.random(cols) < 0.01] = np.inf
    x[rng.random(cols) < 0.1] = -np.inf
    out[4] = x
    out[5] = rng.standard_normal(cols) * 1e-3 + 5
    out[6] = np.where(rng.random(cols) < 0.9, np.float32(2.0),
                      rng.standard_normal(cols).astype(np.float32))
    x = np.full(cols, np.nextafter(np.float32(1.0), np.float32(2.0)), dtype=np.float32)
    x[::3] = 1.0
    out[7] = x
    # exact zeros, as a token whose head scores are all negative produces:
    # the k-th entry falls among many equal values
    x = rng.standard_normal(cols).astype(np.float32)
    x[rng.random(cols) < 0.97] = 0.0
    out[8] = x
    x = -np.abs(rng.standard_normal(cols)).astype(np.float32)
    x[rng.random(cols) < 0.5] = 0.0
    x[rng.random(cols) < 0.005] = 1.0
    out[9] = x
    return out


@dataclasses.dataclass
class KcacheInsertInputs:
    k: np.ndarray             # [T, D] float32 (bf16-representable when bf16=True)
    slot_mapping: np.ndarray  # [T] int64, distinct slots, -1 = padding
    kv_cache: np.ndarray      # [num_blocks, block_size * (D + 4)] uint8, prior contents
    block_size: int
    bf16: bool


def make_kcache_insert(T: int, num_blocks: int, seed: int, block_size: int = KV_BLOCK,
                       D: int = HEAD_DIM, bf16: bool = False, padding: float = 0.1):
    """New K rows for the cache: N(0,1) rows with per-row magnitudes spread
    over 1e-3..1e3 (so scales span many binades), each mapped to a distinct
    random slot of a cache holding random prior bytes; a fraction `padding`
    of the tokens is padding (slot -1)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    k = rng.standard_normal((T, D)).astype(np.float32)
    k *= (10.0 ** rng.uniform(-3, 3, (T, 1))).astype(np.float32)
    if T:
        k[0] = 0.0  # an all-zero token: the scale floor
    if bf16:
        k = (torch.from_numpy(k).to(torch.bfloat16).to(torch.float32)).numpy()
    nslots = num_blocks * block_size
    if T > nslots:
        raise ValueError("more tokens than cache slots")
    slots = rng.permutation(nslots)[:T].astype(np.int64)
    slots[rng.random(T) < padding] = -1
    cache = rng.integers(0, 256, (num_blocks, block_size * (D + 4)), dtype=np.uint8)
    return KcacheInsertInputs(k, slots, cache, block_size, bf16)
