"""CPU oracle for the K-cache quantise-and-insert step -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, the package smoke check and the benchmark's ``cpu_baseline``
leg may import this module; the product path never does.

The step before decode on the pages: new K rows are stored as fp8 e4m3fn next
to a per-token fp32 dequant scale in the paged cache (aiter PR 5047 page,
"Motivation"), with the scale taken as the row's absolute maximum over 448
(the largest e4m3fn value).  Written out:

  amax    = max_d |k[t, d]|                       (fp32, exact)
  scale   = fp32( max(amax, 1e-12) / 448 )        (one correctly rounded division)
  q[t, d] = e4m3fn_rne( clamp( fp32(k[t, d] / scale), -448, 448 ) )

and the token's 128 code bytes and 4 scale bytes go to its slot of the
block-split cache layout (block i = bs*(D+4) bytes: the bs K rows, slot-major,
then the bs fp32 scales).  Tokens whose slot is negative are padding and write
nothing; so do tokens whose slot lies at or past the cache's last slot
(num_blocks * bs).  The pages name no out-of-range rule: the reading taken is
that such a token has no slot to go to and is dropped, like padding, rather
than written past the cache.  e4m3fn_rne picks the representable value nearest to its argument,
ties to the code with the even mantissa, keeping the sign (a negative value
that rounds to zero gives -0, code 0x80); the representable values come from
the format definition (``oracle.e4m3fn_table``, the C decoder).
"""

from __future__ import annotations

import numpy as np

FP8_MAX = 448.0


def _finite_codes():
    """Non-negative finite e4m3fn codes 0x00..0x7E and their values, ascending."""
    import oracle
    table = oracle.e4m3fn_table()
    codes = np.arange(0x7F, dtype=np.int64)
    vals = table[codes]
    assert np.all(np.diff(vals) > 0)
    return codes, vals


def e4m3fn_rne(v: np.ndarray) -> np.ndarray:
    """fp32 values already inside [-448, 448] -> uint8 e4m3fn codes, round to
    nearest, ties to even (the code whose mantissa bit 0 is clear)."""
    v = np.asarray(v, dtype=np.float32)
    if np.any(np.abs(v) > FP8_MAX) or np.any(np.isnan(v)):
        raise ValueError("e4m3fn_rne expects values within [-448, 448]")
    codes, vals = _finite_codes()
    a = np.abs(v.astype(np.float64)).ravel()
    hi = np.searchsorted(vals, a, side="left")          # first value >= a
    hi = np.minimum(hi, codes.size - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - vals[lo]
    d_hi = vals[hi] - a
    pick = np.where(d_lo < d_hi, lo, hi)
    tie = (d_lo == d_hi) & (lo != hi)
    pick = np.where(tie, np.where(codes[lo] % 2 == 0, lo, hi), pick)
    out = codes[pick].astype(np.uint8)
    # the sign bit is kept, so negative values that round to zero give -0 (0x80)
    out = np.where(np.signbit(v.ravel()), out | 0x80, out).astype(np.uint8)
    return out.reshape(v.shape)


def quantize_tokens(k: np.ndarray):
    """k [T, D] (fp32 values) -> (codes uint8 [T, D], scale float32 [T])."""
    k = np.asarray(k, dtype=np.float32)
    amax = np.abs(k).max(axis=-1)
    scale = (np.maximum(amax, np.float32(1e-12)) / np.float32(FP8_MAX)).astype(np.float32)
    q = (k / scale[:, None]).astype(np.float32)
    q = np.clip(q, np.float32(-FP8_MAX), np.float32(FP8_MAX))
    return e4m3fn_rne(q), scale


def insert(kv_cache: np.ndarray, k: np.ndarray, slot_mapping: np.ndarray, block_size: int,
           preshuffle: bool = False):
    """Return a copy of kv_cache [num_blocks, bs*(D+4)] bytes with the tokens
    of k [T, D] quantised into their slots (slot < 0 or slot >=
    num_blocks * block_size: token skipped).

    preshuffle: the K rows of a block are in 16 x 16-byte tiles (the decode
    oracle's layout 1): byte d of slot s at (s/16)*16*D + (d/16)*256 +
    (s%16)*16 + d%16; otherwise slot-major, byte d of slot s at s*D + d."""
    cache = np.array(kv_cache, dtype=np.uint8, copy=True)
    T, D = k.shape
    codes, scale = quantize_tokens(k)
    flat = cache.reshape(cache.shape[0], -1)
    num_slots = cache.shape[0] * block_size
    for t in range(T):
        s = int(slot_mapping[t])
        if s < 0 or s >= num_slots:
            continue
        blk, slot = divmod(s, block_size)
        if preshuffle:
            for d in range(D):
                flat[blk, (slot // 16) * 16 * D + (d // 16) * 256 + (slot % 16) * 16 + d % 16] = \
                    codes[t, d]
        else:
            flat[blk, slot * D:(slot + 1) * D] = codes[t]
        off = block_size * D + 4 * slot
        flat[blk, off:off + 4] = np.frombuffer(np.float32(scale[t]).tobytes(), dtype=np.uint8)
    return cache
