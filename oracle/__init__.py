"""CPU oracle for the lightning-indexer logits -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, the package smoke check and the benchmark's ``cpu_baseline``
leg may import this package.  The product path (the HIP library and its Python
binding) never imports, links or calls anything here, and it never falls back
to it.

Python side of ``oracle/mqa_oracle.c`` (plain fp64 C, OpenMP over rows).  See
that file for the definition, the window rules and the exactness argument.
Inputs are numpy arrays in the op's own layouts; outputs are float64.

The row-wise top-k that consumes the logits is in ``oracle.topk`` and the
K-cache quantise-and-insert step that precedes decode in ``oracle.kcache``
(both numpy).

Every function here is pinned by the ``-m "not gpu"`` tests against things
other than itself: an exact rational brute force (``oracle.brute``), numpy
matmul closed forms, the fp8 table of torch's own e4m3fn conversion, and the
pages' invariants (hoist, paged == contiguous, exact windows, zero weights).
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mqa_oracle.c")
_LIB = os.path.join(_HERE, "liboracle_mqa.so")
_lib = None


def build(force: bool = False) -> str:
    """Compile ``liboracle_mqa.so`` with gcc (plain -O2, no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared",
                               "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        i32, i64 = ctypes.c_int, ctypes.c_int64
        lib.oracle_e4m3fn_value.restype = ctypes.c_double
        lib.oracle_e4m3fn_value.argtypes = [ctypes.c_uint8]
        lib.oracle_e4m3fn_table.argtypes = [P]
        lib.oracle_num_threads.restype = i32
        lib.oracle_set_num_threads.argtypes = [i32]
        lib.oracle_prefill.argtypes = [P, P, P, P, P, P, i64, i64, i32, i32, i32, i32, P]
        lib.oracle_decode.restype = i32
        lib.oracle_decode.argtypes = [P, P, P, P, P, i32, i32, i32, i32, i32, i32, i64, i32,
                                      i64, i32, i32, P]
        _lib = lib
    return _lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def e4m3fn_table() -> np.ndarray:
    out = np.empty(256, dtype=np.float64)
    _load().oracle_e4m3fn_table(_ptr(out))
    return out


def num_threads() -> int:
    return _load().oracle_num_threads()


def set_num_threads(n: int) -> None:
    _load().oracle_set_num_threads(int(n))


def prefill(q, k, kv_scale, weights, ks, ke, clean=True, hoist=False, out=None) -> np.ndarray:
    """Oracle prefill logits (float64 [M, N]).

    q uint8 [M,H,D], k uint8 [N,D], kv_scale f32 [N], weights f32 [M,H],
    ks/ke int32 [M].  With ``clean=False`` columns outside the window keep the
    values of ``out`` (which must then be given).
    """
    q = _c(q, np.uint8)
    k = _c(k, np.uint8)
    M, H, D = q.shape
    N = k.shape[0]
    assert k.shape == (N, D)
    kv_scale = _c(kv_scale, np.float32)
    weights = _c(weights, np.float32)
    ks = _c(ks, np.int32)
    ke = _c(ke, np.int32)
    assert kv_scale.shape == (N,) and weights.shape == (M, H)
    assert ks.shape == (M,) and ke.shape == (M,)
    if out is None:
        if not clean:
            raise ValueError("clean=False needs a pre-filled out array")
        out = np.empty((M, N), dtype=np.float64)
    assert out.dtype == np.float64 and out.shape == (M, N) and out.flags.c_contiguous
    _load().oracle_prefill(_ptr(q), _ptr(k), _ptr(kv_scale), _ptr(weights), _ptr(ks), _ptr(ke),
                           M, N, H, D, int(bool(clean)), int(bool(hoist)), _ptr(out))
    return out


def decode(q, kv_cache, weights, context_lens, block_tables, max_model_len, block_size,
           clean=True, hoist=False, out=None, preshuffle=False) -> np.ndarray:
    """Oracle paged-decode logits (float64 [B*next_n, max_model_len]).

    q uint8 [B,next_n,H,D], kv_cache uint8 [num_blocks, block_size*(D+4)],
    weights f32 [B*next_n,H], context_lens int32 [B], block_tables int32
    [B, max_blocks_per_seq].  preshuffle: the K rows of each block are in the
    16 x 16-byte tiled order (see ``oracle_decode``) instead of slot-major.
    """
    q = _c(q, np.uint8)
    B, next_n, H, D = q.shape
    kv_cache = _c(kv_cache, np.uint8)
    num_blocks = kv_cache.shape[0]
    assert kv_cache.shape == (num_blocks, block_size * (D + 4))
    weights = _c(weights, np.float32)
    assert weights.shape == (B * next_n, H)
    ctx = _c(context_lens, np.int32)
    bt = _c(block_tables, np.int32)
    assert ctx.shape == (B,) and bt.shape[0] == B
    mbps = bt.shape[1]
    if out is None:
        if not clean:
            raise ValueError("clean=False needs a pre-filled out array")
        out = np.empty((B * next_n, max_model_len), dtype=np.float64)
    assert out.dtype == np.float64 and out.shape == (B * next_n, max_model_len)
    rc = _load().oracle_decode(_ptr(q), _ptr(kv_cache), _ptr(weights), _ptr(ctx), _ptr(bt), B,
                               next_n, H, D, block_size, int(bool(preshuffle)), num_blocks, mbps,
                               max_model_len, int(bool(clean)), int(bool(hoist)), _ptr(out))
    if rc == -2:
        raise ValueError("the tiled layout needs block_size and head_dim multiples of 16")
    if rc != 0:
        raise ValueError("block table entry out of range for a position inside a window")
    return out
