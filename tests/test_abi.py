"""The C-ABI library without a GPU: it loads, exports every symbol the header
declares, and rejects bad arguments before touching the device.

Every call here fails validation before any HIP call that could launch work,
so these tests are safe on any machine, GPU or not.  No call passes a pointer
that would pass validation.
"""

from __future__ import annotations

import ctypes
import os
import re

import pytest

import sparse_attention_indexer_scaled_amd as mqa
from sparse_attention_indexer_scaled_amd import _native
from tests.util import ROOT

HEADER = os.path.join(ROOT, "include", "mqa_indexer.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_native.LIB_PATH):
        from sparse_attention_indexer_scaled_amd import build
        build.build()
    return _native.load_library()


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b([a-z_][a-z0-9_]*)\s*\(", text)) - {"defined"})


def test_header_declares_the_boundary():
    assert _declared_functions() == sorted(_native.EXPORTED)


def test_library_exports_every_declared_symbol(lib):
    for name in _declared_functions():
        assert hasattr(lib, name), name
    # and the exports are plain C symbols (no C++ mangling)
    out = os.popen("nm -D --defined-only %s" % _native.LIB_PATH).read()
    for name in _declared_functions():
        assert re.search(r"\bT %s$" % name, out, flags=re.M), name


def test_tunables_struct_matches_header():
    text = open(HEADER).read()
    body = re.search(r"typedef struct mqa_tunables \{(.*?)\} mqa_tunables;", text, flags=re.S).group(1)
    fields = re.findall(r"int\s+(\w+);", body)
    assert fields == [f for f, _ in _native.Tunables._fields_]
    assert ctypes.sizeof(_native.Tunables) == 4 * len(fields)


def test_error_codes_match_header():
    text = open(HEADER).read()
    for name in ("MQA_OK", "MQA_ERR_INVALID_ARG", "MQA_ERR_UNSUPPORTED", "MQA_ERR_LAUNCH",
                 "MQA_ERR_DEVICE", "MQA_DTYPE_FP32", "MQA_DTYPE_BF16", "MQA_KV_SLOT_MAJOR",
                 "MQA_KV_PRESHUFFLED"):
        m = re.search(r"#define %s \(?(-?\d+)\)?" % name, text)
        assert int(m.group(1)) == getattr(_native, name), name


# Shapes the header lists as supported, and shapes it does not.  On gfx950 the
# gate answers 1 and 0 for them (tests/test_gpu_gate.py); without one it
# answers 0 for every shape.
GATE_SUPPORTED = [(h, d, bs) for h in (32, 64, 128) for d in (64, 128) for bs in (0, 1, 16, 64, 128)]
GATE_UNSUPPORTED = [(48, 128, 0), (32, 96, 0), (32, 128, 32), (32, 128, 2), (256, 128, 64),
                    (16, 128, 64), (0, 128, 0), (32, 0, 0), (32, 128, -1), (32, 256, 64),
                    (96, 128, 64), (32, 128, 256)]


def test_gate_answers_zero_without_gfx950(lib):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a HIP device is present; tests/test_gpu_gate.py checks the gate there")
    for h, d, bs in GATE_SUPPORTED + GATE_UNSUPPORTED:
        assert lib.mqa_is_supported(h, d, bs) == 0, (h, d, bs)


P = ctypes.c_void_p


def _prefill(lib, ptrs, M=4, N=8, H=32, D=128, clean=1, tun=None):
    return lib.mqa_logits_prefill(*ptrs, M, N, H, D, clean, tun, None)


def _decode(lib, ptrs, B=2, nn=1, H=32, D=128, bs=64, nb=4, mbps=2, mml=128, tun=None, layout=0):
    return lib.paged_mqa_logits_decode(*ptrs, B, nn, H, D, bs, layout, nb, mbps, mml, 1, tun, None)


def test_prefill_validation(lib):
    nulls = [None] * 7
    assert _prefill(lib, nulls, M=-1) == mqa._native.MQA_ERR_INVALID_ARG
    assert _prefill(lib, nulls, N=-5) == mqa._native.MQA_ERR_INVALID_ARG
    assert _prefill(lib, nulls, H=48) == mqa._native.MQA_ERR_UNSUPPORTED
    assert _prefill(lib, nulls, H=64) == mqa._native.MQA_ERR_INVALID_ARG  # supported; NULLs
    bad = _native.Tunables(block_m=8)  # 64 heads: at most 4 rows per wave
    assert _prefill(lib, nulls, H=64, tun=ctypes.byref(bad)) == mqa._native.MQA_ERR_INVALID_ARG
    assert _prefill(lib, nulls, D=96) == mqa._native.MQA_ERR_UNSUPPORTED
    assert "num_heads" in mqa.last_error()
    for h in (32, 64, 128):
        assert _prefill(lib, nulls, H=h, D=64) == mqa._native.MQA_ERR_INVALID_ARG  # NULLs
    # empty problem: successful no-op, nothing dereferenced
    assert _prefill(lib, nulls, M=0) == 0
    assert _prefill(lib, nulls, N=0) == 0
    assert mqa.last_error() == ""
    assert _prefill(lib, nulls) == mqa._native.MQA_ERR_INVALID_ARG
    assert "NULL" in mqa.last_error()
    # misaligned (never dereferenced: rejected before the device is touched)
    odd = [P(0x1001)] * 7
    assert _prefill(lib, odd) == mqa._native.MQA_ERR_INVALID_ARG
    assert "aligned" in mqa.last_error()
    bad = _native.Tunables(block_m=3)
    assert _prefill(lib, nulls, tun=ctypes.byref(bad)) == mqa._native.MQA_ERR_INVALID_ARG
    bad = _native.Tunables(reverse_rows=2)
    assert _prefill(lib, nulls, tun=ctypes.byref(bad)) == mqa._native.MQA_ERR_INVALID_ARG
    bad = _native.Tunables(num_warps=9)
    assert _prefill(lib, nulls, tun=ctypes.byref(bad)) == mqa._native.MQA_ERR_INVALID_ARG
    # the shared-K ring (1 = per-wave K): head dim 128, num_warps 4; 32 heads
    # with depth 2..7 and block_m 4, 64 (128) heads with depth 3 or 4 and
    # block_m 2 (1)
    for depth in (-1, 8):
        bad = _native.Tunables(ring_depth=depth)
        assert _prefill(lib, nulls, tun=ctypes.byref(bad)) == mqa._native.MQA_ERR_INVALID_ARG
        assert "ring_depth" in mqa.last_error()
    for kw, shape in ((dict(ring_depth=5), dict(H=128)), (dict(ring_depth=4, block_m=2), dict(H=128)),
                      (dict(ring_depth=4), dict(D=64)),
                      (dict(ring_depth=5), dict(H=64)), (dict(ring_depth=4, block_m=4), dict(H=64)),
                      (dict(ring_depth=2, block_m=2), {}),
                      (dict(ring_depth=7, num_warps=1), {})):
        bad = _native.Tunables(**kw)
        assert _prefill(lib, nulls, tun=ctypes.byref(bad), **shape) == \
            mqa._native.MQA_ERR_INVALID_ARG
        assert "shared-K" in mqa.last_error()
    for kw, shape in ((dict(ring_depth=1), {}), (dict(ring_depth=2), {}),
                      (dict(ring_depth=7, block_m=4, num_warps=4), {}),
                      (dict(ring_depth=3, block_m=2), dict(H=64)), (dict(ring_depth=4), dict(H=64)),
                      (dict(ring_depth=4), dict(H=128)), (dict(ring_depth=3, block_m=1), dict(H=128))):
        ok = _native.Tunables(**kw)  # valid: fails only on the NULL pointers
        assert _prefill(lib, nulls, tun=ctypes.byref(ok), **shape) == \
            mqa._native.MQA_ERR_INVALID_ARG
        assert "NULL" in mqa.last_error()


def test_decode_validation(lib):
    nulls = [None] * 6
    assert _decode(lib, nulls, B=-1) == mqa._native.MQA_ERR_INVALID_ARG
    assert _decode(lib, nulls, nn=0) == mqa._native.MQA_ERR_INVALID_ARG
    assert _decode(lib, nulls, nn=9) == mqa._native.MQA_ERR_INVALID_ARG
    assert _decode(lib, nulls, bs=32) == mqa._native.MQA_ERR_UNSUPPORTED
    assert _decode(lib, nulls, bs=16) == mqa._native.MQA_ERR_INVALID_ARG  # supported; NULLs
    assert _decode(lib, nulls, bs=0) == mqa._native.MQA_ERR_UNSUPPORTED
    assert _decode(lib, nulls, H=48) == mqa._native.MQA_ERR_UNSUPPORTED
    assert _decode(lib, nulls, D=96) == mqa._native.MQA_ERR_UNSUPPORTED
    for bs in (1, 16, 64, 128):  # head dim 64: every block size
        assert _decode(lib, nulls, D=64, bs=bs) == mqa._native.MQA_ERR_INVALID_ARG  # NULLs
        assert "NULL" in mqa.last_error()
    bad = _native.Tunables(ring_depth=4)  # head dim 64: ring depth 0 or 3
    assert _decode(lib, nulls, D=64, tun=ctypes.byref(bad)) == mqa._native.MQA_ERR_INVALID_ARG
    assert "ring_depth" in mqa.last_error()
    for H in (64, 128):
        for bs in (1, 16, 128):
            assert _decode(lib, nulls, H=H, bs=bs) == mqa._native.MQA_ERR_INVALID_ARG  # NULLs
    bad = _native.Tunables(rows_per_block=2)  # 128 heads: one row per wave
    assert _decode(lib, nulls, H=128, tun=ctypes.byref(bad)) == mqa._native.MQA_ERR_INVALID_ARG
    assert _decode(lib, nulls, layout=2) == mqa._native.MQA_ERR_INVALID_ARG
    assert "kv_layout" in mqa.last_error()
    assert _decode(lib, nulls, bs=1, layout=1) == mqa._native.MQA_ERR_UNSUPPORTED
    for bs in (16, 64, 128):
        assert _decode(lib, nulls, bs=bs, layout=1) == mqa._native.MQA_ERR_INVALID_ARG  # NULLs
        assert "NULL" in mqa.last_error()
    assert _decode(lib, nulls, B=0) == 0
    assert _decode(lib, nulls, mml=0) == 0
    assert _decode(lib, nulls) == mqa._native.MQA_ERR_INVALID_ARG
    odd = [P(0x2002)] * 6
    assert _decode(lib, odd) == mqa._native.MQA_ERR_INVALID_ARG
    bad = _native.Tunables(ring_depth=4)  # other depths only with 64-token blocks
    assert _decode(lib, nulls, bs=16, tun=ctypes.byref(bad)) == mqa._native.MQA_ERR_INVALID_ARG
    assert "ring_depth" in mqa.last_error()
    bad = _native.Tunables(ring_depth=3)  # per-token blocks: 0 or 4
    assert _decode(lib, nulls, bs=1, tun=ctypes.byref(bad)) == mqa._native.MQA_ERR_INVALID_ARG
    assert "ring_depth" in mqa.last_error()
    for bad in (_native.Tunables(rows_per_block=5), _native.Tunables(ring_depth=1),
                _native.Tunables(ring_depth=8), _native.Tunables(num_warps=2),
                _native.Tunables(split_kv=-1)):
        assert _decode(lib, nulls, tun=ctypes.byref(bad)) == mqa._native.MQA_ERR_INVALID_ARG


def test_topk_validation(lib):
    f = lib.mqa_topk_indices
    assert f(None, -1, 8, 4, None, None) == mqa._native.MQA_ERR_INVALID_ARG
    assert f(None, 2, -8, 4, None, None) == mqa._native.MQA_ERR_INVALID_ARG
    assert f(None, 2, 8, 0, None, None) == mqa._native.MQA_ERR_INVALID_ARG
    assert f(None, 2, 8, 2049, None, None) == mqa._native.MQA_ERR_INVALID_ARG
    assert "k must be" in mqa.last_error()
    assert f(None, 0, 8, 4, None, None) == 0
    assert f(None, 2, 8, 4, None, None) == mqa._native.MQA_ERR_INVALID_ARG
    assert f(P(0x1002), 2, 8, 4, P(0x2000), None) == mqa._native.MQA_ERR_INVALID_ARG
    assert "aligned" in mqa.last_error()


def test_fused_topk_workspace_size(lib):
    ws = lib.paged_mqa_topk_workspace_size
    big = ws(16, 6, 131072)
    assert 96 * 131072 * 8 <= big <= 96 * 131072 * 8 + 96 * 1024 * 4 + 96 * 4096 * 4 + 96 * 8 + 5 * 256
    assert ws(0, 6, 131072) == 0 and ws(16, 0, 131072) == 0 and ws(16, 9, 131072) == 0
    assert ws(16, 6, 0) == 0
    assert ws(1, 1, 1) > 0
    assert mqa.paged_mqa_topk_workspace_size(16, 6, 131072) == big


def test_topk_workspace_size_and_validation(lib):
    ws = lib.mqa_topk_workspace_size
    assert ws(0, 10) == 0 and ws(10, 0) == 0 and ws(-1, 10) == 0
    big = ws(96, 131072)
    assert 96 * 131072 * 8 <= big <= 96 * 131072 * 8 + 96 * 64 * 4 + 2 * 256
    assert mqa.topk_workspace_size(96, 131072) == big
    E = mqa._native
    f = lib.mqa_topk_indices_ws
    assert f(None, 4, 100, 0, None, None, 0, None) == E.MQA_ERR_INVALID_ARG  # k, NULL workspace
    assert f(None, 0, 100, 5, None, ctypes.c_void_p(256), 0, None) == E.MQA_OK  # no rows
    assert f(None, 4, 100, 5, None, ctypes.c_void_p(1000), 1 << 20, None) == E.MQA_ERR_INVALID_ARG
    assert "256-byte" in mqa.last_error()
    assert f(None, 4, 100, 5, None, ctypes.c_void_p(4096), 16, None) == E.MQA_ERR_INVALID_ARG
    assert "smaller than" in mqa.last_error()


def _fused(lib, ptrs, B=2, nn=1, H=32, D=128, bs=64, nb=4, mbps=2, mml=128, k=16, ws=None,
           wsb=0, tun=None, layout=0):
    return lib.paged_mqa_topk_decode(*ptrs, B, nn, H, D, bs, layout, nb, mbps, mml, k, ws, wsb,
                                     tun, None)


def test_fused_topk_validation(lib):
    nulls = [None] * 6
    E = mqa._native
    assert _fused(lib, nulls, k=0) == E.MQA_ERR_INVALID_ARG
    assert "k must be" in mqa.last_error()
    assert _fused(lib, nulls, k=2049) == E.MQA_ERR_INVALID_ARG
    # the shapes the decode takes, checked before any pointer
    assert _fused(lib, nulls, H=48) == E.MQA_ERR_UNSUPPORTED
    assert _fused(lib, nulls, bs=32) == E.MQA_ERR_UNSUPPORTED
    assert _fused(lib, nulls, D=96) == E.MQA_ERR_UNSUPPORTED
    assert _fused(lib, nulls, D=64, bs=1) == E.MQA_ERR_INVALID_ARG  # head dim 64: NULLs
    assert _fused(lib, nulls, D=64) == E.MQA_ERR_INVALID_ARG
    assert _fused(lib, nulls, D=64, tun=ctypes.byref(E.Tunables(ring_depth=4))) == \
        E.MQA_ERR_INVALID_ARG
    assert "ring depth" in mqa.last_error()
    for H, bs in ((64, 64), (128, 64), (32, 16), (32, 1), (32, 128), (64, 16), (128, 1)):
        assert _fused(lib, nulls, H=H, bs=bs) == E.MQA_ERR_INVALID_ARG
        assert "NULL" in mqa.last_error()
    # the ring depth is the logits call's default: 4 for per-token blocks, else 3
    assert _fused(lib, nulls, tun=ctypes.byref(E.Tunables(ring_depth=4))) == E.MQA_ERR_INVALID_ARG
    assert "ring depth" in mqa.last_error()
    assert _fused(lib, nulls, bs=1, tun=ctypes.byref(E.Tunables(ring_depth=3))) == \
        E.MQA_ERR_INVALID_ARG
    assert "ring depth" in mqa.last_error()
    assert _fused(lib, nulls, bs=16, tun=ctypes.byref(E.Tunables(ring_depth=3))) == \
        E.MQA_ERR_INVALID_ARG
    assert "NULL" in mqa.last_error()
    assert _fused(lib, nulls, B=0) == 0          # nothing to do, nothing dereferenced
    assert _fused(lib, nulls, mml=0) == 0
    assert _fused(lib, nulls) == E.MQA_ERR_INVALID_ARG
    assert "NULL" in mqa.last_error()
    # batch x next_n past INT32_MAX: a clear error, not a wrapped row count
    assert _fused(lib, nulls, B=2**30, nn=2) == E.MQA_ERR_INVALID_ARG
    assert "INT32_MAX" in mqa.last_error()
    need = lib.paged_mqa_topk_workspace_size(2, 1, 128)
    fake = [P(0x10000)] * 6  # never dereferenced: rejected before the device is touched
    assert _fused(lib, fake, ws=P(0x20080), wsb=need) == E.MQA_ERR_INVALID_ARG
    assert "aligned" in mqa.last_error()
    assert _fused(lib, fake, ws=P(0x20000), wsb=need - 1) == E.MQA_ERR_INVALID_ARG
    assert "workspace" in mqa.last_error()


def test_kcache_validation(lib):
    f = lib.mqa_kcache_quantize_insert
    assert f(None, 0, None, None, -1, 128, 64, 0, 4, None) == mqa._native.MQA_ERR_INVALID_ARG
    assert f(None, 2, None, None, 5, 128, 64, 0, 4, None) == mqa._native.MQA_ERR_INVALID_ARG
    assert "k_dtype" in mqa.last_error()
    assert f(None, 0, None, None, 5, 96, 64, 0, 4, None) == mqa._native.MQA_ERR_UNSUPPORTED
    assert f(None, 0, None, None, 5, 64, 1, 0, 4, None) == mqa._native.MQA_ERR_INVALID_ARG  # NULLs
    assert f(None, 0, None, None, 5, 64, 1, 1, 4, None) == mqa._native.MQA_ERR_UNSUPPORTED
    assert f(None, 0, None, None, 5, 64, 64, 0, 4, None) == mqa._native.MQA_ERR_INVALID_ARG  # NULLs
    assert f(None, 1, None, None, 5, 128, 32, 0, 4, None) == mqa._native.MQA_ERR_UNSUPPORTED
    assert f(None, 0, None, None, 5, 128, 64, 3, 4, None) == mqa._native.MQA_ERR_INVALID_ARG
    assert "kv_layout" in mqa.last_error()
    assert f(None, 0, None, None, 5, 128, 1, 1, 4, None) == mqa._native.MQA_ERR_UNSUPPORTED
    assert f(None, 0, None, None, 0, 128, 64, 0, 4, None) == 0
    assert f(None, 0, None, None, 5, 128, 64, 0, 4, None) == mqa._native.MQA_ERR_INVALID_ARG
    assert f(None, 0, None, None, 5, 128, 64, 1, 4, None) == mqa._native.MQA_ERR_INVALID_ARG
    assert f(P(0x1004), 0, P(0x2000), P(0x3000), 5, 128, 64, 0, 4, None) == \
        mqa._native.MQA_ERR_INVALID_ARG
    assert "aligned" in mqa.last_error()


def test_binding_raises_on_missing_library(tmp_path):
    saved = _native._lib
    _native._lib = None
    try:
        with pytest.raises(mqa.MQAError):
            _native.load_library(str(tmp_path / "nope.so"))
    finally:
        _native._lib = saved
