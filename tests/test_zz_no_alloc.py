"""The allocation-free fused top-k (paged_mqa_topk_decode_noalloc) against
paged_mqa_topk_decode with a caller-owned workspace.

Two calls in a row through the C ABI, the second with a smaller input, so the
second runs on scratch the first left full of its own entries: the indices of
both must equal the workspace call's bit for bit (the fused call's output is
unique).  The size limit is checked before any device work, so its test runs
without a GPU.
"""

from __future__ import annotations

import ctypes
import os
import re

import numpy as np
import pytest
import torch

from sparse_attention_indexer_scaled_amd import _native, inputs
from tests.util import ROOT


def _lib():
    if not os.path.exists(_native.LIB_PATH):
        from sparse_attention_indexer_scaled_amd import build
        build.build()
    return _native.load_library()


def _say(msg):
    print(msg, flush=True)


def test_header_states_the_scratch_size():
    text = open(os.path.join(ROOT, "include", "mqa_indexer.h")).read()
    m = re.search(r"#define MQA_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == _native.NOALLOC_SCRATCH_BYTES


def test_problem_larger_than_the_scratch_is_rejected():
    """512 rows of 131072 positions need about 537 MB of workspace: rejected
    with a message naming the limit, before any pointer is looked at."""
    lib = _lib()
    assert lib.paged_mqa_topk_workspace_size(64, 8, 131072) > _native.NOALLOC_SCRATCH_BYTES
    rc = lib.paged_mqa_topk_decode_noalloc(None, None, None, None, None, None, 64, 8, 32, 128,
                                           64, 0, 1, 2048, 131072, 2048, None, None)
    assert rc == _native.MQA_ERR_INVALID_ARG
    assert "static scratch" in _native.last_error()


def _dv(d):
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    return dict(q=dev(d.q), cache=dev(d.kv_cache), w=dev(d.weights), ctx=dev(d.context_lens),
                bt=dev(d.block_tables))


def _with_workspace(d, dv, k):
    need = _native.paged_mqa_topk_workspace_size(d.B, d.next_n, d.max_model_len)
    ws = torch.full((need,), 0xA5, dtype=torch.uint8, device="cuda")
    out = torch.full((d.B * d.next_n, k), -7, dtype=torch.int32, device="cuda")
    _native.paged_mqa_topk_decode(dv["q"], dv["cache"], dv["w"], dv["ctx"], dv["bt"],
                                  d.max_model_len, k, kv_block_size=d.block_size, indices=out,
                                  workspace=ws, preshuffle=d.preshuffle)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def _noalloc(d, dv, k):
    out = torch.full((d.B * d.next_n, k), -7, dtype=torch.int32, device="cuda")
    _native.paged_mqa_topk_decode_noalloc(dv["q"], dv["cache"], dv["w"], dv["ctx"], dv["bt"],
                                          d.max_model_len, k, out, kv_block_size=d.block_size,
                                          preshuffle=d.preshuffle)
    torch.cuda.synchronize()
    return out.cpu().numpy()


@pytest.mark.gpu
def test_two_calls_in_a_row_match_the_workspace_call():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    _lib()
    cases = [
        # the benchmark's shape: 96 rows of 131072 positions, k = 2048
        (inputs.make_config(2), 2048),
        # then a smaller, ragged one (an empty-ish sequence, a short one, a
        # sequence past the keep-all size) with padding poisoned
        (inputs.make_decode(3, 2, [30000, 7, 12345], 30016, seed=931, poison=True), 512),
    ]
    for i, (d, k) in enumerate(cases):
        _say("noalloc call %d: B=%d next_n=%d max_model_len=%d k=%d"
             % (i, d.B, d.next_n, d.max_model_len, k))
        dv = _dv(d)
        want = _with_workspace(d, dv, k)
        got = _noalloc(d, dv, k)
        assert np.array_equal(got, want), "call %d: %d rows differ" % (
            i, int((got != want).any(axis=1).sum()))
