"""The named logits workloads at full size, in the launch configuration the
benchmark times (all tunables left to the host heuristic, clean_logits on).

Whole-output checks: the -inf mask equals the window predicate exactly at every
position, and no position is left unwritten (the output is NaN-poisoned before
the call).  Values: sampled rows -- whole rows, every column -- against the
oracle, including the first and last rows and, for ragged decode, the shortest
and longest sequences.
"""

from __future__ import annotations

import time

import numpy as np
import pytest
import torch

from sparse_attention_indexer_scaled_amd import inputs
from tests.gpu_util import (assert_parity, lib, oracle_decode, oracle_prefill, run_decode,
                            run_prefill, say)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    lib()


def _prefill_window(p):
    cols = np.arange(p.N, dtype=np.int64)[None, :]
    lo = np.maximum(p.ks.astype(np.int64), 0)[:, None]
    hi = np.minimum(p.ke.astype(np.int64), p.N)[:, None]
    return (cols >= lo) & (cols < hi)


def _decode_window(d):
    p = np.arange(d.max_model_len, dtype=np.int64)[None, :]
    b = np.repeat(np.arange(d.B), d.next_n)
    j = np.tile(np.arange(d.next_n), d.B)
    bound = d.context_lens.astype(np.int64)[b] - d.next_n + j
    return p <= bound[:, None]


@pytest.mark.parametrize("idx", [0, 3, 13, 25, 15])
def test_prefill_workload(idx):
    t0 = time.time()
    p = inputs.make_config(idx)
    say("workload %d %s: inputs %.1fs" % (idx, inputs.CONFIGS[idx]["name"], time.time() - t0))
    out = run_prefill(p)
    win = _prefill_window(p)
    assert not np.isnan(out).any(), "unwritten output positions"
    assert np.array_equal(np.isneginf(out), ~win)
    assert np.isfinite(out[win]).all()
    # every row of the small chunk; on the long chunks every 16th row plus the
    # first and last rows (the shortest and longest windows)
    rows = np.arange(p.M) if p.M <= 64 else np.unique(np.concatenate(
        [np.arange(0, p.M, 16), [1, 2, 3, 1000, 2047, 3001, p.M - 4, p.M - 3, p.M - 2, p.M - 1]]))
    t0 = time.time()
    ref, mag = oracle_prefill(p, rows)
    say("oracle rows %s: %.1fs" % (len(rows), time.time() - t0))
    assert_parity(out[rows], ref, mag, f"workload{idx}")


@pytest.mark.parametrize("idx", [1, 2, 4, 9, 10, 11, 12, 14, 18, 19, 20, 21, 22, 36, 42])
def test_decode_workload(idx):
    t0 = time.time()
    d = inputs.make_config(idx, poison=True)
    say("workload %d %s: inputs %.1fs, ctx %d..%d" % (idx, inputs.CONFIGS[idx]["name"], time.time() - t0,
                                                       d.context_lens.min(), d.context_lens.max()))
    out = run_decode(d)
    win = _decode_window(d)
    assert not np.isnan(out).any(), "unwritten output positions"
    assert np.array_equal(np.isneginf(out), ~win)
    assert np.isfinite(out[win]).all()
    if idx == 4:
        seqs = [int(np.argmin(d.context_lens)), int(np.argmax(d.context_lens)), 17]
    elif inputs.CONFIGS[idx]["ctx"] is None:  # ragged lengths: the shortest, the longest, one more
        seqs = sorted({int(np.argmin(d.context_lens)), int(np.argmax(d.context_lens)), d.B // 2 + 1})
    elif idx == 2:
        seqs = list(range(d.B))  # the headline: every row
    else:
        seqs = [0, 15]
    t0 = time.time()
    ref, mag, rows = oracle_decode(d, seqs)
    say("oracle seqs %s: %.1fs" % (seqs, time.time() - t0))
    assert_parity(out[rows], ref, mag, f"workload{idx}")
