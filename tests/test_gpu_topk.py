"""GPU parity of the row-wise top-k (mqa_topk_indices, and mqa_topk_indices_ws,
which splits long rows over several workgroups) with the oracle.

Both sides select on the same fp32 logits, so every comparison is taken in
fp32 on both and the outputs (column indices) must match bit for bit.

Cases: every row family of inputs.topk_rows (normal, ties, a constant row, a
masked window, NaN / +-0 / +-inf, a narrow range, mostly-equal, two adjacent
floats) at widths from 1 to 131072 and k from 1 to 2048, so that each radix
depth and the ordered-tie path run; logits produced by the decode kernel
itself; and the edges (k > cols, cols == 0, one column).
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

from oracle.topk import topk_indices as oracle_topk
from sparse_attention_indexer_scaled_amd import _native, inputs
from tests.gpu_util import dev, lib, run_decode, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    lib()


def gpu_topk(x, k):
    t = dev(x)
    out = torch.full((x.shape[0], k), -7, dtype=torch.int32, device="cuda")
    _native.topk_indices(t, k, indices=out)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def gpu_topk_ws(x, k):
    """mqa_topk_indices_ws: long aligned rows split over several workgroups."""
    t = dev(x)
    out = torch.full((x.shape[0], k), -7, dtype=torch.int32, device="cuda")
    ws = torch.full((max(_native.topk_workspace_size(*x.shape), 1),), 0x7f, dtype=torch.uint8,
                    device="cuda")  # stale contents must not matter
    _native.topk_indices_ws(t, k, indices=out, workspace=ws)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def check(x, k, tag):
    """Both entry points against the oracle, bit for bit."""
    want = oracle_topk(x, k)
    for name, fn in (("one-row", gpu_topk), ("workspace", gpu_topk_ws)):
        got = fn(x, k)
        if not np.array_equal(got, want):
            bad = np.nonzero((got != want).any(axis=1))[0]
            r = int(bad[0])
            j = int(np.nonzero(got[r] != want[r])[0][0])
            raise AssertionError("%s (%s): %d rows differ; row %d first at %d: gpu %s oracle %s"
                                 % (tag, name, bad.size, r, j, got[r, j:j + 4], want[r, j:j + 4]))


@pytest.mark.parametrize("cols", [1, 7, 100, 4096, 33000, 131072])
@pytest.mark.parametrize("k", [1, 5, 512, 2048])
def test_row_families(cols, k):
    x = inputs.topk_rows(cols, seed=500 + cols % 97 + k)
    say("topk families cols=%d k=%d" % (cols, k))
    check(x, k, "families cols=%d k=%d" % (cols, k))


@pytest.mark.parametrize("rows,cols", [(1, 32768), (3, 70001), (40, 131072)])
def test_long_rows_with_runs_of_large_values(rows, cols):
    """Long rows whose largest values sit in short runs spread over the row
    (and in the row's last, odd columns)."""
    rng = np.random.default_rng(540 + rows)
    x = rng.standard_normal((rows, cols)).astype(np.float32)
    n4 = cols // 4
    for parts in range(2, 17):
        for p in range(1, parts):
            c = 4 * (n4 * p // parts)
            x[:, max(c - 2, 0):c + 2] = 5.0 + rng.random((rows, min(c + 2, cols) - max(c - 2, 0)))
    x[:, -3:] = 7.0
    say("topk long rows=%d cols=%d" % (rows, cols))
    for k in (1, 100, 2048):
        check(x, k, "long rows=%d cols=%d k=%d" % (rows, cols, k))


def test_skewed_and_overflowing_rows():
    """Sorted rows (every large value at one end), a constant row (every entry
    survives the sampled threshold, so the exact radix select takes over) and
    a mostly masked row."""
    rng = np.random.default_rng(550)
    base = np.sort(rng.standard_normal(131072).astype(np.float32))
    x = np.stack([base, base[::-1].copy(), np.full(131072, 0.25, np.float32),
                  np.where(rng.random(131072) < 0.9, np.float32(-np.inf), base)])
    say("topk skewed rows")
    for k in (7, 2048):
        check(x, k, "skewed k=%d" % k)


def test_decode_logits_feed_topk():
    d = inputs.make_decode(3, 4, [5000, 700, 2100], 6000, seed=520, poison=True)
    say("topk of decode logits")
    logits = np.ascontiguousarray(run_decode(d))
    for k in (1, 64, 512, 2048):
        check(logits, k, "decode logits k=%d" % k)


def test_long_decode_logits():
    """Decode logits of long sequences (rows of 65536 columns, ragged windows,
    so rows end in runs of -inf)."""
    d = inputs.make_decode(2, 3, [65536, 40000], 65536, seed=521)
    logits = np.ascontiguousarray(run_decode(d))
    say("topk of long decode logits")
    for k in (512, 2048):
        check(logits, k, "long decode logits k=%d" % k)


def test_many_rows_and_odd_widths():
    rng = np.random.default_rng(530)
    x = rng.standard_normal((300, 2049)).astype(np.float32)
    x[:, ::5] = -np.inf
    say("topk 300 rows x 2049")
    check(x, 2048, "300x2049")
    check(x[:, :17].copy(), 20, "k > cols")


def test_zero_columns_writes_minus_one():
    out = torch.full((3, 4), 9, dtype=torch.int32, device="cuda")
    empty = torch.empty((3, 0), dtype=torch.float32, device="cuda")
    _native.topk_indices(empty, 4, indices=out)
    torch.cuda.synchronize()
    assert (out.cpu().numpy() == -1).all()


def test_zero_rows_is_a_no_op():
    _native.topk_indices(torch.empty((0, 10), dtype=torch.float32, device="cuda"), 4)
    _native.topk_indices_ws(torch.empty((0, 10), dtype=torch.float32, device="cuda"), 4)


@pytest.mark.parametrize("rows,cols", [(1, 8196), (2, 131072), (7, 100000), (767, 16384)])
def test_split_row_counts_and_widths(rows, cols):
    """The split path at its edges: the shortest split row, a few rows of the
    benchmark's width, slices that do not divide the row, and the largest row
    count that still splits (767 rows of 16384 columns, two workgroups each)."""
    rng = np.random.default_rng(560 + rows)
    x = rng.standard_normal((rows, cols)).astype(np.float32)
    x[:, rng.integers(0, cols, 50)] = 9.0  # ties across slices
    say("topk split rows=%d cols=%d" % (rows, cols))
    for k in (1, 512, 2048):
        check(x, k, "split rows=%d cols=%d k=%d" % (rows, cols, k))


def _bucketed_row(cols, rng):
    """A row whose sorted order has, from the top: 60 distinct large values,
    200 copies of 0.5 (one crowded bucket), 20 values within 1e-6 of 0.25 (one
    small bucket), then distinct small values; positions shuffled."""
    top = 50.0 + rng.permutation(60).astype(np.float32)
    crowd = np.full(200, 0.5, np.float32)
    near = (0.25 + 1e-6 * rng.random(20)).astype(np.float32)
    rest = (0.2 * rng.random(cols - 280)).astype(np.float32)
    row = np.concatenate([top, crowd, near, rest])
    return row[rng.permutation(cols)]


@pytest.mark.parametrize("k", [30, 59, 60, 61, 100, 259, 260, 261, 270, 280, 281, 512])
def test_sort_buckets_around_k(k):
    # The sort leaves unranked the buckets that start at or past position k;
    # k here falls before, at, inside and after the crowded bucket (positions
    # 60..259) and the small one (260..279).  Short rows (every listable entry
    # gathered) and a long row (the sampled threshold) both run the sort.
    rng = np.random.default_rng(4000 + k)
    say("topk buckets around k=%d" % k)
    for cols in (4000, 8192):
        x = np.stack([_bucketed_row(cols, rng) for _ in range(2)])
        check(x, k, "short rows cols=%d k=%d" % (cols, k))
    long = _bucketed_row(131072, rng)[None, :]
    check(long, k, "long row k=%d" % k)
