"""Pins of the top-k oracle (oracle.topk) against things other than itself.

- a hand-worked example (tests/golden/topk_example.txt);
- a brute force written differently (pure Python, pairwise comparison rule);
- properties any correct answer has, on larger random rows.
"""

from __future__ import annotations

import functools
import math

import numpy as np
import pytest

from oracle.topk import topk_indices
from tests.util import read_kv


def _rows():
    g = read_kv("topk_example.txt")
    rows = np.array([[np.float32(t) for t in g["row%d" % r]] for r in range(5)], dtype=np.float32)
    return g, rows


@pytest.mark.parametrize("k", [1, 3, 8])
def test_hand_example(k):
    g, rows = _rows()
    want = np.array([int(t) for t in g["k%d" % k]], dtype=np.int32).reshape(5, k)
    assert np.array_equal(topk_indices(rows, k), want)


def _brute_row(vals, k):
    """Selection by explicit pairwise comparison (functools.cmp_to_key)."""
    def listable(v):
        return not math.isnan(v) and v != -math.inf

    def cmp(a, b):
        va, vb = float(vals[a]), float(vals[b])
        if va > vb:
            return -1
        if va < vb:
            return 1
        return -1 if a < b else (1 if a > b else 0)

    cols = [c for c in range(len(vals)) if listable(float(vals[c]))]
    chosen = sorted(cols, key=functools.cmp_to_key(cmp))[:k]
    return chosen + [-1] * (k - len(chosen))


@pytest.mark.parametrize("seed", range(6))
def test_matches_pairwise_brute_force(seed):
    rng = np.random.default_rng(seed)
    cols = int(rng.integers(1, 40))
    # few distinct values, so ties are common; plus the special values
    pool = np.array([-2, -0.0, 0.0, 0.5, 1, 1, 3, np.inf, -np.inf, np.nan], dtype=np.float32)
    x = rng.choice(pool, size=(4, cols)).astype(np.float32)
    for k in (1, 2, 5, 64):
        want = np.array([_brute_row(x[r], k) for r in range(4)], dtype=np.int32)
        assert np.array_equal(topk_indices(x, k), want), (seed, k)


@pytest.mark.parametrize("k", [1, 17, 512, 2048])
def test_properties_on_random_rows(k):
    rng = np.random.default_rng(7 + k)
    x = rng.standard_normal((3, 5000)).astype(np.float32)
    x[0, rng.random(5000) < 0.6] = -np.inf           # a window mask
    x[1] = np.round(x[1] * 4) / 4                     # heavy ties
    out = topk_indices(x, k)
    for r in range(3):
        v = x[r]
        listable = ~(np.isnan(v) | (v == -np.inf))
        n = min(k, int(listable.sum()))
        sel = out[r, :n]
        assert (out[r, n:] == -1).all()
        assert len(set(sel.tolist())) == n and listable[sel].all()
        vals = v[sel]
        assert (np.diff(vals) <= 0).all()                     # non-increasing
        same = np.diff(vals) == 0
        assert (np.diff(sel)[same] > 0).all()                  # ties by column
        rest = np.ones(v.size, bool)
        rest[sel] = False
        rest &= listable
        if rest.any() and n:
            assert v[rest].max() <= vals[-1]                   # nothing better left out
            # an unselected entry equal to the last value has a larger column
            eq = np.nonzero(rest & (v == vals[-1]))[0]
            assert (eq > sel[vals == vals[-1]].max()).all()
