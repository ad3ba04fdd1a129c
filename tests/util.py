"""Shared test helpers: golden-file parsing and the parity metrics."""

from __future__ import annotations

import os

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def golden_path(name):
    return os.path.join(ROOT, "tests", "golden", name)


def read_kv(name):
    """Parse `key = values...` lines (comments start with #)."""
    out = {}
    with open(golden_path(name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line or "=" not in line:
                continue
            k, v = line.split("=", 1)
            out[k.strip()] = v.split()
    return out


def floats(tokens):
    return np.array([float(t) for t in tokens], dtype=np.float64)


def calc_diff(x, y):
    """Relative squared L2 distance used as the parity gate.

    The pages gate on "calc_diff < 1e-3" without defining it (aiter PR 5047 and
    5046 pages, "Test Plan"); our reading: sum (x-y)^2 / sum (x^2 + y^2) in
    fp64 over positions finite in both, 0 when both are all zero.
    """
    x = np.asarray(x, dtype=np.float64)
    y = np.asarray(y, dtype=np.float64)
    fin = np.isfinite(x) & np.isfinite(y)
    x = x[fin]
    y = y[fin]
    den = float((x * x + y * y).sum())
    if den == 0.0:
        return 0.0
    return float(((x - y) ** 2).sum()) / den


def mask_equal(x, y):
    """Exact -inf mask match: -inf exactly where the other is -inf."""
    return np.array_equal(np.isneginf(x), np.isneginf(y))
