"""Top-k at the benchmark's own shape: the 96 x 131072 logits of paged decode,
batch 16, next_n 6, context 131072, k = 2048 and 512 (the two index_topk values
of the pages).

- The one-row top-k (mqa_topk_indices) and the workspace call that splits
  each row over several workgroups (mqa_topk_indices_ws) rank the oracle's
  logits of that workload (fp64, rounded once to fp32) and must equal the
  oracle's top-k of the same fp32 array bit for bit: both sides take every
  comparison in fp32.
- The fused decode top-k and the unfused pipeline (decode call, then the
  one-row top-k) rank the GPU's own logits, which differ from the oracle's
  within the fp32 parity bound tau = 1e-5 * M per element (M the oracle on
  |Q|, |K|, |w|).  Several outputs are then correct, so the test checks what
  any correct one satisfies against the oracle's logits: k distinct in-window
  columns, an order that holds within tau, no unselected column that beats a
  selected one by more than the two taus, and agreement with the oracle's own
  top-k except at such near-ties.  The fused and unfused outputs must also be
  identical to each other (the fused call's definition).
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

from oracle.topk import topk_indices as oracle_topk
from sparse_attention_indexer_scaled_amd import _native, inputs
from tests.gpu_util import REL_TOL, decode_device_inputs, dev, lib, oracle_decode, run_decode, say

pytestmark = pytest.mark.gpu

KS = (2048, 512)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    lib()


@pytest.fixture(scope="module")
def headline():
    d = inputs.make_config(2)
    say("oracle logits of the headline decode (96 x 131072)")
    ref, mag, _ = oracle_decode(d)
    return d, ref, mag


def _first_diff(got, want, tag):
    bad = np.nonzero((got != want).any(axis=1))[0]
    r = int(bad[0])
    j = int(np.nonzero(got[r] != want[r])[0][0])
    return "%s: %d rows differ; row %d first at %d: got %s want %s" % (
        tag, bad.size, r, j, got[r, j:j + 4], want[r, j:j + 4])


@pytest.mark.parametrize("k", KS)
def test_one_row_topk_of_the_oracle_logits(headline, k):
    _, ref, _ = headline
    x = ref.astype(np.float32)
    say("topk of the headline's oracle logits k=%d" % k)
    want = oracle_topk(x, k)
    t = dev(x)
    out = torch.full((x.shape[0], k), -7, dtype=torch.int32, device="cuda")
    _native.topk_indices(t, k, indices=out)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    assert np.array_equal(got, want), _first_diff(got, want, "k=%d" % k)
    # the workspace call splits each of these rows over several workgroups
    out.fill_(-7)
    ws = torch.full((_native.topk_workspace_size(*x.shape),), 0x5a, dtype=torch.uint8,
                    device="cuda")
    _native.topk_indices_ws(t, k, indices=out, workspace=ws)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    assert np.array_equal(got, want), _first_diff(got, want, "workspace call k=%d" % k)


def _assert_valid_topk(idx, ref, tau, k, tag):
    rows, cols = ref.shape
    want = oracle_topk(ref.astype(np.float32), k)
    near_tie_rows = 0
    for r in range(rows):
        s = idx[r]
        assert s.shape == (k,) and np.all((s >= 0) & (s < cols)), "%s row %d: bad index" % (tag, r)
        assert np.unique(s).size == k, "%s row %d: repeated column" % (tag, r)
        v, t = ref[r], tau[r]
        assert np.all(np.isfinite(v[s])), "%s row %d: a column outside the window" % (tag, r)
        # order within the bound
        assert np.all(v[s][:-1] + t[s][:-1] >= v[s][1:] - t[s][1:]), "%s row %d: order" % (tag, r)
        # no unselected listable column clearly above a selected one
        rest = np.ones(cols, bool)
        rest[s] = False
        rest &= np.isfinite(v)
        lo = float((v[s] + t[s]).min())
        hi = float((v[rest] - t[rest]).max()) if rest.any() else -np.inf
        assert hi <= lo, "%s row %d: an unselected column beats a selected one" % (tag, r)
        if not np.array_equal(s, want[r]):
            # every difference from the oracle's own ranking is a near-tie
            j = np.nonzero(s != want[r])[0]
            a, b = s[j], want[r][j]
            assert np.all(np.abs(v[a] - v[b]) <= t[a] + t[b]), "%s row %d: not a near-tie" % (tag, r)
            near_tie_rows += 1
    return near_tie_rows


def test_fused_and_unfused_topk_at_the_headline_shape(headline):
    d, ref, mag = headline
    tau = REL_TOL * mag
    dv = decode_device_inputs(d)
    logits = dev(run_decode(d, dv=dv))
    need = _native.paged_mqa_topk_workspace_size(d.B, d.next_n, d.max_model_len)
    ws = torch.full((need,), 0xA5, dtype=torch.uint8, device="cuda")
    for k in KS:
        say("fused and unfused topk at the headline shape k=%d" % k)
        fused = torch.full((d.B * d.next_n, k), -7, dtype=torch.int32, device="cuda")
        _native.paged_mqa_topk_decode(dv["q"], dv["cache"], dv["w"], dv["ctx"], dv["bt"],
                                      d.max_model_len, k, kv_block_size=d.block_size,
                                      indices=fused, workspace=ws)
        unfused = _native.topk_indices(logits, k)
        torch.cuda.synchronize()
        f, u = fused.cpu().numpy(), unfused.cpu().numpy()
        assert np.array_equal(f, u), _first_diff(f, u, "fused vs unfused k=%d" % k)
        n = _assert_valid_topk(f, ref, tau, k, "k=%d" % k)
        say("  rows whose order differs from the oracle's only at near-ties: %d of %d"
            % (n, f.shape[0]))
