"""GPU parity of the prefill logits at head dim 64 (the aiter PR 5046 page's
test sweep covers head dims 64 and 128, "Test Plan"): one fp8 MFMA per
32-token tile instead of two, with 32, 64 and 128 heads.

The same bar as at head dim 128: an exact integer pin (bit for bit), random
inputs element by element against the oracle for every window mode and both
clean_logits settings, and bitwise invariance under the launch tunables.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

from sparse_attention_indexer_scaled_amd import Tunables, inputs, is_supported
from tests.gpu_util import assert_parity, lib, oracle_prefill, run_prefill, say

pytestmark = pytest.mark.gpu
D = 64
HEADS = [32, 64, 128]
MODES = ["causal", "misaligned", "empty", "past_end", "multi_req"]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    lib()
    assert all(is_supported(h, D, 0) for h in HEADS)
    # the decode takes head dim 64 in every block size
    assert is_supported(32, D, 64) and is_supported(32, D, 1)


def _block_ms(H):
    return [bm for bm in (1, 2, 4, 8) if bm * H <= 256]


@pytest.mark.parametrize("H", HEADS)
def test_integer_inputs_bit_exact(H):
    """Integers in [-8, 8], power-of-two weights and scales: every partial sum
    is exact in fp32, so the GPU equals the oracle bit for bit."""
    rng = np.random.default_rng(760 + H)
    M, N = 13, 333
    p = inputs.make_prefill(M, N, seed=760 + H, H=H, D=D)
    p.q = inputs.to_fp8_bytes(rng.integers(-8, 9, (M, H, D)).astype(np.float32))
    p.k = inputs.to_fp8_bytes(rng.integers(-8, 9, (N, D)).astype(np.float32))
    p.weights = (rng.choice([-1, 1], (M, H)) * 2.0 ** -rng.integers(0, 4, (M, H))).astype(np.float32)
    p.kv_scale = rng.choice([0.5, 1.0, 2.0], N).astype(np.float32)
    ref, _ = oracle_prefill(p)
    for bm in _block_ms(H):
        say("prefill d64 int H=%d block_m=%d" % (H, bm))
        assert np.array_equal(run_prefill(p, tun=Tunables(block_m=bm)), ref)


@pytest.mark.parametrize("H", HEADS)
@pytest.mark.parametrize("mode", MODES)
def test_matches_oracle(H, mode):
    p = inputs.make_prefill(70, 700, seed=770 + H, H=H, D=D, windows=mode)
    say("prefill d64 H=%d mode=%s" % (H, mode))
    ref, mag = oracle_prefill(p)
    for clean in (True, False):
        out = run_prefill(p, clean=clean)
        if clean:
            assert_parity(out, ref, mag, f"prefill_d64_H{H}_{mode}")
        else:
            win = np.isfinite(ref)
            assert_parity(np.where(win, out, -np.inf), ref, mag, f"prefill_d64_H{H}_{mode}_noclean")


def test_long_chunk_sampled_rows():
    """A 2048 x 8192 causal chunk with 32 heads in the heuristic launch, every
    64th row (plus the last) against the oracle."""
    p = inputs.make_prefill(2048, 8192, seed=780, D=D)
    rows = list(range(0, 2048, 64)) + [2047]
    say("prefill d64 M2048 N8192 sampled rows")
    out = run_prefill(p)[rows]
    ref, mag = oracle_prefill(p, rows=rows)
    assert_parity(out, ref, mag, "prefill_d64_M2048_N8192")


@pytest.mark.parametrize("H", HEADS)
def test_tunables_do_not_change_bits(H):
    p = inputs.make_prefill(50, 600, seed=790 + H, H=H, D=D, windows="multi_req")
    base = run_prefill(p)
    for bm in _block_ms(H):
        for nw, split, rev in ((1, 2, 1), (3, 1, -1), (4, 7, 0)):
            say("prefill d64 tunables H=%d bm=%d nw=%d split=%d" % (H, bm, nw, split))
            out = run_prefill(p, tun=Tunables(block_m=bm, num_warps=nw, split_n=split,
                                              reverse_rows=rev))
            assert np.array_equal(out, base, equal_nan=True)
