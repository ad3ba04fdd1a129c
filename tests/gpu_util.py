"""Helpers for the GPU parity tests: run the HIP library through its binding,
run the oracle on the same bytes, and compare.

Parity bar (per element, on every compared position):
  * the -inf mask matches exactly (the pages' gate, aiter PR 5047 / 5046 pages,
    "Test Plan");
  * calc_diff < 1e-3 (the pages' gate; our reading of calc_diff in tests/util.py);
  * and a bound derived from fp32 arithmetic:
        |gpu - oracle| <= 1e-5 * sum_h |w_h| sum_d |q_hd k_d| * scale
    The right-hand magnitude is the oracle itself evaluated on |Q|, |K|, |w|.
    fp32 accumulation of the 128-term dot and the 32-term head sum, plus the
    two products, stays below (128 + 32 + 2) * 2^-24 ~ 1e-5 of that magnitude.
"""

from __future__ import annotations

import os
import sys

import numpy as np
import torch

import oracle
from sparse_attention_indexer_scaled_amd import _native
from tests.util import calc_diff, mask_equal

OUT_DIR = os.environ.get("MQA_FAIL_DIR",
                         os.path.join(__import__("tempfile").gettempdir(), "mqa_failures"))
REL_TOL = 1e-5
CALC_DIFF_GATE = 1e-3


def lib():
    if not os.path.exists(_native.LIB_PATH):
        from sparse_attention_indexer_scaled_amd import build
        build.build()
    return _native.load_library()


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def dev(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.cuda()


def run_prefill(p, clean=True, tun=None, fill=float("nan")):
    M, N = p.M, p.N
    out = torch.full((M, N), fill, dtype=torch.float32, device="cuda")
    _native.mqa_logits_prefill(dev(p.q), dev(p.k), dev(p.kv_scale), dev(p.weights), dev(p.ks),
                               dev(p.ke), logits=out, clean_logits=clean, tunables=tun)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def decode_device_inputs(d):
    return dict(q=dev(d.q), cache=dev(d.kv_cache), w=dev(d.weights), ctx=dev(d.context_lens),
                bt=dev(d.block_tables))


def run_decode(d, clean=True, tun=None, fill=float("nan"), dv=None):
    dv = dv or decode_device_inputs(d)
    rows = d.B * d.next_n
    out = torch.full((rows, d.max_model_len), fill, dtype=torch.float32, device="cuda")
    _native.paged_mqa_logits_decode(dv["q"], dv["cache"], dv["w"], dv["ctx"], dv["bt"],
                                    d.max_model_len, d.block_size, logits=out,
                                    clean_logits=clean, tunables=tun, preshuffle=d.preshuffle)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def _abs8(codes):
    return codes & np.uint8(0x7F)


def oracle_prefill(p, rows=None):
    """(oracle logits, magnitude bound) for all rows or a subset."""
    sel = slice(None) if rows is None else np.asarray(rows)
    q, w, ks, ke = p.q[sel], p.weights[sel], p.ks[sel], p.ke[sel]
    ref = oracle.prefill(q, p.k, p.kv_scale, w, ks, ke)
    mag = oracle.prefill(_abs8(q), _abs8(p.k), p.kv_scale, np.abs(w), ks, ke)
    return ref, mag


def oracle_decode(d, seqs=None):
    """(oracle logits, magnitude, output row indices) for all sequences or a
    subset; the returned rows are those sequences' rows, in order."""
    b = np.arange(d.B) if seqs is None else np.asarray(seqs)
    rows = (b[:, None] * d.next_n + np.arange(d.next_n)[None, :]).reshape(-1)
    ctx, bt = d.context_lens[b], d.block_tables[b]
    ref = oracle.decode(d.q[b], d.kv_cache, d.weights[rows], ctx, bt, d.max_model_len,
                        d.block_size, preshuffle=d.preshuffle)
    mag = oracle.decode(_abs8(d.q[b]), _abs8_cache(d), np.abs(d.weights[rows]), ctx, bt,
                        d.max_model_len, d.block_size, preshuffle=d.preshuffle)
    return ref, mag, rows


def _abs8_cache(d):
    """The cache with every K byte's sign cleared (scales untouched)."""
    c = d.kv_cache.copy()
    kbytes = d.block_size * d.D
    c[:, :kbytes] &= np.uint8(0x7F)
    return c


def save_failure(name, **arrays):
    try:
        os.makedirs(OUT_DIR, exist_ok=True)
        np.savez_compressed(os.path.join(OUT_DIR, "fail_%s.npz" % name), **arrays)
    except OSError:
        pass


def assert_parity(gpu, ref, mag, name, rel_tol=REL_TOL):
    gpu = np.asarray(gpu, dtype=np.float64)
    ok_mask = mask_equal(gpu, ref)
    fin = np.isfinite(ref)
    nonfinite_gpu = int((~np.isfinite(gpu) & fin).sum())
    cd = calc_diff(gpu, ref)
    err = np.abs(gpu[fin] - ref[fin])
    bound = rel_tol * mag[fin] + 1e-30
    worst = float((err / bound).max()) if err.size else 0.0
    say("[parity] %s: mask %s, calc_diff %.3e, worst err/bound %.3e, nonfinite-in-window %d"
        % (name, "ok" if ok_mask else "MISMATCH", cd, worst, nonfinite_gpu))
    if not (ok_mask and nonfinite_gpu == 0 and cd < CALC_DIFF_GATE and worst <= 1.0):
        save_failure(name, gpu=gpu, ref=ref, mag=mag)
    assert ok_mask, "%s: -inf mask differs at %d positions" % (name, int((np.isneginf(gpu) != np.isneginf(ref)).sum()))
    assert nonfinite_gpu == 0, "%s: %d in-window outputs are not finite" % (name, nonfinite_gpu)
    assert cd < CALC_DIFF_GATE, "%s: calc_diff %.3e" % (name, cd)
    assert worst <= 1.0, "%s: error %.3e x the fp32 bound" % (name, worst)
    return cd, worst
