"""Every entry point captured into a HIP graph and replayed.

Each call is captured once (after one eager call on the capture stream, which
sets the kernels' LDS limits and looks up the static scratch) and replayed
three times.  Between replays the program does eager work of its own: the
output is overwritten (NaN, or -7 for indices), another call of the library
runs on other inputs (for the allocation-free fused top-k, on the same static
scratch), and the device is synchronized.  Every replay must reproduce the
eager call's output bit for bit.  No call issues a memset or an allocation
inside its launches (nothing in a workspace has to start cleared), so the
captures hold kernel nodes only.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

from sparse_attention_indexer_scaled_amd import _native, inputs
from tests.gpu_util import decode_device_inputs, dev, lib, say

pytestmark = pytest.mark.gpu

REPLAYS = 3


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    lib()


def _graph_replays(tag, call, out, poison, between):
    """Eager result of call() (which writes `out`), then REPLAYS replays of
    its captured graph, each checked bit for bit against it."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        out.fill_(poison)
        call()
    torch.cuda.synchronize()
    want = out.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        call()
    torch.cuda.synchronize()
    for i in range(REPLAYS):
        out.fill_(poison)
        between()
        torch.cuda.synchronize()
        say("%s: replay %d" % (tag, i))
        g.replay()
        torch.cuda.synchronize()
        got, ref = out.cpu(), want.cpu()
        same = torch.equal(got.view(torch.int32), ref.view(torch.int32)) \
            if got.dtype == torch.float32 else torch.equal(got, ref)
        assert same, "%s: replay %d differs from the eager call" % (tag, i)
    del g


def _decode_case(seed, ctx, mml=4096):
    d = inputs.make_decode(2, 3, ctx, mml, seed=seed, poison=True)
    return d, decode_device_inputs(d)


def test_decode_and_prefill_graphs():
    d, dv = _decode_case(1200, [3000, 700])
    d2, dv2 = _decode_case(1201, [4096, 1500])
    out = torch.empty((d.B * d.next_n, d.max_model_len), dtype=torch.float32, device="cuda")
    out2 = torch.empty_like(out)
    dec = lambda o, x, v: _native.paged_mqa_logits_decode(
        v["q"], v["cache"], v["w"], v["ctx"], v["bt"], x.max_model_len, x.block_size, logits=o,
        clean_logits=True)
    _graph_replays("decode", lambda: dec(out, d, dv), out, float("nan"),
                   lambda: dec(out2, d2, dv2))

    p = inputs.make_prefill(256, 2048, seed=1202)
    pv = [dev(a) for a in (p.q, p.k, p.kv_scale, p.weights, p.ks, p.ke)]
    pout = torch.empty((p.M, p.N), dtype=torch.float32, device="cuda")
    _graph_replays("prefill", lambda: _native.mqa_logits_prefill(*pv, logits=pout,
                                                                 clean_logits=True),
                   pout, float("nan"), lambda: dec(out2, d2, dv2))


def test_topk_graphs():
    rng = np.random.default_rng(1210)
    x = dev(rng.standard_normal((8, 65536)).astype(np.float32))
    y = dev(rng.standard_normal((8, 65536)).astype(np.float32))
    k = 2048
    idx = torch.empty((8, k), dtype=torch.int32, device="cuda")
    other = torch.empty_like(idx)
    _graph_replays("topk", lambda: _native.topk_indices(x, k, indices=idx), idx, -7,
                   lambda: _native.topk_indices(y, k, indices=other))
    ws = torch.empty(_native.topk_workspace_size(8, 65536), dtype=torch.uint8, device="cuda")
    ws2 = torch.empty_like(ws)
    _graph_replays("topk_ws", lambda: _native.topk_indices_ws(x, k, indices=idx, workspace=ws),
                   idx, -7, lambda: _native.topk_indices_ws(y, k, indices=other, workspace=ws2))


def test_fused_topk_graphs():
    """The fused top-k with a caller workspace, and the allocation-free
    variant with an eager call on other inputs between replays, which leaves
    the static scratch full of that call's entries."""
    d, dv = _decode_case(1220, [20000, 9000], mml=20480)
    d2, dv2 = _decode_case(1221, [20480, 12000], mml=20480)
    k = 512
    rows = d.B * d.next_n
    idx = torch.empty((rows, k), dtype=torch.int32, device="cuda")
    other = torch.empty_like(idx)
    need = _native.paged_mqa_topk_workspace_size(d.B, d.next_n, d.max_model_len)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    ws2 = torch.empty_like(ws)
    fused = lambda o, x, v, w: _native.paged_mqa_topk_decode(
        v["q"], v["cache"], v["w"], v["ctx"], v["bt"], x.max_model_len, k,
        kv_block_size=x.block_size, indices=o, workspace=w)
    _graph_replays("fused", lambda: fused(idx, d, dv, ws), idx, -7,
                   lambda: fused(other, d2, dv2, ws2))
    noalloc = lambda o, x, v: _native.paged_mqa_topk_decode_noalloc(
        v["q"], v["cache"], v["w"], v["ctx"], v["bt"], x.max_model_len, k, o,
        kv_block_size=x.block_size)
    _graph_replays("fused_noalloc", lambda: noalloc(idx, d, dv), idx, -7,
                   lambda: noalloc(other, d2, dv2))
    # the graph's indices are the workspace call's
    assert torch.equal(idx, fused(other, d, dv, ws))


def test_kcache_insert_graph():
    rng = np.random.default_rng(1230)
    T, bs, nb = 300, 64, 16
    k = dev(rng.standard_normal((T, 128)).astype(np.float32))
    slots = dev(rng.permutation(nb * bs)[:T].astype(np.int64))
    cache = torch.zeros((nb, bs * 132), dtype=torch.uint8, device="cuda")
    cache2 = torch.zeros_like(cache)
    _graph_replays("kcache_insert",
                   lambda: _native.kcache_quantize_insert(k, slots, cache, kv_block_size=bs),
                   cache, 0, lambda: _native.kcache_quantize_insert(k, slots, cache2,
                                                                     kv_block_size=bs))
