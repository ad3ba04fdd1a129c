#!/usr/bin/env python3
"""Benchmark of the lightning-indexer logits library on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--repeats R] [--workload IDX]
                    [--hot] [--no-cpu] [--only IDX] [--calib-copy MB] [--calib-mfma]

A step is one call of the op over one batch of synthetic input (every stage of
the kernel: Q/weights prologue, K load or block-table gather, fp8 MFMA,
relu.weight epilogue, lane-permute head reduce, kv-scale, masked store and
-inf fill).  The headline line is paged decode, batch 16, next_n 6, context
131072, 64-token blocks (the workload the pages' own decode timings are quoted
on); the other named workloads are measured in the same run and reported
under "workloads".

Timing: W eager warm-up calls (extended to ~0.3 s so clocks settle), then R
timings of exactly K calls, each between two events on the launch stream with
synchronisation on both sides; the median of the R per-call times is
reported (the repeats beside it).  A call is replayed from one HIP graph when
it is launch-bound (under 20 us), timed as plain back-to-back launches
otherwise.  Inputs rotate over enough copies that the working set exceeds the
256 MB MALL (cold, as a serving step sees per-layer KV); the five named
configurations (and the next_n 1 long-context decode) are also timed on one
copy (hot); --hot keeps one copy throughout.

Measured in the same run: the launch floor (an empty kernel timed the same
two ways), the fp8 MFMA rate of an MFMA-only kernel (the roofline's peak stays
the published 5.0 PFLOP/s; the measured rate is reported beside it), and the
CPU oracle's time on each named configuration (median of three runs on the
short ones, one run on the long prefill chunk's row sample and the ragged
batch).

Prints ONE JSON line.
"""

from __future__ import annotations

import argparse
import json
import os
import platform
import re
import sys
import time

import numpy as np

HBM_PEAK_TBS = 8.0
FP8_PEAK_TFLOPS = 5000.0  # MI355X dense fp8 MFMA (no sparsity)
COLD_BYTES = 512 << 20


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", type=int, default=2, help="headline workload index")
    ap.add_argument("--only", type=int, default=None, help="measure just this workload")
    ap.add_argument("--hot", action="store_true", help="one input copy (MALL-warm)")
    ap.add_argument("--pages-table", action="store_true",
                    help="time the decode shapes of the fp8 paged MQA logits PR page's "
                         "performance table beside that page's HIP kernel (context, not the "
                         "benchmark line)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-graph", action="store_true", help="time eager launches")
    ap.add_argument("--tunables", default="",
                    help="launch overrides, e.g. rows_per_block=3,split_kv=64 (0 = heuristic)")
    ap.add_argument("--write-traffic-profile", nargs=6, default=None,
                    metavar=("WORKLOAD", "FETCH_DIR", "WRITE_DIR", "CAL_FETCH_DIR", "CAL_WRITE_DIR",
                             "CAL_MIB"),
                    help="summarise FETCH_SIZE/WRITE_SIZE runs into profiles/ (no GPU needed)")
    ap.add_argument("--write-kernel-stats", nargs=2, default=None, metavar=("WORKLOAD", "STATS_DIR"),
                    help="summarise a rocprofv3 --stats run into profiles/ (no GPU needed)")
    ap.add_argument("--write-counter-profile", nargs="+", default=None,
                    metavar="WORKLOAD_OR_DIR",
                    help="WORKLOAD DIR [DIR ...]: summarise rocprofv3 --pmc runs of SQ/GRBM "
                         "counters into profiles/ (no GPU needed)")
    ap.add_argument("--profile-command", default="", help="command recorded in the summary")
    ap.add_argument("--repeats", type=int, default=5,
                    help="timings of --steps calls per workload; the median is reported")
    ap.add_argument("--calib-mfma", action="store_true",
                    help="only time the MFMA-only calibration kernel (fp8 TFLOP/s)")
    ap.add_argument("--calib-copy", type=int, default=0,
                    help="only run a plain device copy of this many MiB (counter calibration)")
    return ap.parse_args()


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor()


# Top-k workloads: index -> (decode workload whose logits are ranked, k).  The
# pages' deployments use index_topk 2048 and 512.
TOPK_WORKLOADS = {5: (2, 2048), 6: (2, 512)}
# The same top-k through mqa_topk_indices_ws (each long row split over several
# workgroups, with a workspace allocated once): index -> (decode workload, k).
TOPK_WS_WORKLOADS = {23: (2, 2048), 24: (2, 512)}
# K-cache insert workloads: index -> (tokens, bf16 input).  4096 tokens is the
# long prefill chunk's K; 96 is one decode step of the MTP workload (16 x 6).
KCACHE_WORKLOADS = {7: (4096, False), 8: (96, True)}
# Fused decode top-k workloads: index -> (decode workload, k); the indices
# only, the logits never written.
FUSED_WORKLOADS = {16: (2, 2048), 17: (2, 512)}
# Workloads also timed on one input copy (MALL-warm) beside the cold figure.
HOT_ALSO = (0, 1, 2, 3, 4, 22)
# Workloads whose oracle time is measured in the same run: index -> runs
# (median of three on the short ones, one run on the long prefill chunk's row
# sample and the ragged batch).
CPU_BASELINE_RUNS = {0: 3, 1: 3, 2: 3, 3: 1, 4: 1}


class Workload:
    """Device-resident input copies and output buffers for one named workload."""

    def __init__(self, idx, hot, tunables=None):
        import torch
        from sparse_attention_indexer_scaled_amd import inputs, workload
        self.idx = idx
        self.cfg = inputs.CONFIGS[idx]
        self.kind = self.cfg["kind"]
        t0 = time.time()
        host = inputs.make_config(idx)
        self.gen_s = time.time() - t0
        self.host = host
        dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
        if self.kind == "prefill":
            base = dict(q=dev(host.q), k=dev(host.k), sc=dev(host.kv_scale), w=dev(host.weights),
                        ks=dev(host.ks), ke=dev(host.ke))
            self.out_shape = (host.M, host.N)
            self.bytes = workload.prefill_essential_bytes(host.M, host.N, H=host.H, D=host.D)
            self.pairs = workload.prefill_valid_pairs(host.ks, host.ke, host.N)
            set_bytes = sum(t.numel() * t.element_size() for t in base.values()) + host.M * host.N * 4
        else:
            base = dict(q=dev(host.q), cache=dev(host.kv_cache), w=dev(host.weights),
                        ctx=dev(host.context_lens), bt=dev(host.block_tables))
            self.out_shape = (host.B * host.next_n, host.max_model_len)
            self.bytes = workload.decode_essential_bytes(host.B, host.next_n, host.context_lens,
                                                         host.max_model_len, H=host.H, D=host.D,
                                                         block_size=host.block_size)
            self.pairs = workload.decode_valid_pairs(host.next_n, host.context_lens,
                                                     host.max_model_len)
            set_bytes = sum(t.numel() * t.element_size() for t in base.values()) + \
                self.out_shape[0] * self.out_shape[1] * 4
        self.flops = self.pairs * workload.flops_per_pair(H=host.H, D=host.D)
        nsets = 1 if hot else min(64, max(1, -(-COLD_BYTES // set_bytes)))
        self.sets = [base] + [{k: v.clone() for k, v in base.items()} for _ in range(nsets - 1)]
        self.outs = [torch.empty(self.out_shape, dtype=torch.float32, device="cuda")
                     for _ in range(nsets)]
        self.nsets = nsets
        self.tun = tunables

    def call(self, i):
        from sparse_attention_indexer_scaled_amd import mqa_logits_prefill, paged_mqa_logits_decode
        s = self.sets[i % self.nsets]
        out = self.outs[i % self.nsets]
        if self.kind == "prefill":
            mqa_logits_prefill(s["q"], s["k"], s["sc"], s["w"], s["ks"], s["ke"], logits=out,
                               tunables=self.tun)
        else:
            paged_mqa_logits_decode(s["q"], s["cache"], s["w"], s["ctx"], s["bt"],
                                    self.host.max_model_len, kv_block_size=self.host.block_size,
                                    logits=out, tunables=self.tun, preshuffle=self.host.preshuffle)


class TopkWorkload:
    """Row-wise top-k over the logits of a decode workload (the indexer's
    consumer).  The logits are produced once by the decode kernel, then copied
    so that the timed calls rotate over > COLD_BYTES of input."""

    def __init__(self, idx, hot):
        import torch
        self.split = idx in TOPK_WS_WORKLOADS
        decode_idx, k = (TOPK_WS_WORKLOADS if self.split else TOPK_WORKLOADS)[idx]
        src = Workload(decode_idx, True)
        src.call(0)
        torch.cuda.synchronize()
        logits = src.outs[0]
        rows, cols = logits.shape
        self.idx = idx
        self.kind = "topk"
        self.k = k
        self.cfg = {"kind": "topk",
                    "name": "topk_%sk%d_%s" % ("ws_" if self.split else "", k, src.cfg["name"]),
                    "rows": rows, "cols": cols, "k": k}
        self.host = src.host
        self.bytes = rows * cols * 4 + rows * k * 4
        self.pairs = 0
        self.flops = 0
        set_bytes = rows * cols * 4
        nsets = 1 if hot else min(64, max(1, -(-COLD_BYTES // set_bytes)))
        self.sets = [logits] + [logits.clone() for _ in range(nsets - 1)]
        self.outs = [torch.empty((rows, k), dtype=torch.int32, device="cuda") for _ in range(nsets)]
        self.nsets = nsets
        self.ws = None
        if self.split:
            from sparse_attention_indexer_scaled_amd import topk_workspace_size
            self.ws = torch.empty(topk_workspace_size(rows, cols), dtype=torch.uint8, device="cuda")
        del src

    def call(self, i):
        from sparse_attention_indexer_scaled_amd import topk_indices, topk_indices_ws
        if self.split:
            topk_indices_ws(self.sets[i % self.nsets], self.k, indices=self.outs[i % self.nsets],
                            workspace=self.ws)
        else:
            topk_indices(self.sets[i % self.nsets], self.k, indices=self.outs[i % self.nsets])


class KcacheWorkload:
    """K-cache quantise-and-insert of T new tokens (the step before decode)."""

    def __init__(self, idx, hot):
        import torch
        from sparse_attention_indexer_scaled_amd import inputs
        T, bf16 = KCACHE_WORKLOADS[idx]
        nblocks = -(-T // 64) + 8
        c = inputs.make_kcache_insert(T, nblocks, seed=1000 + idx, bf16=bf16, padding=0.0)
        self.idx = idx
        self.kind = "kcache"
        self.cfg = {"kind": "kcache", "name": "kcache_insert_T%d_%s" % (T, "bf16" if bf16 else "fp32"),
                    "tokens": T}
        self.host = c
        dtype = torch.bfloat16 if bf16 else torch.float32
        base = dict(k=torch.from_numpy(c.k).cuda().to(dtype),
                    slots=torch.from_numpy(c.slot_mapping).cuda(),
                    cache=torch.from_numpy(c.kv_cache).cuda())
        self.bytes = T * 128 * (2 if bf16 else 4) + T * 8 + T * 132
        self.pairs = 0
        self.flops = 0
        set_bytes = sum(t.numel() * t.element_size() for t in base.values())
        nsets = 1 if hot else min(64, max(1, -(-COLD_BYTES // set_bytes)))
        self.sets = [base] + [{k: v.clone() for k, v in base.items()} for _ in range(nsets - 1)]
        self.nsets = nsets

    def call(self, i):
        from sparse_attention_indexer_scaled_amd import kcache_quantize_insert
        s = self.sets[i % self.nsets]
        kcache_quantize_insert(s["k"], s["slots"], s["cache"])


class FusedTopkWorkload:
    """Paged decode fused with the top-k of its logits (paged_mqa_topk_decode).
    Essential bytes: the decode's inputs (K and scales once, Q, weights, used
    table entries, context lengths) plus the indices written."""

    def __init__(self, idx, hot, tunables=None):
        import torch
        from sparse_attention_indexer_scaled_amd import paged_mqa_topk_workspace_size
        decode_idx, k = FUSED_WORKLOADS[idx]
        src = Workload(decode_idx, hot, tunables)
        h = src.host
        rows = h.B * h.next_n
        self.idx = idx
        self.kind = "fused_topk"
        self.k = k
        self.cfg = {"kind": "fused_topk", "name": "decode_topk_k%d_%s" % (k, src.cfg["name"][7:]),
                    "k": k}
        self.host = h
        self.sets = src.sets
        self.nsets = src.nsets
        self.bytes = src.bytes - rows * h.max_model_len * 4 + rows * k * 4
        self.pairs = src.pairs
        self.flops = src.flops
        self.tun = tunables
        self.outs = [torch.empty((rows, k), dtype=torch.int32, device="cuda")
                     for _ in range(self.nsets)]
        self.ws = torch.empty(paged_mqa_topk_workspace_size(h.B, h.next_n, h.max_model_len),
                              dtype=torch.uint8, device="cuda")

    def call(self, i):
        from sparse_attention_indexer_scaled_amd import paged_mqa_topk_decode
        s = self.sets[i % self.nsets]
        paged_mqa_topk_decode(s["q"], s["cache"], s["w"], s["ctx"], s["bt"],
                              self.host.max_model_len, self.k, kv_block_size=self.host.block_size,
                              indices=self.outs[i % self.nsets], workspace=self.ws,
                              tunables=self.tun, preshuffle=self.host.preshuffle)


def make_workload(idx, hot, tunables=None):
    if idx in TOPK_WORKLOADS or idx in TOPK_WS_WORKLOADS:
        return TopkWorkload(idx, hot)
    if idx in FUSED_WORKLOADS:
        return FusedTopkWorkload(idx, hot, tunables)
    if idx in KCACHE_WORKLOADS:
        return KcacheWorkload(idx, hot)
    return Workload(idx, hot, tunables)


def time_workload(wl, steps, warmup, graph=None, settle_s=0.3, repeats=5):
    """Per-call milliseconds: `repeats` timings of exactly `steps` calls, each
    between two events on the launch stream with a synchronisation on both
    sides; returns (median, list of the repeats).  Warm-up: `warmup` calls,
    extended until about settle_s of GPU work has run so that clocks have
    left their idle state before the timed region."""
    import torch
    t0 = time.time()
    i = 0
    while i < warmup or time.time() - t0 < settle_s:
        wl.call(i)
        i += 1
        if i % 16 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    wl.warmup_done = i
    stream = torch.cuda.current_stream()
    if graph is None:
        # Launch-bound calls (a few microseconds) are replayed from a HIP graph;
        # longer ones are timed as plain back-to-back launches, which keeps the
        # host's launch gap inside the measurement.
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for j in range(8):
            wl.call(j)
        e1.record(stream)
        torch.cuda.synchronize()
        graph = e0.elapsed_time(e1) / 8 < 0.02
    wl.graph = graph
    if graph:
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            with torch.cuda.graph(g, stream=side):
                for i in range(steps):
                    wl.call(i)
        stream.wait_stream(side)
        g.replay()  # one untimed replay so the graph itself is resident
        torch.cuda.synchronize()
    reps = []
    for _ in range(repeats):
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record(stream)
        if graph:
            g.replay()
        else:
            for i in range(steps):
                wl.call(i)
        end.record(stream)
        torch.cuda.synchronize()
        reps.append(start.elapsed_time(end) / steps)
    return float(np.median(reps)), reps


def summarize(wl, ms, reps=()):
    us = ms * 1e3
    d = dict(workload=wl.cfg["name"], us_per_call=round(us, 3), input_copies=wl.nsets,
             timing="hip graph replay" if wl.graph else "back-to-back launches",
             essential_bytes=int(wl.bytes), valid_pairs=int(wl.pairs))
    if reps:
        d["repeats_us"] = [round(r * 1e3, 3) for r in reps]
    tbs = wl.bytes / (ms * 1e-3) / 1e12
    tflops = wl.flops / (ms * 1e-3) / 1e12
    d["essential_TBps"] = round(tbs, 4)
    d["hbm_frac"] = round(tbs / HBM_PEAK_TBS, 4)
    if wl.flops:
        d["fp8_TFLOPs"] = round(tflops, 2)
        d["mfma_frac"] = round(tflops / FP8_PEAK_TFLOPS, 4)
    return d


def _oracle_threads():
    import oracle
    n = int(os.environ.get("OMP_NUM_THREADS") or len(os.sched_getaffinity(0)))
    oracle.set_num_threads(n)
    return n


def cpu_baseline_of(wl, runs):
    """The oracle (as it stands) on one named logits workload, in the metric's
    unit: essential TB/s for decode, fp8-equivalent TFLOP/s for prefill.
    Whole workloads where that takes seconds (median of `runs` runs); the long
    prefill chunk on a sample of every 8th query row (its windows, and so its
    work per row, span the whole causal triangle), one run."""
    import oracle
    from sparse_attention_indexer_scaled_amd import workload
    h = wl.host
    nthreads = _oracle_threads()
    times = []
    if wl.kind == "prefill":
        rows = np.arange(h.M) if h.M <= 1024 else np.arange(0, h.M, 8)
        for _ in range(runs):
            t0 = time.time()
            oracle.prefill(h.q[rows], h.k, h.kv_scale, h.weights[rows], h.ks[rows], h.ke[rows])
            times.append(time.time() - t0)
        dt = float(np.median(times))
        flops = workload.prefill_valid_pairs(h.ks[rows], h.ke[rows], h.N) * \
            workload.flops_per_pair(H=h.H, D=h.D)
        value, unit = flops / dt / 1e12, "TFLOP/s"
        sample = ("all %d rows" % h.M if rows.size == h.M else
                  "%d of %d query rows (every 8th)" % (rows.size, h.M))
        full_s = dt * wl.pairs / max(workload.prefill_valid_pairs(h.ks[rows], h.ke[rows], h.N), 1)
    else:
        for _ in range(runs):
            t0 = time.time()
            oracle.decode(h.q, h.kv_cache, h.weights, h.context_lens, h.block_tables,
                          h.max_model_len, h.block_size, preshuffle=h.preshuffle)
            times.append(time.time() - t0)
        dt = float(np.median(times))
        value, unit = wl.bytes / dt / 1e12, "TB/s"
        sample = "all %d sequences, %d rows each, every position to max_model_len" % (
            h.B, h.next_n)
        full_s = dt
    return {"value": round(value, 8), "unit": unit, "cores": nthreads, "kind": "oracle",
            "cpu": cpu_model(), "seconds": round(dt, 3), "runs": runs,
            "us_per_call_full_workload": round(full_s * 1e6, 1), "sample": "%s of %s" % (
                sample, wl.cfg["name"])}


def load_calib():
    import ctypes
    from sparse_attention_indexer_scaled_amd import build
    if not os.path.exists(build.CALIB_LIB):
        build.build_calib()
    lib = ctypes.CDLL(build.CALIB_LIB)
    lib.mqa_calib_empty.restype = ctypes.c_int
    lib.mqa_calib_empty.argtypes = [ctypes.c_int, ctypes.c_void_p]
    lib.mqa_calib_mfma_fp8.restype = ctypes.c_int
    lib.mqa_calib_mfma_fp8.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    return lib


class EmptyKernel:
    """The launch floor: one empty kernel per call, timed like a workload."""

    def __init__(self, lib):
        self.lib = lib
        self.nsets = 1
        self.cfg = {"name": "empty_kernel"}

    def call(self, i):
        import torch
        rc = self.lib.mqa_calib_empty(1, torch.cuda.current_stream().cuda_stream)
        assert rc == 0, "empty kernel launch failed"


def launch_floor(lib, steps, repeats):
    """Per-launch microseconds of an empty kernel: replayed from a HIP graph
    (how the launch-bound workloads are timed) and as back-to-back launches."""
    wl = EmptyKernel(lib)
    g_ms, g_reps = time_workload(wl, steps, 4, graph=True, settle_s=0.05, repeats=repeats)
    e_ms, e_reps = time_workload(wl, steps, 4, graph=False, settle_s=0.05, repeats=repeats)
    return {"graph_us": round(g_ms * 1e3, 3), "eager_us": round(e_ms * 1e3, 3),
            "graph_repeats_us": [round(r * 1e3, 3) for r in g_reps],
            "eager_repeats_us": [round(r * 1e3, 3) for r in e_reps]}


MFMA_CALIB_BLOCKS = 1024  # 4 waves each: 16 waves per CU on 256 CUs
MFMA_CALIB_ITERS = 1024   # 4 MFMAs per iteration and wave


def mfma_peak(lib, repeats=5):
    """fp8 MFMA rate of waves that issue only independent 32x32x64 fp8 MFMAs
    (131072 flops each), median of `repeats` single-launch timings."""
    import torch
    out = torch.empty(MFMA_CALIB_BLOCKS * 256, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    launch = lambda: lib.mqa_calib_mfma_fp8(MFMA_CALIB_BLOCKS, MFMA_CALIB_ITERS, out.data_ptr(),
                                            stream.cuda_stream)
    for _ in range(3):
        assert launch() == 0, "MFMA calibration launch failed"
    torch.cuda.synchronize()
    flops = MFMA_CALIB_BLOCKS * 4 * MFMA_CALIB_ITERS * 4 * 131072
    reps = []
    for _ in range(repeats):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        launch()
        e1.record(stream)
        torch.cuda.synchronize()
        reps.append(flops / (e0.elapsed_time(e1) * 1e-3) / 1e12)
    return {"fp8_TFLOPs": round(float(np.median(reps)), 1),
            "repeats_TFLOPs": [round(r, 1) for r in reps],
            "kernel": "%d workgroups x 4 waves, each %d independent 32x32x64 fp8 MFMAs" % (
                MFMA_CALIB_BLOCKS, MFMA_CALIB_ITERS * 4)}


def parse_tunables(text):
    if not text:
        return None
    from sparse_attention_indexer_scaled_amd import Tunables
    t = Tunables()
    for item in text.split(","):
        k, v = item.split("=")
        setattr(t, k.strip(), int(v))
    return t


def calib_copy(mib):
    """A plain device-to-device copy of known size, for scaling HBM counters."""
    import torch
    n = mib << 20
    a = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"calib_copy_bytes": n, "reads": n, "writes": n}))


PROFILE_DIR = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles")


KERNEL_SOURCES = {
    "decode_kernel": ("device.h", "launch.h", "order_key.h", "api.cpp", "ring.h",
                      "decode_kernel.h", "decode.hip"),
    "prefill_kernel": ("device.h", "launch.h", "api.cpp", "ring.h", "prefill.hip"),
    "topk_kernel": ("device.h", "launch.h", "order_key.h", "api.cpp", "topk.hip"),
    # the fused decode top-k: the decode template's sample and filter modes,
    # then the threshold and select kernels
    "fused_topk": ("device.h", "launch.h", "order_key.h", "api.cpp", "ring.h", "decode_kernel.h",
                   "decode_fused.hip", "topk.hip"),
    "kcache_insert_kernel": ("device.h", "launch.h", "api.cpp", "kcache.hip"),
}


def _code_only(text):
    """Source text without comments and blank lines, so that a profile stays
    valid across comment edits (a '//' inside a string literal is dropped as
    well; that only affects the hash)."""
    import re
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return "\n".join(l.rstrip() for l in text.splitlines() if l.strip())


def source_hash(kernel):
    """Hash of one kernel's sources (with the host launcher that picks its
    launch shape; comments ignored) and the device build flags: a profile is
    only reported while it matches the code being timed."""
    import hashlib
    from sparse_attention_indexer_scaled_amd import build
    h = hashlib.sha256(" ".join(build.DEVICE).encode())
    for name in KERNEL_SOURCES[kernel]:
        with open(os.path.join(build.CSRC, name), encoding="utf-8") as f:
            h.update(name.encode() + _code_only(f.read()).encode())
    return h.hexdigest()[:16]


# Part of the dispatch name that picks a kernel's dispatches out of a
# rocprofv3 run (both prefill kernels, the per-wave and the shared-K one,
# start with "prefill_").
KERNEL_NAME_PART = {"prefill_kernel": "prefill_"}


def kernel_of(workload_name):
    if workload_name.startswith("decode_topk"):
        return "fused_topk"
    for prefix in ("decode", "prefill", "topk", "kcache_insert"):
        if workload_name.startswith(prefix):
            return prefix + "_kernel"
    raise ValueError(workload_name)


def _pmc_avg(csv_dir, counter, name_part):
    """Per-dispatch average of one counter over dispatches whose kernel name
    contains name_part (rocprofv3 --pmc ... --output-format csv)."""
    import csv
    import glob
    vals = {}
    for path in glob.glob(os.path.join(csv_dir, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] == counter and name_part in r["Kernel_Name"]:
                key = (path, r["Dispatch_Id"])
                vals[key] = vals.get(key, 0.0) + float(r["Counter_Value"])
    if not vals:
        raise SystemExit("no %s samples for %r under %s" % (counter, name_part, csv_dir))
    return sum(vals.values()) / len(vals), len(vals)


def write_traffic_profile(workload_name, kernel_part, fetch_dir, write_dir, cal_fetch_dir,
                          cal_write_dir, cal_bytes, command):
    name_part = KERNEL_NAME_PART.get(kernel_part, kernel_part)
    fetch, nf = _pmc_avg(fetch_dir, "FETCH_SIZE", name_part)
    write, nw_ = _pmc_avg(write_dir, "WRITE_SIZE", name_part)
    cfetch, _ = _pmc_avg(cal_fetch_dir, "FETCH_SIZE", "copyBuffer")
    cwrite, _ = _pmc_avg(cal_write_dir, "WRITE_SIZE", "copyBuffer")
    fetch_factor = cal_bytes / (cfetch * 1024)
    write_factor = cal_bytes / (cwrite * 1024)
    out = {"workload": workload_name, "kernel": kernel_part, "source_hash": source_hash(kernel_part),
           "fetch_kib_per_dispatch": round(fetch, 1), "write_kib_per_dispatch": round(write, 1),
           "dispatches": [nf, nw_],
           "calibration": {"copy_bytes": cal_bytes, "fetch_kib": round(cfetch, 1),
                           "write_kib": round(cwrite, 1), "fetch_factor": round(fetch_factor, 4),
                           "write_factor": round(write_factor, 4)},
           "hbm_read_bytes": int(fetch * 1024 * fetch_factor),
           "hbm_write_bytes": int(write * 1024 * write_factor),
           "command": command}
    os.makedirs(PROFILE_DIR, exist_ok=True)
    path = os.path.join(PROFILE_DIR, "%s_traffic.json" % workload_name)
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print(path)


def write_kernel_stats(workload_name, stats_dir, command):
    """Short text summary of a rocprofv3 --kernel-trace --stats run."""
    import csv
    import glob
    paths = glob.glob(os.path.join(stats_dir, "**", "*kernel_stats.csv"), recursive=True)
    if not paths:
        raise SystemExit("no kernel_stats.csv under %s" % stats_dir)
    rows = list(csv.DictReader(open(paths[0])))
    # per-dispatch durations from the kernel trace of the same run, for the median
    durations = {}
    for tp in glob.glob(os.path.join(stats_dir, "**", "*kernel_trace.csv"), recursive=True):
        for t in csv.DictReader(open(tp)):
            durations.setdefault(t["Kernel_Name"], []).append(
                int(t["End_Timestamp"]) - int(t["Start_Timestamp"]))
    lines = ["# rocprofv3 kernel statistics: %s" % workload_name,
             "# command: %s" % command,
             "# source_hash: %s" % source_hash(kernel_of(workload_name)),
             "name | calls | average_ns | median_ns | min_ns | max_ns | percent"]
    for r in rows:
        # drop the argument list: the first "(" that is not part of
        # "(anonymous namespace)"
        full = r["Name"].replace("(anonymous namespace)", "<anon>")
        name = full.split("(")[0].replace("<anon>", "(anonymous namespace)")
        d = durations.get(r["Name"])
        med = "%.1f" % float(np.median(d)) if d else "-"
        lines.append("%s | %s | %.1f | %s | %s | %s | %s" % (
            name, r["Calls"], float(r["AverageNs"]), med, r["MinNs"], r["MaxNs"], r["Percentage"]))
    os.makedirs(PROFILE_DIR, exist_ok=True)
    path = os.path.join(PROFILE_DIR, "%s_kernel_stats.txt" % workload_name)
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print(path)


NUM_SIMDS = 256 * 4   # MI355X: 256 CUs x 4 SIMDs
NUM_XCDS = 8          # GRBM_GUI_ACTIVE is summed over the 8 XCDs
GUI_MIN_DISPATCH_US = 20


def _pmc_dispatches(csv_dir, name_part):
    """{(file, dispatch): {"ns": duration, counter: value}} for dispatches whose
    kernel name contains name_part."""
    import csv
    import glob
    out = {}
    for path in glob.glob(os.path.join(csv_dir, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(path)):
            if name_part not in r["Kernel_Name"]:
                continue
            d = out.setdefault((path, r["Dispatch_Id"]), {})
            d["ns"] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
            d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    return out


def write_counter_profile(workload_name, kernel_part, dirs, command):
    """Per-dispatch averages of SQ/GRBM counters over one or more rocprofv3
    --pmc runs, and what they say about the MFMA and VALU pipes."""
    avg, durations = {}, []
    for d in dirs:
        disp = _pmc_dispatches(d, KERNEL_NAME_PART.get(kernel_part, kernel_part))
        if not disp:
            raise SystemExit("no samples for %r under %s" % (kernel_part, d))
        durations += [v["ns"] for v in disp.values()]
        for name in {k for v in disp.values() for k in v if k != "ns"}:
            vals = [v[name] for v in disp.values() if name in v]
            avg[name] = sum(vals) / len(vals)
    out = {"workload": workload_name, "kernel": kernel_part, "source_hash": source_hash(kernel_part),
           "dispatches": len(durations),
           "median_dispatch_us": round(sorted(durations)[len(durations) // 2] / 1e3, 3),
           "counters_per_dispatch": {k: round(v, 1) for k, v in sorted(avg.items())},
           "command": command}
    derived = {}
    gui = avg.get("GRBM_GUI_ACTIVE")
    if gui and out["median_dispatch_us"] < GUI_MIN_DISPATCH_US:
        # the counter window of a dispatch this short is longer than the
        # dispatch itself, so per-cycle figures would be diluted by idle time
        derived["note"] = ("dispatch under %d us: clock and pipe-busy fractions omitted"
                           % GUI_MIN_DISPATCH_US)
        gui = None
    if gui:
        simd_cycles = NUM_SIMDS * gui / NUM_XCDS
        derived["clock_GHz"] = round(gui / NUM_XCDS / (out["median_dispatch_us"] * 1e3), 3)
        if "SQ_VALU_MFMA_BUSY_CYCLES" in avg:
            derived["mfma_busy_frac"] = round(avg["SQ_VALU_MFMA_BUSY_CYCLES"] / simd_cycles, 4)
        if "SQ_INSTS_VALU" in avg and "SQ_INSTS_MFMA" in avg:
            derived["non_mfma_valu_insts"] = int(avg["SQ_INSTS_VALU"] - avg["SQ_INSTS_MFMA"])
        if avg.get("SQ_VALU_MFMA_BUSY_CYCLES") and "SQ_VALU_MFMA_COEXEC_CYCLES" in avg:
            # share of the MFMA pipe's busy cycles during which VALU work also ran
            derived["valu_coexec_frac_of_mfma_busy"] = round(
                avg["SQ_VALU_MFMA_COEXEC_CYCLES"] / avg["SQ_VALU_MFMA_BUSY_CYCLES"], 4)
    if "SQ_INSTS_VALU_MFMA_MOPS_F8" in avg:
        # one MOPS unit is 512 flops
        derived["mfma_fp8_flops"] = int(avg["SQ_INSTS_VALU_MFMA_MOPS_F8"] * 512)
    hit, miss = avg.get("TCC_HIT_sum"), avg.get("TCC_MISS_sum")
    if hit is not None and miss is not None and hit + miss > 0:
        derived["l2_hit_frac"] = round(hit / (hit + miss), 4)
    if "SQ_INSTS_LDS" in avg:
        derived["lds_insts"] = int(avg["SQ_INSTS_LDS"])
    if "SQ_WAVES" in avg:
        derived["waves"] = int(avg["SQ_WAVES"])
    out["derived"] = derived
    os.makedirs(PROFILE_DIR, exist_ok=True)
    path = os.path.join(PROFILE_DIR, "%s_counters.json" % workload_name)
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print(path)


def read_counters(workload_name):
    path = os.path.join(PROFILE_DIR, "%s_counters.json" % workload_name)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("source_hash") != source_hash(kernel_of(workload_name)):
        return None
    return t["derived"]


def read_traffic(workload_name):
    path = os.path.join(PROFILE_DIR, "%s_traffic.json" % workload_name)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("source_hash") != source_hash(kernel_of(workload_name)):
        return None
    return t["hbm_read_bytes"] + t["hbm_write_bytes"]


def pages_table(args, tun):
    """Our decode on the shapes of the PR page's table (ragged +/- 30 %
    contexts, 32 heads; per-token and preshuffled 64-token blocks), timed as
    the benchmark times its workloads, beside that page's HIP kernel: a markdown
    table and one JSON line of the figures."""
    import torch
    from sparse_attention_indexer_scaled_amd import inputs
    rows = []
    print("| B | next_n | kv_len | block | ours us | page's HIP us | ratio |", flush=True)
    print("|---|---|---|---|---|---|---|", flush=True)
    for idx, (cfg, page_us) in inputs.PAGES_TABLE.items():
        wl = make_workload(idx, False, tun)
        ms, reps = time_workload(wl, args.steps, args.warmup, repeats=args.repeats)
        us = ms * 1e3
        kv_len = int(round((cfg["ctx_range"][0] + cfg["ctx_range"][1]) / 2.0))
        rows.append(dict(workload=cfg["name"], us_per_call=round(us, 3), page_hip_us=page_us,
                         essential_TBps=round(wl.bytes / (us * 1e-6) / 1e12, 4)))
        print("| %d | %d | %d | %d | %.1f | %.1f | %.2fx |" % (
            cfg["B"], cfg["next_n"], kv_len, cfg["block_size"], us, page_us, page_us / us),
            flush=True)
        del wl
        torch.cuda.empty_cache()
    print(json.dumps({"pages_table": rows}))


def main():
    args = parse()
    sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
    if args.write_traffic_profile:
        w, fd, wd, cfd, cwd, mib = args.write_traffic_profile
        kernel = kernel_of(w)
        write_traffic_profile(w, kernel, fd, wd, cfd, cwd, int(mib) << 20, args.profile_command)
        return
    if args.write_counter_profile:
        w, dirs = args.write_counter_profile[0], args.write_counter_profile[1:]
        kernel = kernel_of(w)
        write_counter_profile(w, kernel, dirs, args.profile_command)
        return
    if args.write_kernel_stats:
        write_kernel_stats(args.write_kernel_stats[0], args.write_kernel_stats[1], args.profile_command)
        return
    if args.gpus != 1:
        print("bench.py measures one GPU only: the op shards by sequence or row block "
              "with no exchange between GPUs, so the one-GPU figure is the measurement",
              file=sys.stderr)
        sys.exit(2)
    import torch
    assert torch.cuda.is_available(), "needs a HIP device"
    sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
    from sparse_attention_indexer_scaled_amd import _native
    if not os.path.exists(_native.LIB_PATH):
        from sparse_attention_indexer_scaled_amd import build
        build.build()
    _native.load_library()
    if args.calib_copy:
        calib_copy(args.calib_copy)
        return
    calib = load_calib()
    if args.calib_mfma:
        print(json.dumps(mfma_peak(calib)))
        return

    tun = parse_tunables(args.tunables)
    if args.pages_table:
        pages_table(args, tun)
        return
    order = [args.only] if args.only is not None else [args.workload] + \
        [i for i in (1, 22, 4, 3, 0, 5, 6, 23, 24, 16, 17, 7, 8, 9, 10, 11, 12, 13, 25, 14, 15,
                     18, 19, 20, 21) if i != args.workload]
    results, head, cpu = {}, None, {}
    for idx in order:
        wl = make_workload(idx, args.hot, tun)
        ms, reps = time_workload(wl, args.steps, args.warmup,
                                 graph=False if args.no_graph else None, repeats=args.repeats)
        res = results[wl.cfg["name"]] = summarize(wl, ms, reps)
        if not args.hot and idx in HOT_ALSO and wl.nsets > 1:
            # the same calls on one input copy: what a MALL-resident working set gives
            cold_sets, wl.nsets = wl.nsets, 1
            hms, hreps = time_workload(wl, args.steps, 0, graph=wl.graph, settle_s=0.05,
                                       repeats=args.repeats)
            wl.nsets = cold_sets
            res["hot_us_per_call"] = round(hms * 1e3, 3)
            res["hot_repeats_us"] = [round(r * 1e3, 3) for r in hreps]
            res["hot_essential_TBps"] = round(wl.bytes / (hms * 1e-3) / 1e12, 4)
        counters = read_counters(wl.cfg["name"])
        if counters:
            res["counters"] = counters
        print("[bench] %s: %.2f us/call (repeats %s)" % (
            wl.cfg["name"], ms * 1e3, " ".join("%.2f" % (r * 1e3) for r in reps)),
            file=sys.stderr, flush=True)
        if not args.no_cpu and idx in CPU_BASELINE_RUNS and args.only is None:
            cpu[wl.cfg["name"]] = cpu_baseline_of(wl, CPU_BASELINE_RUNS[idx])
            print("[bench] cpu oracle %s: %.2f s" % (wl.cfg["name"], cpu[wl.cfg["name"]]["seconds"]),
                  file=sys.stderr, flush=True)
        if idx == order[0]:
            head = (wl, ms)
        else:
            del wl
            torch.cuda.empty_cache()
    floor = launch_floor(calib, args.steps, args.repeats)
    peak = mfma_peak(calib)
    print("[bench] launch floor %.2f us (graph) / %.2f us (eager); fp8 MFMA %.0f TFLOP/s" % (
        floor["graph_us"], floor["eager_us"], peak["fp8_TFLOPs"]), file=sys.stderr, flush=True)

    wl, ms = head
    r = results[wl.cfg["name"]]
    h = wl.host
    decode = wl.kind == "decode"
    hbm_bound = wl.kind in ("decode", "topk", "kcache", "fused_topk")
    if wl.kind == "kcache":
        config = {"workload": wl.cfg["name"], "tokens": wl.cfg["tokens"], "cold": not args.hot}
    elif wl.kind == "topk":
        config = {"workload": wl.cfg["name"], "rows": wl.cfg["rows"], "cols": wl.cfg["cols"],
                  "k": wl.k, "cold": not args.hot}
    elif decode or wl.kind == "fused_topk":
        config = {"workload": wl.cfg["name"], "batch": h.B, "next_n": h.next_n,
                  "context": int(h.context_lens.max()), "max_model_len": h.max_model_len,
                  "heads": h.H, "head_dim": h.D, "kv_block_size": h.block_size, "cold": not args.hot}
        if wl.kind == "fused_topk":
            config["k"] = wl.k
    else:
        config = {"workload": wl.cfg["name"], "M": h.M, "N": h.N, "heads": h.H, "head_dim": h.D,
                  "cold": not args.hot}
    line = {
        "metric": "decode essential HBM TB/s (% of 8 TB/s); prefill fp8 TFLOP/s; us/call",
        "value": r["essential_TBps"] if hbm_bound else r["fp8_TFLOPs"],
        "unit": "TB/s" if hbm_bound else "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": wl.warmup_done,
        "ms_per_step": round(ms, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8e4m3 (fp32 accumulate)",
        "data": "synthetic (seeded; N(0,1) Q/K, per-token fp8 K scale, random block table)",
        "config": config,
        "roofline": ({"bound": "hbm", "achieved": round(r["essential_TBps"] * 1e3, 2),
                      "peak": HBM_PEAK_TBS * 1e3, "unit": "GB/s", "frac": r["hbm_frac"],
                      "traffic": read_traffic(wl.cfg["name"])} if hbm_bound else
                     {"bound": "mfma", "achieved": r["fp8_TFLOPs"], "peak": FP8_PEAK_TFLOPS,
                      "unit": "TFLOP/s", "frac": r["mfma_frac"],
                      "peak_measured": peak["fp8_TFLOPs"],
                      "frac_of_measured": round(r["fp8_TFLOPs"] / peak["fp8_TFLOPs"], 4),
                      "traffic": read_traffic(wl.cfg["name"])}),
        "calibration": {"launch_floor": floor, "fp8_mfma_measured": peak},
        "workloads": results,
    }
    for res in results.values():
        if res["timing"] == "hip graph replay":
            res["x_launch_floor"] = round(res["us_per_call"] / floor["graph_us"], 3)
        if "fp8_TFLOPs" in res:
            res["mfma_frac_of_measured"] = round(res["fp8_TFLOPs"] / peak["fp8_TFLOPs"], 4)
    if not args.no_cpu and wl.kind in ("decode", "prefill"):
        line["cpu_baseline"] = cpu.get(wl.cfg["name"]) or cpu_baseline_of(wl, 3)
        if cpu:
            line["cpu_baselines"] = cpu
    print(json.dumps(line))


if __name__ == "__main__":
    main()
