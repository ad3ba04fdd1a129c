"""The benchmark's host-side contract (CPU only): one GPU per run, and profile
hashes that follow the code but not its comments."""

from __future__ import annotations

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_code_only_drops_comments_and_blank_lines():
    src = "int a; // one\n/* two\n   three */ int b;\n\n   // four\nint c = 1; /* five */\n"
    assert bench._code_only(src) == "int a;\n int b;\nint c = 1;"
    assert bench._code_only(src) == bench._code_only(src.replace("one", "uno"))
    assert bench._code_only(src) != bench._code_only(src.replace("c = 1", "c = 2"))


def test_every_kernel_has_a_source_hash():
    hashes = {k: bench.source_hash(k) for k in bench.KERNEL_SOURCES}
    assert len(set(hashes.values())) == len(hashes)
    assert all(len(h) == 16 for h in hashes.values())
    for w in ("decode_B16_nn6_ctx131072", "prefill_M4096_N32768", "topk_k2048_x",
              "kcache_insert_T4096_fp32", "decode_topk_k2048_x"):
        assert bench.kernel_of(w) in hashes


def _profile_hash(path):
    if path.endswith(".json"):
        import json
        with open(path) as f:
            return json.load(f)["source_hash"]
    with open(path) as f:
        return [l for l in f if l.startswith("# source_hash")][0].split(":", 1)[1].strip()


def test_committed_profiles_match_the_kernel_sources():
    """Every summary under profiles/ was taken from the kernel code as it stands
    (comments aside): a kernel change calls for fresh profiles."""
    pdir = os.path.join(ROOT, "profiles")
    names = sorted(os.listdir(pdir))
    assert names
    for name in names:
        if name.endswith(("_traffic.json", "_counters.json")):
            workload = name[: name.rfind("_")]
        elif name.endswith("_kernel_stats.txt"):
            workload = name[: -len("_kernel_stats.txt")]
        else:
            raise AssertionError("unexpected file under profiles/: %s" % name)
        want = bench.source_hash(bench.kernel_of(workload))
        assert _profile_hash(os.path.join(pdir, name)) == want, "stale profile %s" % name
