"""Build libmqa_indexer.so (the C-ABI HIP library) in-tree with hipcc for gfx950.

    python -m sparse_attention_indexer_scaled_amd.build [--resource-usage]

Flags:
  --offload-arch=gfx950        CDNA4 only, no other targets
  -fno-honor-nans              lets the ReLU lower to one v_max_f32 without an
                               IEEE canonicalize first (both pages, "Technical
                               Details")
  -Xclang -target-feature -Xclang -packed-fp32-ops
                               keep the compiler from forming packed fp32
                               arithmetic (v_pk_fma_f32 and friends)
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libmqa_indexer.so")
CALIB_LIB = os.path.join(PKG, "libmqa_calib.so")
SOURCES = ["api.cpp", "prefill.hip", "decode.hip", "decode_heads.hip", "decode_d64.hip",
           "decode_fused.hip", "decode_fused_d64.hip", "topk.hip", "kcache.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-I", INCLUDE, "-I", CSRC]
DEVICE = ["--offload-arch=gfx950", "-fno-honor-nans", "-mllvm", "-amdgpu-mfma-vgpr-form",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _compile(src: str, out: str, extra) -> None:
    cmd = [HIPCC] + COMMON + DEVICE + list(extra) + ["-c", os.path.join(CSRC, src), "-o", out]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    subprocess.check_call(cmd)


def build(resource_usage: bool = False) -> str:
    bdir = os.path.join(PKG, "_build")
    os.makedirs(bdir, exist_ok=True)
    extra = ["-Rpass-analysis=kernel-resource-usage"] if resource_usage else []
    objs = [os.path.join(bdir, os.path.splitext(s)[0] + ".o") for s in SOURCES]
    with cf.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        list(ex.map(lambda a: _compile(a[0], a[1], extra), zip(SOURCES, objs)))
    tmp = LIB + ".tmp%d" % os.getpid()
    subprocess.check_call([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs)
    os.replace(tmp, LIB)
    build_calib()
    return LIB


def build_calib() -> str:
    """The benchmark's calibration kernels (empty launch, MFMA-only loop) in a
    library of their own, so the op's library holds only the op."""
    tmp = CALIB_LIB + ".tmp%d" % os.getpid()
    subprocess.check_call([HIPCC] + COMMON + DEVICE + ["-shared", os.path.join(CSRC, "calib.hip"),
                                                      "-o", tmp])
    os.replace(tmp, CALIB_LIB)
    return CALIB_LIB


if __name__ == "__main__":
    print(build(resource_usage="--resource-usage" in sys.argv))
