"""Build libcsa.so (hand-written HIP for gfx950) in-tree with hipcc.

    python -m long_context_compressed_04_amd.build_lib

Every HIP source is compiled for gfx950 only, with packed-FP32 instructions
disabled, then linked into ``long_context_compressed_04_amd/libcsa.so``.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libcsa.so")
BUILD = os.path.join(PKG, "_build")

SOURCES = ["compress.hip", "indexer.hip", "topk.hip", "mqa.hip", "csa_api.cpp", "validate.cpp", "launch_timer.cpp", "noalloc.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", INCLUDE, "-I", CSRC]


# Per-source options.  MFMA results go to ordinary VGPRs in the indexer and the MQA
# kernels: an epilogue reads every accumulator once, and from AGPRs each read is one
# more instruction (v_accvgpr_read), behind a wait for the matrix pipe before the
# registers are reused.  Every kernel keeps its occupancy or gains; the decode and
# prefill MQA kernels compile to the same code either way.  The top-k and indexer
# sources use LLVM's ILP-first machine scheduler (same-box A/B: csa_decode_64k step
# 33.21 -> 33.07 us, csa_decode_1m_fp4 35.03 -> 34.76 us, prefill unchanged); on the
# MQA source it adds spills, so that source keeps the default scheduler.
_ILP = ["-mllvm", "-amdgpu-sched-strategy=max-ilp"]
SOURCE_FLAGS = {
    "indexer.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"] + _ILP,
    "mqa.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
    "topk.hip": _ILP,
}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    lang = ["-x", "hip"] if src.endswith(".cpp") else []
    cmd = [HIPCC] + FLAGS + SOURCE_FLAGS.get(src, []) + lang + ["-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s" % (src, res.stderr))
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("link failed:\n%s" % res.stderr)
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
