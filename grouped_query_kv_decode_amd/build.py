"""Builds libgqa.so (HIP kernels + C ABI) for gfx950 in-tree.

    python -m grouped_query_kv_decode_amd.build

hipcc cross-compiles, so this runs on a machine without a GPU.
"""
from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libgqa.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

COMMON = [
    "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
    "-I" + INCLUDE, "-I" + CSRC,
    # no packed-FP32 instructions: generate scalar FP32 arithmetic only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]

# (source, extra flags)
SOURCES = [
    # keep MFMA accumulators in VGPRs: the softmax rescale then needs no
    # AGPR<->VGPR copies in the streaming loop
    ("gqa_decode_mfma.hip", ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]),
    ("gqa_decode_mfma_f32.hip", ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]),
    ("gqa_decode_valu.hip", []),
    ("gqa_merge.hip", []),
    ("gqa_order.hip", []),
    ("gqa_stream.hip", []),
    ("gqa_linear.hip", ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]),
    ("gqa_linear_packed.hip", ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]),
    # bit-exact conversion arithmetic: no contraction of any kind
    ("gqa_meanpool.hip", ["-ffp-contract=off"]),
    ("gqa_api.hip", []),
]


def _compile(src: str, extra) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *COMMON, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (src, " ".join(cmd), res.stderr))
    # the host pass warns that it does not know the packed-fp32 feature; drop that noise
    noise = ("packed-fp32-ops", "is not a recognized feature", "warning generated", "warnings generated")
    err = "\n".join(x for x in res.stderr.splitlines() if x.strip() and not any(n in x for n in noise))
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


def build(verbose: bool = True) -> str:
    """Compile every HIP source and link libgqa.so; returns its path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda s: _compile(*s), SOURCES))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (" ".join(cmd), res.stderr))
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build()
