"""Ahead-of-time build of libpmqa.so for gfx950 with hipcc.

Every HIP source is compiled for gfx950 only, with packed-FP32 instruction
selection disabled, into a shared library placed next to this file.
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libpmqa.so")
BUILD_DIR = os.path.join(ROOT, "_build")
SOURCES = ["api.hip", "mqa_logits.hip", "mqa_any.hip", "indexer.hip", "proxy.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for c in (os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc"),
              shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found: the gfx950 library cannot be built")


# Per-source extras.  The logits kernels: MFMA results in VGPRs (no copies out
# of accumulation registers), and no NaN semantics for arithmetic so the
# rectifier is one v_max_f32 (NaN outputs are written as bit patterns there).
_LOGITS_FLAGS = ["-fno-honor-nans", "-mllvm", "-amdgpu-mfma-vgpr-form"]
EXTRA_FLAGS = {"mqa_logits.hip": _LOGITS_FLAGS, "mqa_any.hip": _LOGITS_FLAGS,
               "proxy.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def compile_flags(src=None):
    return (["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-Wall",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-I", INCLUDE, "-I", CSRC] + EXTRA_FLAGS.get(src, []))


def build(verbose: bool = False) -> str:
    """Compile every HIP source and link libpmqa.so (always rebuilds)."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    cc = hipcc()

    def one(src):
        obj = os.path.join(BUILD_DIR, src + ".o")
        cmd = [cc] + compile_flags(src) + ["-c", os.path.join(CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (src, " ".join(cmd), r.stderr))
        if verbose and r.stderr.strip():
            print(r.stderr)
        return obj

    with concurrent.futures.ThreadPoolExecutor(len(SOURCES)) as ex:
        objs = list(ex.map(one, SOURCES))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [cc, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (" ".join(cmd), r.stderr))
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
