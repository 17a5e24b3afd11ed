"""Ahead-of-time build of libpmqa_calib.so for gfx950: the page-gather
read-rate kernel (csrc/calib.hip) that bench.py --read-calibration runs.  A
measurement tool, kept out of libpmqa.so and built with the same compiler and
flags."""
from __future__ import annotations

import importlib.util
import os
import subprocess

# build.py by path (this file may run as a script or be loaded by path)
_spec = importlib.util.spec_from_file_location(
    "_pmqa_build_flags", os.path.join(os.path.dirname(os.path.abspath(__file__)), "build.py"))
_b = importlib.util.module_from_spec(_spec)
_spec.loader.exec_module(_b)

SOURCE = os.path.join(_b.CSRC, "calib.hip")
LIB = os.path.join(_b.PKG, "libpmqa_calib.so")


def build() -> str:
    """Compile calib.hip and link libpmqa_calib.so (always rebuilds)."""
    cc = _b.hipcc()
    os.makedirs(_b.BUILD_DIR, exist_ok=True)
    obj = os.path.join(_b.BUILD_DIR, "calib.hip.o")
    cmd = [cc] + _b.compile_flags("calib.hip") + ["-c", SOURCE, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for calib.hip:\n%s\n%s" % (" ".join(cmd), r.stderr))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [cc, "--offload-arch=" + _b.ARCH, "-shared", "-fPIC", "-o", tmp, obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (" ".join(cmd), r.stderr))
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
