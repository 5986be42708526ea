"""Build libwire_demo.so: custom kernels written against include/llar_wire.h
(the device-side primitive API), used by the GPU tests of that API."""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
SRC = os.path.join(HERE, "wire_demo.hip")
LIB = os.path.join(HERE, "libwire_demo.so")


def build(verbose: bool = False) -> str:
    from message_allreduce_amd import _build
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [_build.hipcc(), "--offload-arch=" + _build.ARCH, "-O3", "-std=c++17", "-fPIC", "-shared",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-Wno-unused-command-line-argument",
           "-I", os.path.join(ROOT, "include"), SRC, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed for wire_demo.hip:\n%s\n%s" % (" ".join(cmd), res.stderr[-4000:]))
    os.replace(tmp, LIB)
    if verbose:
        print("built %s" % LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
