"""Build of the gfx950 HIP library ``liblrs_ssd.so`` (in-tree, no JIT cache)."""
from __future__ import annotations

import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB_PATH = os.path.join(HERE, "liblrs_ssd.so")
SOURCES = ["ssd_kernels.hip", "ssd_ngram.hip", "ssd_api.hip", "ssd_policy.cpp"]
HEADERS = ["ssd_device.h", "ssd_kernels.h", "ssd_ngram.h"]
ARCH = "gfx950"


def hipcc() -> str:
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found; the HIP library cannot be built")
    return exe


def compile_cmd(out: str):
    return [hipcc(), "--offload-arch=%s" % ARCH, "-O3", "-std=c++17", "-fPIC", "-shared",
            "-ffp-contract=off", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", os.path.join(os.path.dirname(HERE), "include"),
            "-o", out] + [os.path.join(CSRC, s) for s in SOURCES]


def build(verbose: bool = False) -> str:
    """Compile every HIP source for gfx950 into ``liblrs_ssd.so`` (always rebuilds)."""
    tmp = LIB_PATH + ".tmp%d" % os.getpid()
    cmd = compile_cmd(tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
