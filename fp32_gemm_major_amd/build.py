"""Compile the HIP library ``libsgemm.so`` in place for gfx950.

    python -m fp32_gemm_major_amd.build

The library is plain HIP (no torch symbols); hipcc cross-compiles it on a
machine without a GPU.  Packed FP32 arithmetic is switched off for every HIP
source (``-packed-fp32-ops``): the VALU kernel then uses one v_fma_f32 per
multiply-add.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIBRARY = os.path.join(PKG, "libsgemm.so")
SOURCES = [os.path.join(CSRC, "sgemm.hip")]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def command(output: str = LIBRARY, extra=()) -> list:
    return [HIPCC, *FLAGS, *extra, "-o", output, *SOURCES]


def build(output: str = LIBRARY, verbose: bool = False) -> str:
    tmp = output + ".tmp%d" % os.getpid()
    cmd = command(tmp)
    proc = subprocess.run(cmd, capture_output=True, text=True)
    if proc.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + " ".join(cmd) + "\n" + proc.stderr)
    if verbose and proc.stderr:
        sys.stderr.write(proc.stderr)
    os.replace(tmp, output)
    return output


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
