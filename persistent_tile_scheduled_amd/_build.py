"""Build step for libtsgemm.so (hipcc, gfx950), kept beside the sources it builds."""

from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(HERE, "csrc", "tsgemm.hip")
OUT = os.path.join(HERE, "libtsgemm.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-shared", "-fPIC",
    # packed fp32 VALU ops are kept off in every HIP build of this project
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", os.path.join(HERE, "csrc"),
]


def build_library(out: str = OUT, verbose: bool = False) -> str:
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [HIPCC] + FLAGS + [SRC, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + r.stderr[-4000:])
    if verbose and r.stderr:
        print(r.stderr[-2000:])
    os.replace(tmp, out)
    return out
