"""Build step for libtsgemm.so (hipcc, gfx950), kept beside the sources it builds.

The kernels are split over translation units that compile in parallel: the
host code (tsgemm.hip), one unit per fp16/bf16 dtype and tile shape
(tsgemm_gemm_tu.hip with -DTSG_TU_*), and the block-scaled FP8 unit
(tsgemm_mx_tu.hip).  The objects are linked into one shared library.
"""

from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libtsgemm.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 VALU ops are kept off in every HIP build of this project
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]

# (source, extra defines, object name)
GEMM_TUS = [(dt, bm, bk) for dt in (1, 2) for bm in (128, 256) for bk in (32, 64)]
UNITS = ([("tsgemm.hip", [], "host.o"), ("tsgemm_mx_tu.hip", [], "mx.o")] +
         [("tsgemm_gemm_tu.hip", [f"-DTSG_TU_DT={dt}", f"-DTSG_TU_BM={bm}", f"-DTSG_TU_BK={bk}"],
           f"gemm_{dt}_{bm}_{bk}.o") for dt, bm, bk in GEMM_TUS])


def _jobs() -> int:
    n = os.cpu_count() or 4
    cap = int(os.environ.get("MAX_JOBS", "16"))
    return max(1, min(n, cap, len(UNITS)))


STRESS_OUT = os.path.join(HERE, "libtsgemm_stress.so")


def build_stress_library(out: str = STRESS_OUT) -> str:
    """The race-detection build (-DTSG_STRESS=1: random pauses at every barrier
    and DMA).  Tests run against it with TSGEMM_LIB=<this file>."""
    return build_library(out=out, extra_flags=["-DTSG_STRESS=1"])


def build_library(out: str = OUT, verbose: bool = False, extra_flags=()) -> str:
    """Compile every unit (in parallel) and link libtsgemm.so at `out`.
    `extra_flags` are added to every compile (e.g. -D switches of a variant build)."""
    tmpdir = tempfile.mkdtemp(prefix="tsgemm_build_")
    try:
        def compile_one(unit):
            src, defs, obj = unit
            cmd = [HIPCC] + FLAGS + list(extra_flags) + defs + ["-c", os.path.join(CSRC, src),
                                                                "-o", os.path.join(tmpdir, obj)]
            r = subprocess.run(cmd, capture_output=True, text=True)
            return unit, r

        with concurrent.futures.ThreadPoolExecutor(_jobs()) as ex:
            results = list(ex.map(compile_one, UNITS))
        for (src, defs, _), r in results:
            if r.returncode != 0:
                raise RuntimeError(f"hipcc failed on {src} {' '.join(defs)}:\n" + r.stderr[-4000:])
            if verbose and r.stderr:
                print(r.stderr[-2000:])
        tmp = out + ".tmp%d" % os.getpid()
        cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC"] + \
            [os.path.join(tmpdir, obj) for _, _, obj in UNITS] + ["-o", tmp]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError("link failed:\n" + r.stderr[-4000:])
        os.replace(tmp, out)
    finally:
        shutil.rmtree(tmpdir, ignore_errors=True)
    return out


if __name__ == "__main__":
    import sys
    print(build_stress_library() if "--stress" in sys.argv[1:] else build_library())
