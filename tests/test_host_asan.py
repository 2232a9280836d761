"""Host AddressSanitizer run of the C ABI (CPU only, opt-in: TSGEMM_ASAN_TEST=1).

Builds libtsgemm with the host half of every translation unit instrumented
(the device code is not: GPU sanitizers are not used here), then runs the host
ABI tests (plan creation and validation, error codes, launch geometry, the host
scheduler against the oracle, the worker numbering) in a child process against
that build with the ASan runtime preloaded.  Any heap or stack error in the
host code fails the child.  Takes about a minute, so it is not part of the
default CPU run.
"""

import glob
import os
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

pytestmark = pytest.mark.skipif(os.environ.get("TSGEMM_ASAN_TEST") != "1",
                                reason="opt-in: set TSGEMM_ASAN_TEST=1")


def test_host_abi_under_address_sanitizer():
    sys.path.insert(0, ROOT)
    from persistent_tile_scheduled_amd import _build
    runtimes = glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
    if not runtimes:
        pytest.skip("no clang ASan runtime in /opt/rocm/llvm")
    with tempfile.TemporaryDirectory() as d:
        lib = os.path.join(d, "libtsgemm_asan.so")
        _build.build_library(out=lib, extra_flags=["-Xarch_host", "-fsanitize=address",
                                                   "-Xarch_host", "-fno-omit-frame-pointer"])
        syms = subprocess.run(["nm", "-D", lib], capture_output=True, text=True).stdout
        assert "__asan_report" in syms, "the host code was not instrumented"
        env = dict(os.environ, TSGEMM_LIB=lib, LD_PRELOAD=runtimes[0],
                   ASAN_OPTIONS="detect_leaks=0:abort_on_error=1")
        env.pop("TSGEMM_ASAN_TEST", None)
        r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-m", "not gpu", "-p", "no:cacheprovider",
                            os.path.join(ROOT, "tests", "test_abi_host.py")],
                           cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
        assert r.returncode == 0, (r.stdout[-3000:] + r.stderr[-3000:])
        assert "passed" in r.stdout
