"""Host-side pieces of bench.py that need no GPU: the amd-smi text parser and
the one-GPU guard."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402

# The layout `amd-smi metric -p -c` prints (values made up for the test).
SMI_TEXT = """GPU: 0
    POWER:
        SOCKET_POWER: 1387 W
        GFX_VOLTAGE: N/A
    CLOCK:
        GFX_0:
            CLK: 1910 MHz
            MIN_CLK: 500 MHz
            MAX_CLK: 2400 MHz
        GFX_1:
            CLK: 1797 MHz
            MIN_CLK: 500 MHz
        MEM_0:
            CLK: 2000 MHz
        VCLK_0:
            CLK: 29 MHz
"""


def test_parse_smi_reads_socket_power_and_gfx_clocks_only():
    watts, clks = bench.parse_smi(SMI_TEXT)
    assert watts == 1387.0
    assert clks == [1910.0, 1797.0]  # memory and video clocks are not graphics clocks


def test_parse_smi_without_power_reading():
    assert bench.parse_smi("ERROR: amdgpu not found\n") is None
    assert bench.parse_smi(SMI_TEXT.replace("1387 W", "N/A")) is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_recorded_traffic_matches_the_kernel_sources():
    """The HBM traffic the bench line reports comes from profiles/ only while
    the kernel sources still hash to the value recorded with it; a kernel
    change without new counter runs would leave `roofline.traffic` null."""
    t = bench.recorded_traffic("cfg3_8192_bf16")
    assert t is not None, "profiles/gemm_8192_bf16.md was taken with other kernel sources"
    assert 402.7e6 <= t < 10 * 402.7e6  # at least the algorithmic bytes of A + B + C
    t = bench.recorded_traffic("mx_8192_mxfp8", "mx")
    assert t is not None, "profiles/gemm_8192_mxfp8.md was taken with other kernel sources"
    assert 272.6e6 <= t < 10 * 272.6e6
