"""Host-side parts of bench.py (no GPU): the refusal of more than one GPU, the
algorithmic byte count of the headline GEMV, and the launch geometry it
reports for the measured kernel."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_headline_algorithmic_bytes():
    # packed weights N*K/4 + int8 x K + bf16 y 2N + fp32 s + two bf16 weight scales
    assert bench.gemv_bytes(1, 13824, 2560, 2) == 13824 * 2560 // 4 + 2560 + 2 * 13824 + 4 + 4
    assert bench.gemv_bytes(1, 13824, 2560, 2) == 8877576
    # bf16 activations count twice the activation bytes
    assert bench.gemv_bytes(1, 13824, 2560, 2, x_bytes=2) == 8877576 + 2560


def test_reported_geometry():
    # (bands per workgroup, wavefronts per workgroup, steps per wavefront)
    assert bench.gemv_geometry(13824, 2560) == (4, 4, 10)     # the headline
    assert bench.gemv_geometry(2560, 2560) == (1, 4, 3)       # narrow: runs of at most 4
    assert bench.gemv_geometry(6912, 2560) == (2, 4, 5)       # 400-767 bands: runs of at most 5
    assert bench.gemv_geometry(2560, 13824) == (1, 8, 7)      # at most 8 wavefronts per band
    assert bench.gemv_geometry(20, 61440) == (1, 16, 15)      # unless runs would exceed 15
