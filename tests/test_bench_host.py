"""Host-side parts of bench.py (no GPU): the refusal of more than one GPU, the
algorithmic byte count of the headline GEMV, the launch geometry it
reports for the measured kernel, and its summary of rocprofv3 databases."""
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


def test_summarize_profile(tmp_path, capsys):
    # a database with the rocpd tables the summary reads: per-kernel durations,
    # the last 400 dispatches of a kernel with at least 800, and counters with
    # their largest values (the calibration copies)
    import sqlite3
    d = tmp_path / "run" / "host"
    d.mkdir(parents=True)
    db = sqlite3.connect(str(d / "pmc_results.db"))
    db.execute("create table kernels (name text, start integer, end integer)")
    db.execute("create table counters_collection (kernel_name text, counter_name text, value real)")
    rows = [("k_long", 1000 * i, 1000 * i + 400) for i in range(800)]
    rows += [("k_long", 800000 + 100 * i, 800000 + 100 * i + 90) for i in range(400)]
    rows += [("copy", 10 ** 7 + 10 * i, 10 ** 7 + 10 * i + 5) for i in range(3)]
    db.executemany("insert into kernels values (?, ?, ?)", rows)
    db.executemany("insert into counters_collection values (?, ?, ?)",
                   [("copy", "FETCH_SIZE", v) for v in (1.5, 131083.5, 131084.5)] +
                   [("k_long", "FETCH_SIZE", 4371.0)] * 10)
    db.commit()
    db.close()
    bench.summarize_profile(str(tmp_path))
    out = capsys.readouterr().out
    lines = out.splitlines()
    assert any(l.startswith("k_long | 1200 |") for l in lines)
    # the last 400: durations 90 ns, back to back every 100 ns
    last = [l for l in lines if l.startswith("## last 400 dispatches: k_long")]
    assert last and last[0].endswith("| 400 | 90.0 | 90 | 90 | 90 | 90 | 100")
    fetch = [l for l in lines if l.startswith("copy | FETCH_SIZE")]
    assert fetch and fetch[0].endswith("| 131084.5, 131083.5, 1.5")
