"""Host-side parts of bench.py that need no GPU: the one-GPU refusal, the algorithmic byte model,
and the conversion of rocprofv3 FETCH_SIZE / WRITE_SIZE counters into HBM bytes per launch."""
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)


def test_algorithmic_bytes():
    n = 3840 * 2160
    nc = 1920 * 1080
    # 8-bit: the six planes of 50 pairs once, the blurred uint16 state in and out (4 bytes/pixel)
    assert bench.algorithmic_bytes(3840, 2160, 8, 50) == 50 * 2 * (n + 2 * nc) + 4 * n
    assert bench.algorithmic_bytes(3840, 2160, 8, 50) == 1_277_337_600
    # 10-bit samples take two bytes
    assert bench.algorithmic_bytes(3840, 2160, 10, 50) == 2_521_497_600
    # motion v2 carries the raw reference luma (one sample per pixel each way)
    assert bench.algorithmic_bytes(3840, 2160, 8, 50, True) == 50 * 2 * (n + 2 * nc) + 2 * n
    # odd sizes round the chroma planes up
    assert bench.algorithmic_bytes(5, 3, 8, 1) == 2 * (15 + 2 * 6) + 4 * 15


def _counter_csv(path, counter, main_kib, copy_kib):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for v in main_kib:
            w.writerow({"Kernel_Name": "void iir::frames_kernel<8, 16>(iir::KernelArgs)",
                        "Counter_Name": counter, "Counter_Value": v})
        for v in copy_kib:
            w.writerow({"Kernel_Name": "void iir::probe_copy<4>(...)", "Counter_Name": counter,
                        "Counter_Value": v})
        # rows of another counter and another kernel are ignored
        w.writerow({"Kernel_Name": "void iir::frames_kernel<8, 16>(iir::KernelArgs)",
                    "Counter_Name": "OTHER", "Counter_Value": 1e9})
        w.writerow({"Kernel_Name": "fill", "Counter_Name": counter, "Counter_Value": 1e9})


def test_traffic_from_counters(tmp_path):
    """The counters are scaled by what they read for the copy probe, whose bytes are known: a
    probe that reads as twice its size halves every reading."""
    gib_kib = bench.PROBE_BYTES / 1024.0
    fetch = tmp_path / "fetch.csv"
    write = tmp_path / "write.csv"
    _counter_csv(fetch, "FETCH_SIZE", [1000.0, 3000.0], [2 * gib_kib])
    _counter_csv(write, "WRITE_SIZE", [500.0], [gib_kib, gib_kib])
    d = bench.write_traffic("c3", False, False, str(fetch), str(write), out_dir=str(tmp_path))
    assert d["fetch_kib_per_launch"] == 2000.0 and d["fetch_dispatches"] == 2
    assert d["fetch_scale"] == pytest.approx(0.5)
    assert d["write_scale"] == pytest.approx(1.0)
    assert d["hbm_fetch_bytes_per_launch"] == pytest.approx(2000.0 * 1024 * 0.5)
    assert d["hbm_write_bytes_per_launch"] == pytest.approx(500.0 * 1024)
    assert d["hbm_bytes_per_launch"] == pytest.approx(1000.0 * 1024 + 500.0 * 1024)
    assert d["algorithmic_bytes_per_launch"] == 1_277_337_600
    assert d["kernel_sha256"] == bench.kernel_sha()
    saved = json.loads((tmp_path / "frames_kernel_c3_traffic.json").read_text())
    assert saved["hbm_bytes_per_launch"] == d["hbm_bytes_per_launch"]


def test_traffic_needs_both_kernels(tmp_path):
    p = tmp_path / "only_main.csv"
    _counter_csv(p, "FETCH_SIZE", [1.0], [])
    with pytest.raises(SystemExit):
        bench.write_traffic("c3", False, False, str(p), str(p), out_dir=str(tmp_path))


def test_kernel_hash_ignores_comments_only():
    """The traffic counters stay valid across comment edits, and not across code edits."""
    base = "int f(int a) {\n    return a + 1;  // one more\n}\n/* block\n comment */\n"
    assert bench._code_only(base) == bench._code_only(base.replace("one more", "the next"))
    assert bench._code_only(base) == bench._code_only(base.replace("/* block", "/* other"))
    assert bench._code_only(base) == bench._code_only(base.replace("    return", "  return"))
    assert bench._code_only(base) != bench._code_only(base.replace("a + 1", "a + 2"))


def test_committed_traffic_summaries_match_the_kernel_code():
    """Every committed counter summary was taken on the frames kernel's current code, so the
    benchmark line reports its traffic (a stale summary would make it report null)."""
    import glob
    paths = sorted(glob.glob(os.path.join(bench.ROOT, "profiles", "frames_kernel_*_traffic.json")))
    assert paths
    for p in paths:
        with open(p) as f:
            d = json.load(f)
        assert d["kernel_sha256"] == bench.kernel_sha(), os.path.basename(p)
        assert 1.0 <= d["hbm_bytes_per_launch"] / d["algorithmic_bytes_per_launch"] < 1.5, p
