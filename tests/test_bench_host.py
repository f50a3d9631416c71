"""Host logic of bench.py that runs without a GPU: the one-GPU contract and the gate that
reports the decode attention's counter-measured traffic only while the kernel's sources
are the ones the counters were taken on."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused_before_any_device_work():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert p.returncode == 2
    assert "one GPU" in p.stderr
    assert p.stdout == ""


def test_traffic_is_read_from_the_committed_summary_for_the_current_sources():
    """The committed summary names the hash of the sources it was measured on; bench.py
    reports its traffic exactly when that hash is the tree's."""
    vals = {}
    with open(bench.TRAFFIC_FILE) as fh:
        for line in fh:
            if line.strip().startswith("- ") and ":" in line:
                k, v = line.strip()[2:].split(":", 1)
                vals[k.strip()] = v.strip().strip("`")
    if vals.get("source_sha256") != bench.kernel_source_hash():
        pytest.skip("the committed counter summary predates the current kernel sources")
    t = bench.measured_traffic()
    assert t == int(vals["traffic_bytes_per_launch"])
    # fetch + write (each rounded to a byte on its own), and within a few percent of the
    # algorithmic bytes it is compared with
    assert abs(t - int(vals["fetch_bytes_per_launch"]) - int(vals["write_bytes_per_launch"])) <= 1
    assert 1.0 <= t / int(vals["algorithmic_bytes_per_launch"]) < 1.1


def test_traffic_is_withheld_once_a_kernel_source_changes(tmp_path, monkeypatch):
    """A copy of the sources with one byte more hashes differently, so the traffic of the
    committed summary is not reported for it."""
    copies = []
    for f in bench.TRAFFIC_SOURCES:
        dst = tmp_path / os.path.basename(f)
        shutil.copy(f, dst)
        copies.append(str(dst))
    monkeypatch.setattr(bench, "TRAFFIC_SOURCES", copies)
    same = bench.kernel_source_hash()
    with open(copies[0], "a") as fh:
        fh.write("\n")
    assert bench.kernel_source_hash() != same
    assert bench.measured_traffic() is None


def test_missing_summary_gives_no_traffic(monkeypatch, tmp_path):
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "absent.md"))
    assert bench.measured_traffic() is None
