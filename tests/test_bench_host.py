"""Host-side checks of bench.py's contract (no GPU is touched)."""
import json
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_exits_with_a_message():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert p.returncode == 2
    assert "exactly one GPU" in p.stderr
    assert p.stdout == ""


def test_kernel_fingerprint_follows_the_kernel_sources(tmp_path, monkeypatch):
    csrc = tmp_path / "fp32_gemm_amd" / "csrc"
    csrc.mkdir(parents=True)
    for name in bench.KERNEL_SOURCES:
        shutil.copy(os.path.join(ROOT, "fp32_gemm_amd", "csrc", name), csrc / name)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    first = bench.kernel_fingerprint()
    assert first == bench.kernel_fingerprint()
    # The dispatch table is not kernel code: changing it keeps the counters.
    (csrc / "tuned_table.inc").write_text("// another table\n")
    assert bench.kernel_fingerprint() == first
    with open(csrc / bench.KERNEL_SOURCES[0], "a") as f:
        f.write("\n")
    assert bench.kernel_fingerprint() != first


def test_traffic_records_name_their_summaries():
    with open(os.path.join(ROOT, "profiles", "traffic.json")) as f:
        records = json.load(f)
    assert records
    for key, r in records.items():
        workload, tile = key.split(":")
        assert len(tile.split("/")) == 12, key
        assert r["bytes_per_launch"] == pytest.approx(r["fetch_bytes"] + r["write_bytes"], abs=2), key
        assert os.path.exists(os.path.join(ROOT, "profiles", r["summary"])), key
        assert len(r["kernel"]) == 16, key
