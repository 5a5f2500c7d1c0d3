"""Host-side logic of bench.py (no GPU): the one-GPU guard, the kernel-source
hash that keys the committed HBM counter summary, and the traffic lookup."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


@pytest.mark.parametrize("n", [0, 2, 8])
def test_more_than_one_gpu_exits_with_a_message(n):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", str(n)],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""


def test_world_size_above_one_exits():
    env = dict(os.environ, WORLD_SIZE="2")
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")], capture_output=True,
                       text=True, timeout=120, env=env)
    assert r.returncode == 2 and "one GPU only" in r.stderr


def test_kernel_sha_covers_the_kernel_sources_and_changes_with_them(tmp_path, monkeypatch):
    base = bench.kernel_sha()
    assert len(base) == 64
    copies = []
    for p in bench.KERNEL_SOURCES:
        q = tmp_path / os.path.basename(p)
        q.write_bytes(open(p, "rb").read())
        copies.append(str(q))
    monkeypatch.setattr(bench, "KERNEL_SOURCES", copies)
    assert bench.kernel_sha() == base
    with open(copies[0], "ab") as f:
        f.write(b"\n// edited\n")
    assert bench.kernel_sha() != base


def test_traffic_is_reported_only_for_the_source_it_was_measured_on(tmp_path, monkeypatch):
    t = {"kernel_sha256": bench.kernel_sha(),
         "workloads": {"ref": {"hbm_bytes_per_launch": 123456}}}
    f = tmp_path / "traffic.json"
    f.write_text(json.dumps(t))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.measured_traffic("ref") == 123456
    assert bench.measured_traffic("hd128_16k") is None
    t["kernel_sha256"] = "0" * 64
    f.write_text(json.dumps(t))
    assert bench.measured_traffic("ref") is None
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "missing.json"))
    assert bench.measured_traffic("ref") is None


def test_committed_traffic_summary_is_well_formed():
    with open(bench.TRAFFIC_FILE) as f:
        t = json.load(f)
    assert len(t["kernel_sha256"]) == 64
    cal = t["calibration"]
    assert cal["fetch_factor"] > 0 and cal["write_factor"] > 0
    for name, w in t["workloads"].items():
        assert w["hbm_bytes_per_launch"] == w["hbm_read_bytes"] + w["hbm_write_bytes"], name
        assert w["ratio_to_algorithmic"] == pytest.approx(
            w["hbm_bytes_per_launch"] / w["algorithmic_bytes"], rel=1e-3), name
