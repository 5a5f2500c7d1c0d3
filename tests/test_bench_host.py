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


@pytest.mark.parametrize("path", ["fwd", "bwd", "fa1", "decode"])
def test_kernel_sha_covers_the_kernel_sources_and_changes_with_them(tmp_path, monkeypatch, path):
    base = bench.kernel_sha(path)
    assert len(base) == 64
    copies = {}
    for k, files in bench.KERNEL_SOURCES.items():
        copies[k] = []
        for p in files:
            q = tmp_path / k / os.path.basename(p)
            q.parent.mkdir(exist_ok=True)
            q.write_bytes(open(p, "rb").read())
            copies[k].append(str(q))
    monkeypatch.setattr(bench, "KERNEL_SOURCES", copies)
    assert bench.kernel_sha(path) == base
    with open(copies[path][0], "ab") as f:
        f.write(b"\n// edited\n")
    assert bench.kernel_sha(path) != base


def test_each_path_hashes_its_own_kernel_file():
    files = {k: os.path.basename(v[0]) for k, v in bench.KERNEL_SOURCES.items()}
    assert files == {"fwd": "fa2_fwd_gfx950.hip", "bwd": "fa2_bwd_gfx950.hip",
                     "fa1": "fa1_fwd_gfx950.hip", "decode": "fa2_splitkv_gfx950.hip"}
    assert len({bench.kernel_sha(k) for k in files}) == 4


def test_traffic_is_reported_only_for_the_source_it_was_measured_on(tmp_path, monkeypatch):
    t = {"workloads": {"ref": {"kernel_sha256": bench.kernel_sha("fwd"), "hbm_bytes_per_launch": 123456},
                       "bwd:ref": {"kernel_sha256": bench.kernel_sha("bwd"), "hbm_bytes_per_launch": 7},
                       "decode:decode_64k": {"kernel_sha256": "0" * 64, "hbm_bytes_per_launch": 9}}}
    f = tmp_path / "traffic.json"
    f.write_text(json.dumps(t))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.measured_traffic("fwd", "ref") == 123456
    assert bench.measured_traffic("bwd", "ref") == 7
    assert bench.measured_traffic("decode", "decode_64k") is None   # other source
    assert bench.measured_traffic("fwd", "hd128_16k") is None       # not measured
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "missing.json"))
    assert bench.measured_traffic("fwd", "ref") is None


def test_counter_summary_from_rocprof_csvs(tmp_path):
    """A synthetic rocprofv3 layout: the copy calibration and a two-kernel
    backward call; bytes are summed over the call's kernels and scaled."""
    def write(sub, rows):
        d = tmp_path / sub / "host"
        d.mkdir(parents=True)
        with open(d / "x_counter_collection.csv", "w") as fh:
            fh.write("Kernel_Name,Counter_Value\n")
            for name, val in rows:
                fh.write(f"{name},{val}\n")
    write("copy_FETCH_SIZE", [("__amd_rocclr_copyBuffer", 262144.0)] * 5)
    write("copy_WRITE_SIZE", [("__amd_rocclr_copyBuffer", 524288.0)] * 5)
    write("pmc_bwd_ref_FETCH_SIZE", [("fa2_bwd_dq_kernel<64>", 100.0), ("fa2_bwd_dkdv_stream_kernel<64>", 50.0)] * 3)
    write("pmc_bwd_ref_WRITE_SIZE", [("fa2_bwd_dq_kernel<64>", 10.0), ("fa2_bwd_dkdv_kernel<64>", 20.0)] * 3)
    res = bench.summarize_counters(str(tmp_path))
    assert res["calibration"]["fetch_factor"] == 2.0 and res["calibration"]["write_factor"] == 1.0
    e = res["workloads"]["bwd:ref"]
    assert e["hbm_read_bytes"] == 150 * 1024 * 2 and e["hbm_write_bytes"] == 30 * 1024
    assert e["kernel_sha256"] == bench.kernel_sha("bwd")


def test_committed_traffic_summary_is_well_formed():
    with open(bench.TRAFFIC_FILE) as f:
        t = json.load(f)
    cal = t["calibration"]
    assert cal["fetch_factor"] > 0 and cal["write_factor"] > 0
    for name, w in t["workloads"].items():
        assert len(w["kernel_sha256"]) == 64, name
        assert w["hbm_bytes_per_launch"] == w["hbm_read_bytes"] + w["hbm_write_bytes"], name
        assert w["ratio_to_algorithmic"] == pytest.approx(
            w["hbm_bytes_per_launch"] / w["algorithmic_bytes"], rel=1e-3), name


@pytest.mark.parametrize("argv", [["--workload", "decode_64k", "--pass", "bwd"],
                                  ["--workload", "decode_64k", "--impl", "fa1"],
                                  ["--impl", "fa1", "--pass", "bwd"],
                                  ["--impl", "fa1", "--workload", "ref_d128"]])
def test_meaningless_flag_combinations_are_rejected(argv):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *argv], capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 2 and "error" in r.stderr and r.stdout == ""
