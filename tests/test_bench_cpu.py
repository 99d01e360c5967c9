"""bench.py host logic: the one-GPU contract and the source-hash gate on the
recorded HBM traffic (no GPU needed)."""
import json
import os
import shutil
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_recorded_traffic_present_for_every_workload():
    with open(os.path.join(ROOT, "profiles", "traffic.json")) as f:
        rec = json.load(f)
    assert set(rec) == set(bench.WORKLOADS)
    for name, r in rec.items():
        assert r["traffic_bytes"] > 0 and os.path.exists(os.path.join(ROOT, r["profile"]))


def test_recorded_traffic_is_dropped_when_a_kernel_source_changes(tmp_path, monkeypatch):
    name = "nvfp4_gemv"
    with open(os.path.join(ROOT, "profiles", "traffic.json")) as f:
        rec = json.load(f)[name]
    # a copy of the repository pieces the gate reads, with one source byte changed
    (tmp_path / "profiles").mkdir()
    shutil.copy(os.path.join(ROOT, "profiles", "traffic.json"), tmp_path / "profiles" / "traffic.json")
    for rel in rec["source"]:
        dst = tmp_path / rel
        dst.parent.mkdir(parents=True, exist_ok=True)
        shutil.copy(os.path.join(ROOT, rel), dst)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    unchanged = bench.recorded_traffic(name)
    with open(tmp_path / rec["source"][0], "ab") as f:
        f.write(b"\n// edited\n")
    changed = bench.recorded_traffic(name)
    assert unchanged == rec["traffic_bytes"] or unchanged is None  # None if the tree itself changed since
    assert changed is None
