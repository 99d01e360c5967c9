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


def _small_inputs(spec):
    """The workload's recipe at a small shape (the CPU-baseline leg reads the
    shapes from its inputs)."""
    import numpy as np
    import torch

    import oracle
    import workloads

    cfg = spec["cfg"]
    if cfg in (1, 2, 3, 6, 8):
        inp = workloads.workload(cfg, n=24, k=512)
    elif cfg == 4:
        inp = workloads.workload(4, n=16, k=256, m=8)
    elif cfg == 5:
        inp = workloads.workload(5, n=64, k=256)
    elif cfg == 7:
        inp = workloads.workload(7, n=64, k=256)
    elif cfg == 10:
        inp = workloads.workload(10, n=64, k=256)
    elif cfg == 11:
        inp = workloads.workload(11, n=4096)
    elif cfg == 12:
        inp = workloads.workload(12, n=64, k=256)
    else:
        inp = workloads.workload(9, n=64, k=256, m=8)
    if spec["kind"] == "encode":  # the bench dequantizes the weights on the device; here the oracle does
        w = oracle.dequant_rows(oracle.NVFP4, inp["data"], inp["scales"], inp["scale2"], inp["k"], range(inp["n"]))
        inp = dict(inp, Wbits=oracle.bf16_rne_array(w))
    return inp


def test_cpu_baseline_leg_runs_for_every_workload():
    for name, spec in bench.WORKLOADS.items():
        out = bench.cpu_baseline(name, spec, _small_inputs(spec), 0.02)
        assert out["kind"] == "oracle" and out["cores"] == bench.host_cores() >= 1, name
        assert out["value"] > 0 and out["unit"] == spec["unit"], name
        assert isinstance(out["sample"], str) and out["sample"], name
        assert out["one_core"]["cores"] == 1 and out["one_core"]["value"] > 0, name
        assert out["cpu"], name


def test_default_line_is_the_largest_configuration():
    """The headline is the MXFP4 GEMM (2.75e11 flops, 103 MB), with the two
    large decode GEMVs timed alongside."""
    import sys as _sys

    old = _sys.argv
    try:
        _sys.argv = ["bench.py"]
        args = bench.parse()
    finally:
        _sys.argv = old
    assert args.workload == "mxfp4_gemm" and args.gpus == 1
    assert set(args.also) == {"q4k_gemv", "nvfp4_gemv"}
    spec = bench.WORKLOADS[args.workload]
    assert spec["flops"] == 2.0 * 2048 * 8192 * 8192
    assert max(w.get("flops", 0) for w in bench.WORKLOADS.values()) == spec["flops"]
