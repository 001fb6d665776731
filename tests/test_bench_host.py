"""bench.py's host logic, without a GPU: the one-GPU refusal, the traffic
file built from counter CSVs (scaled by the plain copy's reading), and the
rule that traffic figures are used only on the kernel sources they were
taken on."""

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
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def _counter_csv(path, counter, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for name, v in rows:
            w.writerow({"Kernel_Name": name, "Counter_Name": counter, "Counter_Value": v})


def test_traffic_scaled_by_the_copy_probe(tmp_path, monkeypatch):
    """FETCH_SIZE reading half of a 1 GiB copy scales reads by 2, WRITE_SIZE
    reading all of it by 1; per kernel the dispatches are averaged; small
    copies (uploads) do not enter the scale."""
    out = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_JSON", str(out))
    amax = "void nc::(anonymous namespace)::k_amax<1>(nc::SegBatch, nc::Tail)"
    cast = "void nc::(anonymous namespace)::k_cast_pt<0, 1, false>(nc::SegBatch, nc_scale_state const*, x)"
    _counter_csv(tmp_path / "f.csv", "FETCH_SIZE",
                 [("__amd_rocclr_copyBuffer", 524288.0), ("__amd_rocclr_copyBuffer", 12.0),
                  (amax, 1048576.0), (amax, 1048580.0), (cast, 1048600.0)])
    _counter_csv(tmp_path / "w.csv", "WRITE_SIZE",
                 [("__amd_rocclr_copyBuffer", 1048576.0), (amax, 2.0), (amax, 2.0), (cast, 1052672.0)])
    bench.write_traffic(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"))
    t = json.loads(out.read_text())
    assert t["source_hash"] == bench.source_hash()
    assert t["scale"]["FETCH_SIZE"]["bytes_per_count_kib"] == pytest.approx(2.0)
    assert t["scale"]["WRITE_SIZE"]["bytes_per_count_kib"] == pytest.approx(1.0)
    a = t["kernels"]["k_amax<1>"]
    assert a["read_bytes"] == round(1024 * 2 * 1048578.0) and a["write_bytes"] == 2048
    assert a["hbm_bytes_per_launch"] == a["read_bytes"] + a["write_bytes"]
    c = t["kernels"]["k_cast_pt<0, 1, false>"]
    assert c["read_bytes"] == round(1024 * 2 * 1048600.0) and c["write_bytes"] == 1024 * 1052672
    # used only on the sources it was taken on
    assert bench.traffic_for("amax", bench.source_hash()) == a["hbm_bytes_per_launch"]
    assert bench.traffic_for("amax", "0" * 16) is None
    assert bench.traffic_for("cast_mx", bench.source_hash()) is None


def test_traffic_needs_the_copy_probe(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "TRAFFIC_JSON", str(tmp_path / "traffic.json"))
    _counter_csv(tmp_path / "f.csv", "FETCH_SIZE", [("k_amax<1>", 1.0)])
    _counter_csv(tmp_path / "w.csv", "WRITE_SIZE", [("k_amax<1>", 1.0)])
    with pytest.raises(SystemExit):
        bench.write_traffic(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"))


def test_committed_traffic_file_names_step_kernels():
    """profiles/traffic.json holds a source hash and bytes for every kernel
    the bench reports beside its name."""
    with open(bench.TRAFFIC_JSON) as f:
        t = json.load(f)
    assert len(t["source_hash"]) == 16
    for call in ("amax", "cast_tensor", "cast_mx", "dequant_pt", "dequant_mx", "stats_pt", "stats_mx"):
        k = t["kernels"][bench.KERNEL_SIG[call]]
        assert k["hbm_bytes_per_launch"] == k["read_bytes"] + k["write_bytes"] > 0
