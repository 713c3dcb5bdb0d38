"""Host logic of bench.py (no GPU): the one-GPU guard, the comment-blind
kernel source hash, and the HBM-traffic record written from rocprofv3
counter CSVs and read back only for the kernel source it was taken on."""
import csv
import json
import os
import subprocess
import sys

import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_code_only_ignores_comments_and_blank_lines():
    a = "int f(int x) {\n  // the value\n  return x + 1;  /* plus one */\n}\n"
    b = "/* header\n   lines */\nint f(int x) {\n\n  return x + 1;\n}  // end\n"
    c = "int f(int x) {\n  return x + 2;\n}\n"
    assert bench._code_only(a) == bench._code_only(b)
    assert bench._code_only(a) != bench._code_only(c)


def test_kernel_source_hash_follows_code_not_comments(tmp_path):
    src = tmp_path / "k.hpp"
    src.write_text("// v1\nint k() { return 1; }\n")
    h1 = bench.kernel_source_hash([str(src)])
    src.write_text("// v2, reworded\nint k() { return 1; }  // same code\n")
    assert bench.kernel_source_hash([str(src)]) == h1
    src.write_text("int k() { return 2; }\n")
    assert bench.kernel_source_hash([str(src)]) != h1


def _write_counter_csv(path, rows):
    os.makedirs(path, exist_ok=True)
    with open(os.path.join(path, "p_counter_collection.csv"), "w", newline="") as f:
        wr = csv.writer(f)
        wr.writerow(["Kernel_Name", "Counter_Name", "Counter_Value"])
        for r in rows:
            wr.writerow(r)


def test_traffic_record_round_trip(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "traffic.json"))
    kib = 1024
    # a 256 MiB copy: FETCH_SIZE reads half the bytes, WRITE_SIZE all of them
    _write_counter_csv(tmp_path / "cf", [("__amd_rocclr_copyBuffer", "FETCH_SIZE", 128 * kib)])
    _write_counter_csv(tmp_path / "cw", [("__amd_rocclr_copyBuffer", "WRITE_SIZE", 256 * kib)])
    # three dispatches of the forward kernel: median 50 MiB fetched, 20 MiB written (as counted)
    name = "_ZN2fa15fa_fwd16_kernelIL..."
    _write_counter_csv(tmp_path / "f", [(name, "FETCH_SIZE", v * kib) for v in (49, 50, 60)])
    _write_counter_csv(tmp_path / "w", [(name, "WRITE_SIZE", v * kib) for v in (20, 20, 21)])
    ent = bench.write_traffic("wl", str(tmp_path / "f"), str(tmp_path / "w"), str(tmp_path / "cf"),
                              str(tmp_path / "cw"), 256, "cmd")
    assert ent["fetch_scale"] == pytest.approx(2.0) and ent["write_scale"] == pytest.approx(1.0)
    assert ent["fetch_bytes_per_launch"] == 100 * (1 << 20)
    assert ent["write_bytes_per_launch"] == 20 * (1 << 20)
    assert bench.measured_traffic("wl") == 120 * (1 << 20)
    assert bench.measured_traffic("other") is None
    # a record taken on other kernel code is not reported
    rec = json.loads((tmp_path / "traffic.json").read_text())
    rec["workloads"]["wl"]["kernel_source_sha"] = "0" * 16
    (tmp_path / "traffic.json").write_text(json.dumps(rec))
    assert bench.measured_traffic("wl") is None


def test_traffic_needs_every_counter(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "traffic.json"))
    _write_counter_csv(tmp_path / "cf", [("copyBuffer", "FETCH_SIZE", 1.0)])
    _write_counter_csv(tmp_path / "empty", [])
    with pytest.raises(RuntimeError):
        bench.write_traffic("wl", str(tmp_path / "empty"), str(tmp_path / "empty"),
                            str(tmp_path / "cf"), str(tmp_path / "empty"), 256, "cmd")
