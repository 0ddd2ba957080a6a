"""bench.py's contract, on the CPU: the refusal of more than one GPU, the
fields of the JSON line, and the rule that recorded HBM traffic is reported
only for the kernel sources it was measured on."""
import argparse
import json
import os
import shutil
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "--gpus must be 1" in r.stderr and r.stdout == ""


def test_json_line_fields():
    args = argparse.Namespace(steps=1000, warmup=20)
    cpu = {"value": 2.33, "unit": "GB/s", "cores": 1, "kind": "oracle", "sample": "s", "us_per_call": 1237.0}
    line = bench.make_line(args, 9.0, cpu, {})
    json.dumps(line)
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
              "scaling", "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline"):
        assert k in line, k
    assert line["n_gpus"] == 1 and line["steps"] == 1000 and line["warmup"] == 20
    assert line["unit"] == "GB/s" and line["higher_is_better"] is True and line["vs_baseline"] is None
    bytes_call = (8 + 3) * 2 * 131072
    assert abs(line["value"] - bytes_call / 9.0 / 1e3) < 0.01
    assert abs(line["ms_per_step"] - 0.009) < 1e-9
    assert "workload" in line["config"] and "model" not in line["config"]
    rf = line["roofline"]
    assert rf["bound"] == "hbm" and rf["peak"] == 8000.0 and rf["unit"] == "GB/s"
    assert rf["achieved"] == line["value"] and abs(rf["frac"] - rf["achieved"] / rf["peak"]) < 1e-5
    assert rf["bytes_per_launch"] == bytes_call
    assert rf["event_us_per_launch"] == 9.0 and "kernel_us" not in rf   # event time per launch, named as such
    assert line["cpu_baseline"]["kind"] == "oracle" and line["cpu_baseline"]["cores"] >= 1


def test_json_line_without_measurement():
    line = bench.make_line(argparse.Namespace(steps=5, warmup=1), None, None, {})
    assert line["value"] is None and line["roofline"]["achieved"] is None and line["roofline"]["frac"] is None


def test_traffic_only_for_the_sources_it_was_measured_on(tmp_path):
    csrc = tmp_path / "csrc"
    shutil.copytree(os.path.join(ROOT, "signal_pad_sync_amd", "csrc"), csrc)
    rec = tmp_path / "traffic.json"
    rec.write_text(json.dumps({"kernel_source_sha256": bench.kernel_source_hash(str(csrc)), "k": 1234}))
    assert bench.recorded_traffic("k", str(rec), str(csrc)) == 1234
    assert bench.recorded_traffic("missing", str(rec), str(csrc)) is None
    with open(csrc / "arx_reduce.hip", "a") as f:          # any change to a kernel source
        f.write("\n// changed\n")
    assert bench.recorded_traffic("k", str(rec), str(csrc)) is None
    assert bench.recorded_traffic("k", str(tmp_path / "absent.json"), str(csrc)) is None
