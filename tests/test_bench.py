"""The bench.py output contract: one JSON line on stdout with the metric and its unit, the step's
throughput and time, the run's shape, a roofline object for the dominant kernel (achieved over
peak) and a CPU-baseline object (the oracle timed on a bounded sample); more than one GPU is
refused with a message, before any GPU is touched; and the roofline's counter-measured traffic is
reported only while the sources it was measured on are unchanged."""
import json
import os
import subprocess
import sys

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run_bench(*args, timeout=300):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          timeout=timeout, cwd=ROOT)


def last_json(stdout):
    return json.loads(stdout.strip().splitlines()[-1])


def test_more_than_one_gpu_is_refused():
    r = run_bench("--gpus", "2", timeout=120)
    assert r.returncode == 2
    line = last_json(r.stdout)
    assert "--gpus 1" in line["error"]
    assert "single GPU" in r.stderr


@pytest.mark.gpu
@pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")
def test_json_line_contract():
    print("[gpu] bench.py --workload 1 --steps 3 --warmup 1", flush=True)
    r = run_bench("--workload", "1", "--steps", "3", "--warmup", "1", "--cpu-budget", "1")
    assert r.returncode == 0, r.stderr[-2000:]
    d = last_json(r.stdout)
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
                "scaling", "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 1
    assert d["higher_is_better"] is True and d["scaling"] in ("weak", "strong")
    assert d["value"] > 0 and d["ms_per_step"] > 0 and d["unit"] == "GB/s"
    assert d["config"]["workload"] == "tiny_mha_fp32_split4" and "model" not in d["config"]
    rf = d["roofline"]
    assert rf["bound"] in ("hbm", "mfma", "alu") and rf["unit"] in ("GB/s", "TFLOP/s")
    assert rf["peak"] > 0 and abs(rf["frac"] - rf["achieved"] / rf["peak"]) < 1e-3
    assert "traffic" in rf
    cb = d["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["cores"] >= 1 and cb["value"] > 0 and cb["unit"] == d["unit"]
    assert cb["sample"]


def test_traffic_record_goes_stale_with_its_sources(tmp_path, monkeypatch):
    """`roofline.traffic` comes from a committed counter record that names the sources it was
    measured on and their sha256: it is reported while they are unchanged, and null (None) once
    any of them changes (a comment included) or is missing."""
    import shutil
    import bench
    rec = json.load(open(os.path.join(ROOT, "profiles", "traffic_mla_partial.json")))
    for rel in rec["sources"]:
        os.makedirs(tmp_path / os.path.dirname(rel), exist_ok=True)
        shutil.copy(os.path.join(ROOT, rel), tmp_path / rel)
    os.makedirs(tmp_path / "profiles")
    shutil.copy(os.path.join(ROOT, "profiles", "traffic_mla_partial.json"), tmp_path / "profiles")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.load_traffic("mla_partial") == rec["bytes_per_launch"]
    planner = tmp_path / "attention_decode_amd" / "csrc" / "api.cpp"
    planner.write_text(planner.read_text() + "// edited\n")
    assert bench.load_traffic("mla_partial") is None
    planner.unlink()
    assert bench.load_traffic("mla_partial") is None
    assert bench.load_traffic("no_such_kernel") is None


def test_committed_traffic_records_are_current():
    """Every committed counter record matches the sources as they stand, so the traffic that
    bench reports comes from the kernels in this tree."""
    import glob
    import bench
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "traffic_*.json"))):
        tag = os.path.basename(path)[len("traffic_"):-len(".json")]
        assert bench.load_traffic(tag) is not None, f"{tag}: sources changed since its counter run"
