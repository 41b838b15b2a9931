"""Host-side checks of bench.py: the byte model, the hash gate on the traffic
record, and the one-GPU contract.  No GPU and no kernel launch."""

import hashlib
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_algorithmic_bytes_llama_layers():
    # codes N*K/2 + one scale byte per G weights + BF16 activations and outputs
    assert bench.algorithmic_bytes(16, 57344, 8192, 16) == 234881024 + 29360128 + 262144 + 1835008
    assert bench.algorithmic_bytes(16, 8192, 28672, 32) == 117440512 + 7340032 + 917504 + 262144
    assert bench.algorithmic_bytes(0, 16, 32, 16) == 256 + 32


def _record(tmp_path, sha):
    rec = json.load(open(bench.TRAFFIC_RECORD))
    rec["source_sha256"] = sha
    rec["hbm_bytes_per_launch"] = 123456789
    p = tmp_path / "traffic.json"
    p.write_text(json.dumps(rec))
    return str(p), rec["sources"]


def test_traffic_reported_only_while_sources_match(tmp_path, monkeypatch):
    rec = json.load(open(bench.TRAFFIC_RECORD))
    h = hashlib.sha256()
    for f in rec["sources"]:
        h.update(open(os.path.join(ROOT, f), "rb").read())
    good, _ = _record(tmp_path, h.hexdigest())
    monkeypatch.setattr(bench, "TRAFFIC_RECORD", good)
    assert bench.measured_traffic() == 123456789
    bad, _ = _record(tmp_path, "0" * 64)
    monkeypatch.setattr(bench, "TRAFFIC_RECORD", bad)
    assert bench.measured_traffic() is None
    monkeypatch.setattr(bench, "TRAFFIC_RECORD", str(tmp_path / "missing.json"))
    assert bench.measured_traffic() is None


def test_committed_traffic_record_is_plausible():
    rec = json.load(open(bench.TRAFFIC_RECORD))
    alg = bench.algorithmic_bytes(16, 57344, 8192, 16)
    assert rec["algorithmic_bytes_per_launch"] == alg
    # HBM bytes from the counters: every weight byte read once, little more
    assert alg <= rec["hbm_bytes_per_launch"] <= 1.1 * alg
    cal = rec["calibration"]
    assert cal["copy_bytes"] == 268435456
    assert abs(cal["fetch_factor"] - cal["copy_bytes"] / (cal["copy_fetch_kib"] * 1024)) < 1e-5
    for f in rec["sources"]:
        assert os.path.exists(os.path.join(ROOT, f)), f


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


@pytest.mark.parametrize("flag", ["--no-prefill", "--no-fp16", "--no-moe", "--no-blas", "--no-configs"])
def test_parse_accepts_documented_flags(flag, monkeypatch):
    monkeypatch.setattr(sys, "argv", ["bench.py", flag, "--steps", "3", "--warmup", "1"])
    a = bench.parse()
    assert a.steps == 3 and a.warmup == 1 and a.gpus == 1
