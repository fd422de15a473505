"""Host-side checks of bench.py (no GPU): the algorithmic work formulas, the
measured-traffic lookup and its source-hash guard, the clock-file parser and
the refusal of more than one GPU."""
import importlib.util
import json
import os
import subprocess
import sys
import threading
import time

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_algorithmic_work(bench):
    # 70B-shaped 32k prefill: 4 * 64 heads * 128 dims * (32768 * 32769 / 2) pairs
    assert bench.prefill_flops(1, 32768, 64, 128) == 4 * 64 * 128 * 32768 * 32769 // 2
    assert abs(bench.prefill_flops(1, 32768, 64, 128) - 1.7593e13) / 1.7593e13 < 1e-4
    # 1 token: the diagonal pair only
    assert bench.prefill_flops(1, 1, 1, 64) == 4 * 64
    # decode_100k: K and V of 16 x 100001 x 8 heads x 128 dims in bf16, plus q and o
    assert bench.decode_bytes(16, 100001, 64, 8, 128) == 16 * 100001 * 8 * 128 * 2 * 2 + 2 * 16 * 64 * 128 * 2


def test_measured_traffic_follows_the_source_hash(bench, tmp_path, monkeypatch):
    src = tmp_path / "kernel.hip"
    src.write_text("// one version\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    f = tmp_path / "traffic.json"
    entry = {"sources": ["kernel.hip"], "source_sha256": bench.source_hash(["kernel.hip"]), "bytes_per_launch": 123.0}
    f.write_text(json.dumps({"k": entry}))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.measured_traffic("k") == 123.0
    assert bench.measured_traffic("missing") is None
    src.write_text("// the kernel changed since the counters were taken\n")
    assert bench.measured_traffic("k") is None


def test_committed_traffic_file_names_existing_sources(bench):
    with open(bench.TRAFFIC_FILE) as fh:
        t = json.load(fh)
    for key in ("prefill_attend", "prefill_prepare", "decode_split", "rope_remap"):
        assert key in t, key
        for rel in t[key]["sources"]:
            assert os.path.exists(os.path.join(ROOT, rel)), rel
        assert t[key]["bytes_per_launch"] >= 0.99 * t[key]["algorithmic_bytes_per_launch"]


def test_clock_sampler_reads_the_starred_level(bench, tmp_path):
    f = tmp_path / "pp_dpm_sclk"
    f.write_text("S: 1865Mhz *\n0: 500Mhz\n1: 2400Mhz\n")
    c = bench.ClockSampler.__new__(bench.ClockSampler)
    c.path, c.power_path, c.samples, c.power, c.period = str(f), None, [], [], 0.001
    c._stop, c._thread = threading.Event(), None
    with c:
        time.sleep(0.05)
    s = c.summary()
    assert s["median_mhz"] == 1865 and s["samples"] >= 2 and s["power_w_median"] is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300)
    assert r.returncode != 0
    assert "one GPU" in r.stderr or "1 GPU" in r.stderr or "single" in r.stderr, r.stderr


def test_cpu_full_oracle_labels_whole_calls(bench):
    # the tiny fp32 prefill is timed whole and labelled; the decode sequence
    # only when one is handed over (here a small stand-in of the same form)
    out = bench.cpu_full_oracle(None)
    assert len(out) == 1 and out[0]["label"].startswith("tiny_f32 whole prefill")
    assert out[0]["seconds"] > 0 and out[0]["value"] > 0 and out[0]["unit"] == "GFLOP/s"
    import torch
    g = torch.Generator().manual_seed(0)
    dq = torch.randn(1, 64, 128, generator=g).to(torch.bfloat16)
    dk = torch.randn(1, 300, 8, 128, generator=g).to(torch.bfloat16)
    dv = torch.randn(1, 300, 8, 128, generator=g).to(torch.bfloat16)
    out = bench.cpu_full_oracle((dq, dk, dv))
    assert len(out) == 2 and out[1]["label"].startswith("decode_100k sequence 0") and out[1]["unit"] == "GB/s"
