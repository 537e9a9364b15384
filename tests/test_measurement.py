"""Host-side measurement logic (no GPU): the rocprofv3 counter calibration
that turns FETCH_SIZE / WRITE_SIZE into bytes per launch, the source-hash
gate on the stored traffic record, and bench.py's one-GPU contract."""

import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

GATE_UP = "void moe::(anonymous namespace)::gate_up_decode_kernel<1, 2, 2, true>(moe::GateUpArgs)"
COPY = "moe::(anonymous namespace)::copy_kernel(unsigned int __vector(4) const*, unsigned long)"


def _write_counters(folder, counter, rows):
    os.makedirs(folder, exist_ok=True)
    with open(os.path.join(folder, "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for name, value in rows:
            w.writerow({"Kernel_Name": name, "Counter_Name": counter, "Counter_Value": value})


def test_traffic_calibration_against_the_copy_kernel(tmp_path):
    from mixture_experts_decode_amd import traffic_summary as ts
    gib4 = 4 * 2 ** 30
    # FETCH_SIZE reads half of the copy kernel's 4 GiB, WRITE_SIZE all of it
    # (KiB per dispatch); a kernel's bytes are its counter times the factor
    _write_counters(tmp_path / "f", "FETCH_SIZE",
                    [(COPY, gib4 / 2 / 1024)] * 2 + [(GATE_UP, 100_000.0), (GATE_UP, 102_000.0)])
    _write_counters(tmp_path / "w", "WRITE_SIZE",
                    [(COPY, gib4 / 1024)] * 2 + [(GATE_UP, 768.0), (GATE_UP, 768.0)])
    ff, fw, rows = ts.summarise(str(tmp_path / "f"), str(tmp_path / "w"))
    assert ff == pytest.approx(2.0) and fw == pytest.approx(1.0)
    (name, r), = rows.items()
    assert "gate_up_decode_kernel" in name and r["dispatches"] == 2
    assert r["fetch"] == pytest.approx(101_000.0 * 1024 * 2.0)
    assert r["write"] == pytest.approx(768.0 * 1024)


def test_traffic_summary_needs_the_copy_kernel(tmp_path):
    from mixture_experts_decode_amd import traffic_summary as ts
    _write_counters(tmp_path / "f", "FETCH_SIZE", [(GATE_UP, 1.0)])
    _write_counters(tmp_path / "w", "WRITE_SIZE", [(GATE_UP, 1.0)])
    with pytest.raises(SystemExit):
        ts.summarise(str(tmp_path / "f"), str(tmp_path / "w"))


def test_stored_traffic_is_reported_only_for_the_sources_it_was_taken_on(monkeypatch):
    sys.path.insert(0, ROOT)
    import bench
    path = os.path.join(ROOT, "profiles",
                        "traffic_gate_up_decode_kernel_qwen3_decode_mxfp8_b32.json")
    rec = json.load(open(path))
    # the record is reported exactly when it was taken on the current sources
    fresh = rec["kernel_source_hash"] == bench.kernel_source_hash()
    assert bench.load_traffic("qwen3_decode_mxfp8", 32) == (rec["hbm_bytes_per_launch"] if fresh
                                                            else None)
    # and the counters agree with the launch's algorithmic bytes: the touched
    # experts' gate and up rows with their E8M0 scales, x, the ids and the BF16
    # h, averaged over the routing draws the bench's steps cycle through
    import workloads as W
    cfg = W.QWEN3_DECODE_MXFP8
    t, k, h_dim, i_dim = 32, cfg.top_k, cfg.hidden, cfg.inter
    algo = []
    for v in range(5):
        ids, _ = W.routing(cfg, t, variant=v)
        u = len(W.touched_experts(cfg, ids))
        algo.append(u * 2 * i_dim * (h_dim + h_dim // 32) + t * h_dim * 2 + t * k * 4
                    + t * k * i_dim * 2)
    assert abs(rec["hbm_bytes_per_launch"] / (sum(algo) / len(algo)) - 1) < 0.01
    # a changed kernel source (another hash) reports no traffic
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "0" * 16)
    assert bench.load_traffic("qwen3_decode_mxfp8", 32) is None
    assert bench.load_traffic("qwen3_decode_mxfp8", 64) is None


def test_bench_measures_one_gpu_only():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_bench_helpers():
    sys.path.insert(0, ROOT)
    import bench
    assert bench.sample_rows(5, None) == [0, 1, 2, 3, 4]
    assert bench.sample_rows(5, 9) == [0, 1, 2, 3, 4]
    assert bench.sample_rows(100, 3) == [0, 49, 99]
    s = bench.spread([3.0, 1.0, 2.0])
    assert s["p50"] == 2.0 and s["n"] == 3 and s["p10"] <= s["p50"] <= s["p90"]
