"""Host logic of bench.py on the CPU: the refusal of several GPUs, the
kernel-trace and counter summaries on synthetic rocprofv3 output (dispatch
windows, launches per step, byte calibration), the traffic lookup's source
check, and the CPU baseline's whole-layer and sampled modes."""
from __future__ import annotations

import csv
import os
import re
import sqlite3
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


def _row(md, kernel):
    for line in md.splitlines():
        if line.startswith("| `") and kernel in line:
            return [c.strip() for c in line.strip("|").split("|")]
    raise AssertionError(f"no row for {kernel}")


def test_trace_summary_takes_the_timed_steps(tmp_path):
    """A gemm kernel launched twice per step: 2 * (W + K) rounds of two
    dispatches, then K + 1 back-to-back rounds of the stage alone; the timed
    moe_forward steps are dispatches [2W*2, (2W+K)*2)."""
    W_, K = 1, 2
    rounds = 2 * (W_ + K) + K + 1
    assert rounds == bench.gemm_rounds(W_, K)
    path = tmp_path / "run_kernel_trace.csv"
    t = 0
    durs = []
    with open(path, "w", newline="") as f:
        wr = csv.writer(f)
        wr.writerow(["Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        for i in range(rounds * 2):
            d = 1000 * (i + 1)  # ns
            durs.append(d)
            wr.writerow(["void moe::gemm_dma_kernel<256, 256, 64, 2, 2, 8, true>(moe::GemmParams, int)",
                         t, t + d])
            t += d + 10
        wr.writerow(["void moe::route_select_kernel<32>(moe::RouteParams)", t, t + 5000])
    md = bench._trace_summary(str(path), "w", K, W_)
    row = _row(md, "gemm_dma_kernel")
    assert row[1] == str(rounds * 2) and row[2] == "2"
    timed = sum(durs[2 * W_ * 2:(2 * W_ + K) * 2]) / K / 1e3
    assert float(row[3]) == pytest.approx(timed, abs=0.05)
    assert f"{timed:.1f} us per step" in md
    assert _row(md, "route_select_kernel")[3] == "-"  # not a whole number of launches per step
    assert "--no-graph" in md  # the command that made it


def _pmc_db(path, counter, rows):
    con = sqlite3.connect(path)
    con.execute("create table pmc_events (name text, dispatch_id int, counter_name text, "
                "counter_value real, duration real)")
    con.executemany("insert into pmc_events values (?, ?, ?, ?, ?)",
                    [(n, d, counter, v, dur) for n, d, v, dur in rows])
    con.commit()
    con.close()


def test_pmc_summary_splits_launches_and_calibrates(tmp_path):
    """Counter units become bytes through the calibration kernel's reading of
    its known 1 GiB; a gemm kernel with two launches per step gets one row
    per launch and both count in the step's bytes."""
    rounds = bench.gemm_rounds(bench.PMC_WARMUP, bench.PMC_STEPS)
    assert rounds == 2 * (bench.PMC_WARMUP + bench.PMC_STEPS) + bench.PMC_STEPS + 1
    gemm = "void moe::gemm_dma_kernel<256, 256, 64, 2, 2, 8, false>(moe::GemmParams, int)"
    calib = "void at::native::neg_kernel"
    f_units, w_units = 524288.0, 1048576.0  # units per GiB: 2048 B and 1024 B per unit
    fetch, write = [(calib, 0, f_units, 4e5)], [(calib, 0, w_units, 4e5)]
    for i in range(rounds * 2):
        launch = i % 2  # routed, then shared
        fetch.append((gemm, i + 1, 1000.0 * (launch + 1), 1e6))      # 2 or 4 MB read
        write.append((gemm, i + 1, 100.0 * (launch + 1), 1e6))       # 0.1 or 0.2 MB written
    _pmc_db(tmp_path / "f.db", "FETCH_SIZE", fetch)
    _pmc_db(tmp_path / "w.db", "WRITE_SIZE", write)
    md = bench._pmc_summary(str(tmp_path / "f.db"), str(tmp_path / "w.db"), "w")
    r1, r2 = _row(md, "1 of 2"), _row(md, "2 of 2")
    assert float(r1[4]) == pytest.approx(1000 * 2048 / 1e6, abs=0.05)
    assert float(r2[4]) == pytest.approx(2000 * 2048 / 1e6, abs=0.05)
    assert float(r2[5]) == pytest.approx(200 * 1024 / 1e6, abs=0.05)
    step = float(re.search(r"hbm_bytes_per_step: (\S+)", md).group(1))
    assert step == pytest.approx(3000 * 2048 + 300 * 1024, rel=1e-4)


def test_traffic_is_null_on_other_source(tmp_path, monkeypatch):
    path = tmp_path / "grouped_swiglu_traffic_{workload}.md"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(path))
    (tmp_path / "grouped_swiglu_traffic_w.md").write_text(
        "source_sha256_16: 0000000000000000\n\nhbm_bytes_per_step: 1e9\n")
    assert bench._traffic("w", 1) is None
    (tmp_path / "grouped_swiglu_traffic_w.md").write_text(
        f"source_sha256_16: {bench._source_hash()}\n\nhbm_bytes_per_step: 1e9\n")
    assert bench._traffic("w", 1) == pytest.approx(1e9)
    assert bench._traffic("absent", 1) is None


def test_f64_experts_upcast_only_what_is_read():
    import torch
    t = torch.arange(24, dtype=torch.float32).reshape(4, 2, 3).to(torch.bfloat16)
    fx = bench._F64Experts(t)
    assert fx.shape == (4, 2, 3) and fx.cache == {}
    a = fx[2]
    assert a.dtype.name == "float64" and (a == t[2].double().numpy()).all()
    assert list(fx.cache) == [2]


def test_cpu_baseline_whole_layer_and_sample(monkeypatch):
    import workloads as W
    w = W.SMALL["deepseek_small"]
    inp = W.make_inputs(w, "cpu", seed=0)
    whole = bench._cpu_baseline(w, inp, 0.01)
    assert whole["kind"] == "oracle" and whole["value"] > 0 and whole["cores"] >= 1
    assert whole["sample"].startswith("the whole layer")
    # a float64 cap below one expert forces the bounded sample
    monkeypatch.setattr(bench, "CPU_F64_CAP", 1.0)
    samp = bench._cpu_baseline(w, inp, 0.01)
    assert samp["value"] > 0 and "evenly spaced" in samp["sample"]
