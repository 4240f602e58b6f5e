"""bench.py's contract and its measurement plumbing, on the CPU: the one-GPU
exit, the rocprofv3 command lines (counter limits per pass, no counters
combined with tracing), the FLOP conventions, and the profile summarizer's
arithmetic on synthetic rocprofv3 CSV files."""
import csv
import json
import os
import re
import subprocess
import sys

import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120)
    assert res.returncode == 2
    assert "one GPU" in res.stderr or "single" in res.stderr


def test_gemm_pass_rejects_attention_workloads():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--pass", "gemm",
                          "--workload", "mha_128k"], capture_output=True, text=True, timeout=120)
    assert res.returncode == 2 and "gemm_" in res.stderr


# Per-block limits of one rocprofv3 --pmc run (FETCH_SIZE takes 3 TCC
# counters, WRITE_SIZE 2).
TCC_COST = {"FETCH_SIZE": 3, "WRITE_SIZE": 2}


@pytest.mark.parametrize("which,workload", [("fwd", "mha_128k"), ("bwd", "mha_32k_causal"),
                                            ("gemm", "gemm_tall_64k_2k_8k"),
                                            ("decode", "decode_gqa64x8_b16_128k")])
def test_profile_commands_respect_counter_limits(which, workload):
    cmds = bench.profile_commands(workload, "/tmp/out", which)
    assert "trace" in cmds and "--kernel-trace" in cmds["trace"] and "--pmc" not in cmds["trace"]
    for name, cmd in cmds.items():
        if "--pmc" not in cmd:
            continue
        for bad in (" -s ", "--sys-trace", " -r ", "--runtime-trace", "--kernel-trace",
                    "--hip-trace", "--hsa-trace", "--memory-copy-trace", "--marker-trace"):
            assert bad not in cmd, (name, bad)
        ctrs = cmd.split("--pmc", 1)[1].split("--output-format")[0].split()
        sq = [c for c in ctrs if c.startswith("SQ_")]
        grbm = [c for c in ctrs if c.startswith("GRBM_")]
        tcc = sum(TCC_COST.get(c, 1) for c in ctrs if c.startswith("TCC_") or c in TCC_COST)
        assert len(sq) <= 8 and len(grbm) <= 2 and tcc <= 4, (name, ctrs)
        assert cmd.split(" -- ", 1)[1].startswith("python3 "), name   # the program itself after --
        if which != "fwd":
            assert f"--pass {which}" in cmd or "--copy-calibration" in cmd


def test_flop_conventions():
    f = bench.attn_flops(1, 2, 4, 8, False)
    assert f == 4.0 * 2 * 8 * 16
    assert bench.attn_flops(1, 2, 4, 8, True) == 4.0 * 2 * 8 * 10
    assert bench.pass_flops("bwd", 1, 2, 4, 8, True) == 2.5 * bench.attn_flops(1, 2, 4, 8, True)
    assert bench.pass_flops("fwd", 1, 2, 4, 8, False) == f


def _write_counters(path, kernel, rows):
    """rows: list of dicts counter -> value, one per dispatch (1 ms each)."""
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as fh:
        w = csv.writer(fh)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value",
                    "Start_Timestamp", "End_Timestamp"])
        for i, r in enumerate(rows):
            for name, val in r.items():
                w.writerow([i + 1, kernel, name, val, 1_000_000 * i, 1_000_000 * i + 1_000_000])


def test_summarize_profile_arithmetic(tmp_path, monkeypatch):
    """Synthetic counters: L2 hit = hit / (hit + miss); HBM bytes = KiB x 1024
    x the copy calibration; MFMA busy = busy / (GRBM_GUI_ACTIVE / 8 x 1024)."""
    d = tmp_path / "prof"
    n = len(bench.PROFILE_MODES)
    k = "attn_numa::attn_fwd_kernel<128, false, true>"
    _write_counters(str(d / "l2" / "l2_counter_collection.csv"), k,
                    [{"TCC_HIT_sum": 90.0 + m, "TCC_MISS_sum": 10.0 - m} for m in range(n)])
    _write_counters(str(d / "fetch" / "fetch_counter_collection.csv"), k,
                    [{"FETCH_SIZE": 1024.0 * (m + 1)} for m in range(n)])
    _write_counters(str(d / "write" / "write_counter_collection.csv"), k,
                    [{"WRITE_SIZE": 512.0} for m in range(n)])
    gui = 8 * 2.0e6  # 2e6 cycles per XCD in 1 ms: 2 GHz
    _write_counters(str(d / "mfma" / "mfma_counter_collection.csv"), k,
                    [{"SQ_VALU_MFMA_BUSY_CYCLES": 0.5 * 2.0e6 * 1024, "SQ_INSTS_VALU_MFMA_MOPS_BF16": 1.0,
                      "SQ_BUSY_CYCLES": 1.0, "GRBM_GUI_ACTIVE": gui} for m in range(n)])
    # copy calibration: 1 GiB read counts as 512 MiB (x2), written as 1 GiB (x1)
    _write_counters(str(d / "copy_fetch" / "c_counter_collection.csv"), "__amd_rocclr_copyBuffer",
                    [{"FETCH_SIZE": float(1 << 19)}])
    _write_counters(str(d / "copy_write" / "c_counter_collection.csv"), "__amd_rocclr_copyBuffer",
                    [{"WRITE_SIZE": float(1 << 20)}])
    out_dir = tmp_path / "profiles"
    monkeypatch.setattr(bench, "PROFILES", str(out_dir))
    bench.summarize_profile(str(d), "mha_h8_1k")
    data = json.load(open(out_dir / "counters_attn_fwd_mha_h8_1k.json"))
    assert data["calibration"]["scale"]["FETCH_SIZE"] == pytest.approx(2.0)
    assert data["calibration"]["scale"]["WRITE_SIZE"] == pytest.approx(1.0)
    for m, mode in enumerate(bench.PROFILE_MODES):
        mm = data["modes"][bench.MODE_NAMES[mode]]
        assert mm["l2_hit_pct"] == pytest.approx(90.0 + m, abs=0.01)
        assert mm["fetch_bytes"] == pytest.approx(1024.0 * (m + 1) * 1024 * 2.0)
        assert mm["write_bytes"] == pytest.approx(512.0 * 1024)
        assert mm["mfma_busy_pct"] == pytest.approx(50.0, abs=0.01)
        assert mm["clock_ghz"] == pytest.approx(2.0, abs=1e-3)
    md = open(out_dir / "attn_fwd_mha_h8_1k.md").read()
    assert re.search(r"Kernel source hash [0-9a-f]{16}", md)


def test_backward_executed_work():
    """attn_bwd executes 14 MFMA FLOP per (query, visible key) per padded
    head dimension (S, dP, dV, dK; then S, dP and dQ again) against the
    10 d credited, so at d = 128 the executed rate is 1.4x the credited one,
    and at d = 56 (run on 64 padded columns) 1.6x."""
    e = bench._bwd_executed(1000.0, 128)
    assert e["tflops"] == pytest.approx(1400.0)
    assert e["frac"] == pytest.approx(1400.0 / bench.PEAK_BF16_TFLOPS, abs=1e-4)
    assert bench._bwd_executed(1000.0, 56)["tflops"] == pytest.approx(1600.0)
    assert bench._bwd_executed(1000.0, 96)["tflops"] == pytest.approx(1000.0 * 14 * 128 / 960, abs=0.01)
