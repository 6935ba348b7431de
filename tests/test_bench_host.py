"""Host-side checks of bench.py (CPU only): the one-GPU guard and the two
rocprofv3 summarisers on synthetic result files."""

import csv
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BENCH = os.path.join(ROOT, "bench.py")


def _run(*args, env=None):
    return subprocess.run([sys.executable, BENCH, *args], capture_output=True, text=True,
                          env=env, timeout=120)


def test_more_than_one_gpu_exits_with_a_message():
    r = _run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""
    env = dict(os.environ, WORLD_SIZE="4")
    r = _run(env=env)
    assert r.returncode == 2 and "one GPU" in r.stderr


def _write_csv(path, header, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(header)
        w.writerows(rows)


def test_summarize_trace_table(tmp_path):
    d = tmp_path / "trace"
    _write_csv(str(d / "run_kernel_stats.csv"),
               ["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage", "MinNs", "MaxNs"],
               [["void nf4moe::grouped_gemm_kernel<true, 0, false, 2, 0, false>(nf4moe::GemmArgs, int)",
                 "19", "6000000", "315790.5", "61.5", "300000", "330000"],
                ["combine|kernel", "7", "168000", "24000", "1.7", "23000", "25000"]])
    r = _run("--summarize-trace", str(d))
    assert r.returncode == 0, r.stderr
    lines = r.stdout.strip().splitlines()
    assert lines[0].startswith("| kernel | calls | avg us")
    assert "| 19 | 315.79 | 300.00 | 330.00 | 61.50 |" in lines[2]
    assert "combine/kernel" in lines[3]  # a '|' in a name cannot break the table


def test_summarize_counters_scales_by_the_copy(tmp_path):
    hdr = ["Kernel_Name", "Counter_Name", "Counter_Value"]
    gemm = "void nf4moe::grouped_gemm_kernel<true, 0, false, 2, 0, false>(nf4moe::GemmArgs, int)"
    copy = "__amd_rocclr_copyBuffer"
    mib512 = 512 * 1024  # KiB
    _write_csv(str(tmp_path / "f" / "run_counter_collection.csv"), hdr,
               [[gemm, "FETCH_SIZE", "1000"], [gemm, "FETCH_SIZE", "3000"],
                [copy, "FETCH_SIZE", str(mib512 // 2)], [copy, "FETCH_SIZE", "5"]])
    _write_csv(str(tmp_path / "w" / "run_counter_collection.csv"), hdr,
               [[gemm, "WRITE_SIZE", "640"], [copy, "WRITE_SIZE", str(mib512)]])
    r = _run("--summarize-counters", str(tmp_path / "f"), str(tmp_path / "w"))
    assert r.returncode == 0, r.stderr
    rec = json.loads(r.stdout.split("```json", 1)[1].split("```", 1)[0])
    # fetch reads half the copied bytes: scale 2; the GEMM's mean 2000 KiB -> 4000 KiB
    assert rec["fetch_scale"] == 2.0 and rec["write_scale"] == 1.0
    assert rec["hbm_fetch_bytes_per_launch"] == 4000 * 1024
    assert rec["hbm_write_bytes_per_launch"] == 640 * 1024
    assert rec["gemm_dispatches"] == [2, 1]
