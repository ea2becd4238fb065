"""Host-side logic of the measurement (no GPU): the one-GPU contract of
bench.py, the algorithmic byte counts the roofline fractions divide by (each
recomputed here from the tensors a launch reads and writes), and the profile
summary's averaging over exactly the timed launches and its counter scaling
(synthetic rocprofv3 CSV files)."""
import csv
import json
import os
import subprocess
import sys

import bench
from subquadratic_attention_amd import prof

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_forward_bytes_per_head_token():
    # one token of one head: q, k, v and y rows (d elements each) in bf16,
    # the log-gate row in float32; with logits the gate row is bf16 too
    d = 128
    assert bench.fwd_bytes_per_head_token(d) == 4 * d * 2 + d * 4 == 1536
    assert bench.fwd_logit_bytes_per_head_token(d) == 5 * d * 2 == 1280
    # the 4K prefill, B = 4, H = 32, L = 4096: the figure the bench reports
    assert 4 * 32 * 4096 * bench.fwd_bytes_per_head_token(d) == 805306368


def test_backward_bytes_per_head_token():
    # reads q, k, v, dY (bf16), log_g (f32) and one lse value (f32); writes
    # dq, dk, dv (bf16) and dlog_g (f32)
    d = 128
    assert bench.bwd_bytes_per_head_token(d) == 4 * d * 2 + d * 4 + 4 + 3 * d * 2 + d * 4 == 2820
    assert 8 * 32 * 2048 * bench.bwd_bytes_per_head_token(d) == 1478492160


def test_decode_bytes_per_step():
    # per (b, h): the fp32 state read and written, the window's other w - 1
    # keys and values, the token's q, k, v (bf16) and log-gate (f32) in, its
    # key and value to the ring slot and y out (bf16)
    d, w = 128, 64
    expect = 2 * d * d * 4 + 2 * (w - 1) * d * 2 + 3 * d * 2 + d * 4 + 2 * d * 2 + d * 2
    assert bench.decode_bytes_per_bh(d, w) == expect == 165376
    assert 64 * 32 * bench.decode_bytes_per_bh(d, w) == 338690048


def _write_csv(path, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        wr = csv.DictWriter(f, fieldnames=list(rows[0].keys()))
        wr.writeheader()
        wr.writerows(rows)


def test_profile_summary_averages_the_timed_launches(tmp_path):
    # a kernel launched 10 times: 5 warm-up launches of 100 us, then the 3
    # timed steps' launches of 10, 20 and 30 us at the end of the trace
    # (with 2 other launches of 100 us between), another kernel once per step
    trace = tmp_path / "trace"
    durs = [100e3] * 7 + [10e3, 20e3, 30e3]
    rows, t = [], 0
    for dur in durs:
        rows.append({"Kernel_Name": "k_main<1>", "Start_Timestamp": t, "End_Timestamp": int(t + dur)})
        rows.append({"Kernel_Name": "k_side", "Start_Timestamp": t + 200000, "End_Timestamp": t + 205000})
        t += 1000000
    _write_csv(str(trace / "run_kernel_trace.csv"), rows)
    stats = [{"Name": "k_main<1>", "Calls": 10, "AverageNs": 1, "MinNs": 1, "MaxNs": 1, "Percentage": 50},
             {"Name": "k_side", "Calls": 10, "AverageNs": 1, "MinNs": 1, "MaxNs": 1, "Percentage": 50}]
    _write_csv(str(trace / "run_kernel_stats.csv"), stats)
    n, avg = prof.timed_average_us(str(trace), "k_main", 3)
    assert (n, avg) == (3, 20.0)
    # counters: a 1 GiB copy reads as 512 MiB fetched (in KiB) and 1 GiB
    # written, so fetch is scaled by 2 and write by 1
    fetch, write = tmp_path / "fetch", tmp_path / "write"
    _write_csv(str(fetch / "run_counter_collection.csv"),
               [{"Kernel_Name": prof.COPY_KERNEL, "Counter_Name": "FETCH_SIZE", "Counter_Value": 512 * 1024},
                {"Kernel_Name": "k_main<1>", "Counter_Name": "FETCH_SIZE", "Counter_Value": 1000},
                {"Kernel_Name": "k_main<1>", "Counter_Name": "FETCH_SIZE", "Counter_Value": 3000},
                {"Kernel_Name": "k_side", "Counter_Name": "FETCH_SIZE", "Counter_Value": 10}])
    _write_csv(str(write / "run_counter_collection.csv"),
               [{"Kernel_Name": prof.COPY_KERNEL, "Counter_Name": "WRITE_SIZE", "Counter_Value": 1024 * 1024},
                {"Kernel_Name": "k_main<1>", "Counter_Name": "WRITE_SIZE", "Counter_Value": 500},
                {"Kernel_Name": "k_side", "Counter_Name": "WRITE_SIZE", "Counter_Value": 5}])
    out = tmp_path / "out"
    prof.main(["lizard_test", "wl", "k_main,k_side", "bench.py", str(trace), str(fetch), str(write), str(out), "3",
               "echo", "command"])
    rec = json.load(open(out / "lizard_test_wl_counters.json"))
    assert rec["fetch_scale"] == 2.0 and rec["write_scale"] == 1.0 and rec["timed_steps"] == 3
    assert rec["kernels"]["k_main"]["read_bytes_per_launch"] == 2000 * 1024 * 2.0
    assert rec["kernels"]["k_main"]["write_bytes_per_launch"] == 500 * 1024
    assert rec["hbm_bytes_per_launch"] == (2000 * 2 + 10 * 2 + 500 + 5) * 1024
    assert rec["source_hash"] == bench.source_hash("bench.py")
    text = open(out / "lizard_test_wl.md").read()
    assert "| `k_main` | 3 | 20.00 |" in text and "timed_steps = 3" in text
