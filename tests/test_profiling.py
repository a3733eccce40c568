"""Host logic of the rocprofv3 summaries (synthetic CSV files, no GPU)."""
import csv
import json
import os

from exact_io_aware_26_amd import profiling

KV = "void fa2::(anonymous namespace)::bwd_kv_kernel<128, true>(fa2::BwdParams)"
COPY = "__amd_rocclr_copyBuffer"


def _write_counters(path, counter, values):
    os.makedirs(path, exist_ok=True)
    with open(os.path.join(path, "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for name, v in values:
            w.writerow({"Kernel_Name": name, "Counter_Name": counter, "Counter_Value": v})


def test_traffic_scales_each_counter_by_the_copy_calibration(tmp_path):
    copy_bytes = 1 << 20
    # FETCH_SIZE reads half the bytes the copy moved, WRITE_SIZE all of them.
    _write_counters(tmp_path / "f", "FETCH_SIZE", [(COPY, 512.0), (KV, 100.0)])
    _write_counters(tmp_path / "w", "WRITE_SIZE", [(COPY, 1024.0), (KV, 30.0)])
    rec, md = profiling.traffic(str(tmp_path / "f"), str(tmp_path / "w"), "bwd_kv_kernel<128, true>",
                                copy_bytes, ["cmd1", "cmd2"])
    assert rec["fetch_scale"] == 2.0 and rec["write_scale"] == 1.0
    assert rec["read_bytes"] == 100.0 * 1024 * 2.0
    assert rec["write_bytes"] == 30.0 * 1024
    assert rec["bytes_per_launch"] == rec["read_bytes"] + rec["write_bytes"]
    assert rec["source_sha256"] == profiling.kernel_source_digest()
    assert "cmd1" in md and "bwd_kv_kernel<128, true>" in md
    json.dumps(rec)


def test_trace_averages_the_timed_launches(tmp_path):
    d = tmp_path / "t"
    d.mkdir()
    with open(d / "run_kernel_stats.csv", "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage",
                                          "MinNs", "MaxNs", "StdDev"])
        w.writeheader()
        w.writerow({"Name": KV, "Calls": 3, "TotalDurationNs": 9000, "AverageNs": 3000, "Percentage": 100,
                    "MinNs": 2000, "MaxNs": 5000, "StdDev": 0})
    with open(d / "run_kernel_trace.csv", "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        w.writeheader()
        for start, dur in ((0, 5000), (10000, 2000), (20000, 2000)):   # one warmup launch, two timed
            w.writerow({"Kernel_Name": KV, "Start_Timestamp": start, "End_Timestamp": start + dur})
    bench = tmp_path / "b.json"
    bench.write_text("noise\n" + json.dumps({"steps": 2, "roofline": {"kernel": "k", "avg_launch_ms": 0.002,
                                                                     "achieved": 1.0, "unit": "TFLOP/s",
                                                                     "frac": 0.5}}) + "\n")
    md = profiling.trace(str(d), str(bench), "the command")
    row = [l for l in md.splitlines() if l.startswith("| bwd_kv_kernel")][0]
    assert row.rstrip(" |").endswith("2.0")      # mean of the last two launches, in us
    assert "the command" in md and "2.0 us per launch" in md


def test_source_digest_ignores_comments_and_layout():
    a = "int f(int x) {  // one\n    return x + 1; /* two\n three */ }\n"
    b = "int f(int x) { return x + 1; }"
    c = "int f(int x) { return x + 2; }"
    assert profiling._code_only(a) == profiling._code_only(b)
    assert profiling._code_only(b) != profiling._code_only(c)


def _write_trace(path, rows):
    os.makedirs(path, exist_ok=True)
    with open(os.path.join(path, "run_kernel_trace.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        w.writeheader()
        t = 0
        for name, ns in rows:
            w.writerow({"Kernel_Name": name, "Start_Timestamp": t, "End_Timestamp": t + ns})
            t += ns + 1000


def test_counters_derive_clock_and_mfma_busy(tmp_path):
    a, b = tmp_path / "a", tmp_path / "b"
    t_ns = 1_000_000                                   # 1 ms
    clock = 2.0e9
    busy_cycles = profiling.N_SE * clock * 1e-3        # all shader engines busy for the whole launch
    mfma = 1000.0
    for d, cvals in ((a, {"SQ_BUSY_CYCLES": busy_cycles, "SQ_VALU_MFMA_BUSY_CYCLES":
                          0.5 * profiling.N_SIMD * clock * 1e-3, "SQ_INSTS_MFMA": mfma,
                          "SQ_INSTS_VALU": 4 * mfma, "SQ_WAVE_CYCLES": 100.0}),
                     (b, {"SQ_LDS_BANK_CONFLICT": 1.0, "SQ_LDS_IDX_ACTIVE": 100.0, "SQ_WAIT_INST_LDS": 10.0})):
        os.makedirs(d, exist_ok=True)
        with open(d / "run_counter_collection.csv", "w", newline="") as f:
            w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
            w.writeheader()
            for cn, v in cvals.items():
                w.writerow({"Kernel_Name": KV, "Counter_Name": cn, "Counter_Value": v})
        _write_trace(d, [(KV, 5 * t_ns), (KV, t_ns)])   # a cold dispatch, then the one reported
    _write_counters(tmp_path / "f", "FETCH_SIZE", [(COPY, 512.0), (KV, 1024.0)])
    _write_counters(tmp_path / "w", "WRITE_SIZE", [(COPY, 1024.0), (KV, 0.0)])
    md = profiling.counters([str(a), str(b)], str(tmp_path / "f"), str(tmp_path / "w"), 1 << 20, ["c1", "c2"])
    row = [l for l in md.splitlines() if l.startswith("| bwd_kv_kernel") and "SQ_" not in l][0]
    cells = [c.strip() for c in row.strip("|").split("|")]
    assert cells[1] == "1000.0" and cells[2] == "2.00" and cells[3] == "50.0 %" and cells[4] == "3.00"
    assert cells[5] == "1.00 %" and cells[6] == "10.0 %"
    assert cells[7] == "2"                              # 1024 KiB x 2.0 read in 1 ms = 2.1 GB/s
