"""Host logic of the benchmark and of the profile summaries (no GPU): the
one-GPU contract of bench.py and the HBM-traffic arithmetic of
profile_summary (counters scaled by a copy kernel of known size)."""
import csv
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def _counters(d, rows):
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for k, c, v in rows:
            w.writerow({"Kernel_Name": k, "Counter_Name": c, "Counter_Value": v})


def test_traffic_summary_scales_counters_by_the_copy(tmp_path):
    from hierarchical_sparse_attention_amd import profile_summary
    import bench
    kname = "void hs::(anonymous namespace)::k_step<hs::bf16_t, 128, 1, 4>(hs::StepParams, int)"
    _counters(tmp_path / "f", [(kname, "FETCH_SIZE", 1000.0), (kname, "FETCH_SIZE", 3000.0),
                               ("other", "FETCH_SIZE", 9.0)])
    _counters(tmp_path / "w", [(kname, "WRITE_SIZE", 10.0), (kname, "WRITE_SIZE", 30.0)])
    # a 1 GiB copy that FETCH_SIZE sees as half its bytes and WRITE_SIZE as all
    _counters(tmp_path / "cf", [("copy", "FETCH_SIZE", 524288.0), ("fill", "FETCH_SIZE", 3.0)])
    _counters(tmp_path / "cw", [("copy", "WRITE_SIZE", 1048576.0)])
    out = tmp_path / "t.json"
    profile_summary.main(["traffic", str(tmp_path / "f"), str(tmp_path / "w"), str(tmp_path / "cf"),
                          str(tmp_path / "cw"), "k_step", "hs_decode_step", "wl", str(out),
                          "--command", "cmd"])
    rec = json.load(open(out))
    assert rec["fetch_kib_per_dispatch"] == 2000.0 and rec["write_kib_per_dispatch"] == 20.0
    assert rec["calibration"]["fetch_factor"] == 2.0 and rec["calibration"]["write_factor"] == 1.0
    assert rec["hbm_bytes_per_launch"] == 2000.0 * 1024 * 2 + 20.0 * 1024
    assert rec["source_sha256"] == bench.source_digest(bench.KERNEL_SOURCES["hs_decode_step"])


def _stats(d, rows):
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "run_kernel_stats.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Name", "Calls", "TotalDurationNs", "AverageNs",
                                          "MinNs", "MaxNs"])
        w.writeheader()
        for name, calls, avg in rows:
            w.writerow({"Name": name, "Calls": calls, "TotalDurationNs": calls * avg,
                        "AverageNs": avg, "MinNs": avg, "MaxNs": avg})


def test_stats_summary_of_a_figure_run(tmp_path):
    """bench.py --mode shared prints one figure instead of the benchmark line;
    the stats summary lists the library's kernels, slowest in total first, and
    the figure's fields."""
    from hierarchical_sparse_attention_amd import profile_summary
    dec = "void hs::(anonymous namespace)::k_decode<hs::bf16_t, 128, 4, false>(hs::DecodeParams)"
    step = "void hs::(anonymous namespace)::k_step<hs::bf16_t, 128, 0, 4>(hs::StepParams, int)"
    _stats(tmp_path / "tr", [(step, 10, 120000.0), (dec, 70, 97000.0), ("copyBuffer", 5, 1.0)])
    fig = {"mode": "shared", "figure": "shared_selection", "reps": 4,
           "config": {"workload": "wl"},
           "shared_selection": {"layers": 8, "shared": {"ms_per_token": 0.78}}}
    bj = tmp_path / "b.json"
    bj.write_text(json.dumps(fig))
    out = tmp_path / "k.md"
    profile_summary.main(["stats", str(tmp_path / "tr"), str(bj), str(out), "--command", "cmd"])
    text = out.read_text()
    assert text.startswith("# Kernel durations: wl")
    rows = [l for l in text.splitlines() if l.startswith("| `")]
    assert [r.split("`")[1] for r in rows] == ["k_decode<hs::bf16_t, 128, 4, false>",
                                               "k_step<hs::bf16_t, 128, 0, 4>"]
    assert "| 70 | 97.00 |" in rows[0]
    assert '- shared: {"ms_per_token": 0.78}' in text and "- layers: 8" in text
